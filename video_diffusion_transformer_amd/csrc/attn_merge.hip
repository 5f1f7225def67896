// Merge of two partial attentions over disjoint key sets -- the per-round
// combine of ring attention ("Optimizing High-Quality Offline Video
// Generation", Context parallelism: each rank's queries attend K/V chunks that
// rotate around the ring, and the partial results are combined).
//
// For each (b, s, head): L = log(exp(la) + exp(lc)); acc = exp(la - L) acc +
// exp(lc - L) chunk; la = L. One wavefront owns one (b, s, head) row of 128
// channels (two per lane), so the log-sum-exp it reads and rewrites is never
// touched by another wave. HBM-bound: 12 bytes per channel (+2 with the bf16
// copy).
#include "common.hpp"
#include "kernels.hpp"

namespace wan {

namespace {

__global__ void __launch_bounds__(256)
attn_merge_kernel(float* __restrict__ acc, float* __restrict__ acc_lse, const float* __restrict__ co,
                  const float* __restrict__ clse, uint16_t* __restrict__ out16, int Sq, int heads, int64_t groups) {
  const int64_t g = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);  // (b, s, head) row
  if (g >= groups) return;
  const int lane = threadIdx.x & 63;
  const int h = static_cast<int>(g % heads);
  const int64_t row = g / heads;  // b * Sq + s
  const int64_t b = row / Sq, s = row % Sq;
  const int64_t li = (b * heads + h) * Sq + s;
  const LseFold fo = lse_fold(acc_lse[li], clse[li]);
  const int64_t off = row * (int64_t)heads * 128 + h * 128 + 2 * lane;
  // An empty accumulator row is not read: whatever it holds (e.g. a fresh
  // allocation) must not leak into the result through 0 * NaN.
  const float2 a = fo.acc_empty ? make_float2(0.f, 0.f) : *reinterpret_cast<const float2*>(acc + off);
  const float2 c = *reinterpret_cast<const float2*>(co + off);
  const float2 r = make_float2(lse_fold_value(fo, a.x, c.x), lse_fold_value(fo, a.y, c.y));
  *reinterpret_cast<float2*>(acc + off) = r;
  if (out16) *reinterpret_cast<uint32_t*>(out16 + off) = pack_bf16x2(r.x, r.y);
  if (lane == 0) acc_lse[li] = fo.L;
}

}  // namespace

hipError_t launch_attn_merge(float* acc, float* acc_lse, const float* chunk, const float* chunk_lse, void* out16,
                             int B, int Sq, int heads, hipStream_t stream) {
  const int64_t groups = (int64_t)B * Sq * heads;
  const int64_t blocks = (groups + 3) / 4;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, acc, acc_lse, chunk,
                     chunk_lse, static_cast<uint16_t*>(out16), Sq, heads, groups);
  return hipGetLastError();
}

}  // namespace wan
