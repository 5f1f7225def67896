// In-place Q/K RMSNorm + bf16 rounding point + 3-D RoPE on the packed QKV
// buffer (TensorRT-LLM pull request "Optimize Wan2.2 Dataflow": change 1, the
// "Fused Q/K Norm and RoPE" numerics, and the review comments on the reduction
// width and the weight index).
//
// Design (gfx950): one workgroup per token row. Each thread owns 16-byte
// chunks (8 channels) of Q and the chunk of K at the same channel offset, so
// the channel's gamma index and its rotary angles are shared by the Q and K
// halves. Q and K stay in registers between the reduction and the store: every
// element is read once and written once (HBM-bound, ~2 FLOP/byte). The full-width
// mean square is a wavefront butterfly reduction followed by a cross-wave sum in
// LDS. V is never touched.
#include "common.hpp"
#include "kernels.hpp"

namespace wan {

namespace {

constexpr int kPairsT = 22, kPairsH = 21, kPairsW = 21;  // 44/42/42 channels per axis

template <int CPT>
__global__ void __launch_bounds__(1024)
qknorm_rope_kernel(uint16_t* __restrict__ qkv, const uint16_t* __restrict__ gq,
                   const uint16_t* __restrict__ gk, const float2* __restrict__ tab, int64_t row0,
                   int S, int H, int W, int D, int offH, int offW, float inv_d, float eps) {
  const int64_t row = row0 + blockIdx.x;
  const int s = static_cast<int>(row % S);
  const int f = s / (H * W), y = (s / W) % H, x = s % W;
  const int nchunks = D >> 3;
  uint16_t* qrow = qkv + row * (3 * (int64_t)D);
  uint16_t* krow = qrow + D;

  u32x4_t qv[CPT], kv[CPT];
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * blockDim.x;
    if (c < nchunks) {
#if WAN_NORM_NT & 1
      qv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(qrow + 8 * c));
      kv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(krow + 8 * c));
#else
      qv[i] = *reinterpret_cast<const u32x4_t*>(qrow + 8 * c);
      kv[i] = *reinterpret_cast<const u32x4_t*>(krow + 8 * c);
#endif
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float a = bf16_lo(qv[i][j]), b = bf16_hi(qv[i][j]);
        sq += a * a + b * b;
        a = bf16_lo(kv[i][j]);
        b = bf16_hi(kv[i][j]);
        sk += a * a + b * b;
      }
    }
  }
  sq = wave_sum(sq);
  sk = wave_sum(sk);
  __shared__ float part[32][2];
  const int wave = threadIdx.x >> 6, nwaves = (blockDim.x + 63) >> 6;
  if ((threadIdx.x & 63) == 0) {
    part[wave][0] = sq;
    part[wave][1] = sk;
  }
  __syncthreads();
  sq = 0.f;
  sk = 0.f;
  for (int w = 0; w < nwaves; ++w) {
    sq += part[w][0];
    sk += part[w][1];
  }
  const float rq = rsqrtf(sq * inv_d + eps);
  const float rk = rsqrtf(sk * inv_d + eps);

  const float2* tt = tab + f * kPairsT;
  const float2* th = tab + offH + y * kPairsH;
  const float2* tw = tab + offW + x * kPairsW;

#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * blockDim.x;
    if (c < nchunks) {
      const u32x4_t g1 = *reinterpret_cast<const u32x4_t*>(gq + 8 * c);
      const u32x4_t g2 = *reinterpret_cast<const u32x4_t*>(gk + 8 * c);
      const int p0 = (4 * c) & 63;  // first rotary pair of this chunk within its head
      u32x4_t qo, ko;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = p0 + j;
        const float2 cs = p < kPairsT ? tt[p] : (p < kPairsT + kPairsH ? th[p - kPairsT] : tw[p - kPairsT - kPairsH]);
        // norm, x gamma, bf16 rounding point
        const uint32_t nq = pack_bf16x2(bf16_lo(qv[i][j]) * rq * bf16_lo(g1[j]),
                                        bf16_hi(qv[i][j]) * rq * bf16_hi(g1[j]));
        const uint32_t nk = pack_bf16x2(bf16_lo(kv[i][j]) * rk * bf16_lo(g2[j]),
                                        bf16_hi(kv[i][j]) * rk * bf16_hi(g2[j]));
        // rotation in fp32, bf16 out
        float a = bf16_lo(nq), b = bf16_hi(nq);
        qo[j] = pack_bf16x2(a * cs.x - b * cs.y, a * cs.y + b * cs.x);
        a = bf16_lo(nk);
        b = bf16_hi(nk);
        ko[j] = pack_bf16x2(a * cs.x - b * cs.y, a * cs.y + b * cs.x);
      }
#if WAN_NORM_NT & 2
      __builtin_nontemporal_store(qo, reinterpret_cast<u32x4_t*>(qrow + 8 * c));
      __builtin_nontemporal_store(ko, reinterpret_cast<u32x4_t*>(krow + 8 * c));
#else
      *reinterpret_cast<u32x4_t*>(qrow + 8 * c) = qo;
      *reinterpret_cast<u32x4_t*>(krow + 8 * c) = ko;
#endif
    }
  }
}

}  // namespace

hipError_t launch_qknorm_rope(void* qkv, const void* gq, const void* gk, const float2* tab,
                              int64_t row0, int64_t rows, int S, int T, int H, int W, int D,
                              float eps, hipStream_t stream) {
#ifndef WAN_NORM_MIN_CPT
#define WAN_NORM_MIN_CPT 2  // two 16-byte chunks of Q and of K per thread: more bytes in flight per CU
#endif
#ifndef WAN_NORM_NT
#define WAN_NORM_NT 3  // non-temporal loads (1) and stores (2): the rows are touched once
#endif
  const int nchunks = D / 8;
  int cpt = nchunks <= 1024 ? 1 : (nchunks <= 2048 ? 2 : 4);
  cpt = cpt < WAN_NORM_MIN_CPT ? WAN_NORM_MIN_CPT : cpt;
  const int per = (nchunks + cpt - 1) / cpt;
  const int threads = ((per + 63) / 64) * 64;
  const int offH = T * kPairsT, offW = offH + H * kPairsH;
  const float inv_d = 1.0f / static_cast<float>(D);
  auto* q = static_cast<uint16_t*>(qkv);
  auto* a = static_cast<const uint16_t*>(gq);
  auto* b = static_cast<const uint16_t*>(gk);
  dim3 grid(static_cast<unsigned>(rows));
  if (cpt == 1)
    hipLaunchKernelGGL(qknorm_rope_kernel<1>, grid, dim3(threads), 0, stream, q, a, b, tab, row0, S, H, W, D, offH, offW, inv_d, eps);
  else if (cpt == 2)
    hipLaunchKernelGGL(qknorm_rope_kernel<2>, grid, dim3(threads), 0, stream, q, a, b, tab, row0, S, H, W, D, offH, offW, inv_d, eps);
  else
    hipLaunchKernelGGL(qknorm_rope_kernel<4>, grid, dim3(threads), 0, stream, q, a, b, tab, row0, S, H, W, D, offH, offW, inv_d, eps);
  return hipGetLastError();
}

}  // namespace wan
