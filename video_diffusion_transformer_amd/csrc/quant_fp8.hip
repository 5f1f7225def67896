// Per-tensor fp8 (OCP e4m3) quantisation of Q, K and V for the fp8 attention
// path: amax of each tensor over all (B, S, D), scale = 448 / amax (fp32, IEEE
// division; an all-zero tensor keeps scale 1), e4m3 = round-to-nearest-even of
// fl32(x * scale), saturated to +-448. This is the amax -> E4M3 scale -> quantise
// recipe the TensorRT-LLM pull request "Optimize Wan2.2 Dataflow" fuses for its
// FFN activation (change 2), applied here to the attention inputs.
//
// Layout of the outputs (our own, consumed only by the fp8 attention kernel):
//   qk8 : [B, S, 2D] bytes -- per token Q (all heads) then K (all heads);
//   vt8 : [B, heads, 128, S_pad] bytes -- V transposed per head (channel-major,
//         keys contiguous), S_pad = S rounded up to 128, zero past S. Writing V
//         transposed costs no extra traffic (V is written once either way) and
//         lets the attention kernel read the PV operand with plain 16-byte LDS
//         loads.
#include "common.hpp"
#include "kernels.hpp"

namespace wan {

namespace {

#ifndef WAN_QUANT_NT
#define WAN_QUANT_NT 3  // non-temporal loads (1) and stores (2) in the quantise pass (+2%)
#endif
#ifndef WAN_QUANT_TOK
#define WAN_QUANT_TOK 128
#endif
constexpr int kTok = WAN_QUANT_TOK;  // tokens per quantisation tile: 128 keys fill whole 128-byte lines of V^T

__global__ void amax_clear_kernel(float* amax) {
  if (threadIdx.x < 3) amax[threadIdx.x] = 0.f;
}

// Grid-stride over token rows; each block folds |x| of Q, K and V separately and
// publishes three atomic maxima (non-negative floats order like their bits).
__global__ void __launch_bounds__(256) amax_kernel(const uint16_t* __restrict__ qkv, float* amax, int64_t rows,
                                                   int D) {
  const int chunks = 3 * D / 8, per = D / 8;
  float m[3] = {0.f, 0.f, 0.f};
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint16_t* row = qkv + r * 3 * (int64_t)D;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + 8 * c);
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) a = fmaxf(a, fmaxf(fabsf(bf16_lo(v[j])), fabsf(bf16_hi(v[j]))));
      const int part = c / per;
      m[0] = part == 0 ? fmaxf(m[0], a) : m[0];
      m[1] = part == 1 ? fmaxf(m[1], a) : m[1];
      m[2] = part == 2 ? fmaxf(m[2], a) : m[2];
    }
  }
  __shared__ float red[4][3];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    float x = m[p];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    if (lane == 0) red[wave][p] = x;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    float x = red[0][threadIdx.x];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) x = fmaxf(x, red[w][threadIdx.x]);
    atomicMax(reinterpret_cast<unsigned int*>(amax) + threadIdx.x, __float_as_uint(x));
  }
}

// One block = kTok tokens of one (b, head): Q and K rows are quantised in place
// of their packed position; V goes through LDS to be stored channel-major.
// VOnly (the delayed-scale producer, whose norm pass already wrote the e4m3 Q
// and K): only V is read and quantised, with the scale of amax[2] (the amax an
// earlier call reported), and its max |v| is folded into amax_out[2].
template <bool VOnly>
__global__ void __launch_bounds__(256)
quant_kernel(const uint16_t* __restrict__ qkv, uint8_t* __restrict__ qk8, uint8_t* __restrict__ vt8,
             const float* __restrict__ amax, float* __restrict__ scales, float* __restrict__ amax_out, int S,
             int S_pad, int heads) {
  __shared__ uint8_t vt[128][kTok + 16];
  const int h = blockIdx.y, b = blockIdx.z, s0 = blockIdx.x * kTok;
  const int D = heads * 128;
  const float sq = fp8_scale_of(amax[0]), sk = fp8_scale_of(amax[1]), sv = fp8_scale_of(amax[2]);
  if (s0 == 0 && h == 0 && b == 0 && threadIdx.x == 0) {
    scales[0] = sq;
    scales[1] = sk;
    scales[2] = sv;
  }
  float mv = 0.f;
  // kTok tokens x 16 chunks of 8 channels, kTok / 16 per thread.
#pragma unroll
  for (int i = 0; i < kTok / 16; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int t = c >> 4, ch = c & 15;
    const int s = s0 + t;
    u32x2_t vq = {0u, 0u};
    if (s < S) {
      const uint16_t* row = qkv + ((int64_t)b * S + s) * 3 * (int64_t)D + h * 128 + 8 * ch;
      u32x4_t xq, xk;
#if WAN_QUANT_NT & 1
      if constexpr (!VOnly) {
        xq = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row));
        xk = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + D));
      }
      const u32x4_t xv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + 2 * D));
#else
      if constexpr (!VOnly) {
        xq = *reinterpret_cast<const u32x4_t*>(row);
        xk = *reinterpret_cast<const u32x4_t*>(row + D);
      }
      const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(row + 2 * D);
#endif
      if constexpr (!VOnly) {
        uint8_t* orow = qk8 + ((int64_t)b * S + s) * 2 * (int64_t)D + h * 128 + 8 * ch;
#if WAN_QUANT_NT & 2
        __builtin_nontemporal_store(quant8_e4m3(xq, sq), reinterpret_cast<u32x2_t*>(orow));
        __builtin_nontemporal_store(quant8_e4m3(xk, sk), reinterpret_cast<u32x2_t*>(orow + D));
#else
        *reinterpret_cast<u32x2_t*>(orow) = quant8_e4m3(xq, sq);
        *reinterpret_cast<u32x2_t*>(orow + D) = quant8_e4m3(xk, sk);
#endif
      }
      if constexpr (VOnly) mv = absmax8(mv, xv);
      vq = quant8_e4m3(xv, sv);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vt[8 * ch + j][t] = static_cast<uint8_t>(vq.x >> (8 * j));
      vt[8 * ch + 4 + j][t] = static_cast<uint8_t>(vq.y >> (8 * j));
    }
  }
  __syncthreads();
  // 128 channel rows x kTok keys = 128 x (kTok / 16) chunks of 16 B.
  uint8_t* vbase = vt8 + (((int64_t)b * heads + h) * 128) * S_pad + s0;
  constexpr int kParts = kTok / 16;
#pragma unroll
  for (int i = 0; i < kParts / 2; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int d = c / kParts, part = c % kParts;
#if WAN_QUANT_NT & 2
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(&vt[d][16 * part]),
                                reinterpret_cast<u32x4_t*>(vbase + (int64_t)d * S_pad + 16 * part));
#else
    *reinterpret_cast<u32x4_t*>(vbase + (int64_t)d * S_pad + 16 * part) =
        *reinterpret_cast<const u32x4_t*>(&vt[d][16 * part]);
#endif
  }
  if constexpr (VOnly) {
    __shared__ float red[4];
    block_atomic_max(mv, amax_out + 2, red);
  }
}

}  // namespace

hipError_t launch_amax_clear(float* amax, hipStream_t stream) {
  hipLaunchKernelGGL(amax_clear_kernel, dim3(1), dim3(64), 0, stream, amax);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const void* qkv, void* qk8, void* vt8, float* scales, const float* amax, int B, int S,
                            int heads, hipStream_t stream) {
  const int S_pad = (S + 127) / 128 * 128;
  hipLaunchKernelGGL(quant_kernel<false>, dim3(S_pad / kTok, heads, B), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(qkv), static_cast<uint8_t*>(qk8), static_cast<uint8_t*>(vt8),
                     amax, scales, nullptr, S, S_pad, heads);
  return hipGetLastError();
}

hipError_t launch_quant_v_delayed(const void* qkv, void* vt8, const float* amax_prev, float* scales, float* amax,
                                  int B, int S, int heads, hipStream_t stream) {
  const int S_pad = (S + 127) / 128 * 128;
  hipLaunchKernelGGL(quant_kernel<true>, dim3(S_pad / kTok, heads, B), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(qkv), nullptr, static_cast<uint8_t*>(vt8), amax_prev, scales, amax,
                     S, S_pad, heads);
  return hipGetLastError();
}

hipError_t launch_qkv_quant_fp8(const void* qkv, void* qk8, void* vt8, float* scales, float* amax, int B, int S,
                                int heads, hipStream_t stream) {
  const int D = heads * 128;
  const int64_t rows = (int64_t)B * S;
  hipLaunchKernelGGL(amax_clear_kernel, dim3(1), dim3(64), 0, stream, amax);
  const int64_t nb = rows < 8192 ? rows : 8192;
  hipLaunchKernelGGL(amax_kernel, dim3(static_cast<unsigned>(nb)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(qkv), amax, rows, D);
  return launch_quant_fp8(qkv, qk8, vt8, scales, amax, B, S, heads, stream);
}

}  // namespace wan
