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
// LDS. V is never written. The token's 64 rotary (cos, sin) pairs are gathered
// from the three per-axis tables once per workgroup, by one wave, into LDS:
// read per thread and per chunk from the tables instead, they cost 4% of the
// kernel's bandwidth (eight 8-byte loads per thread against four 16-byte Q/K loads).
//
// The fp8 variant (Amax) also takes, in the same pass, max |x| of the rounded Q
// and K it writes and of V (read once for it), and folds them into amax[0..2]:
// the amax step of the amax -> E4M3 scale -> quantise recipe ("Optimize Wan2.2
// Dataflow", change 2) moved into the norm epilogue, so the quantisation pass
// that follows needs no separate amax pass over Q, K and V.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

// Tuning defaults (the kernel below reads them, so they come first).
#ifndef WAN_NORM_MIN_CPT
#define WAN_NORM_MIN_CPT 2  // two 16-byte chunks of Q and of K per thread: more bytes in flight per CU
#endif
#ifndef WAN_NORM_NT
#define WAN_NORM_NT 3  // non-temporal loads (1) and stores (2): the rows are touched once
#endif

namespace wan {

namespace {

constexpr int kPairsT = 22, kPairsH = 21, kPairsW = 21;  // 44/42/42 channels per axis

// What the kernel does with the rotated bf16 Q and K: store them in place;
// store them in place and fold max |x| of Q, K and V into amax; or quantise
// them to e4m3 at the scales of an earlier amax (qk8, not in place) and fold
// max |x| of Q and K into amax.
enum NormMode { kNormInPlace = 0, kNormAmax = 1, kNormFp8Delayed = 2 };

template <int CPT, int Mode>
__global__ void __launch_bounds__(1024)
qknorm_rope_kernel(uint16_t* __restrict__ qkv, const uint16_t* __restrict__ gq,
                   const uint16_t* __restrict__ gk, const float2* __restrict__ tab, int64_t row0,
                   int S, int H, int W, int D, int offH, int offW, float inv_d, float eps, float* __restrict__ amax,
                   uint8_t* __restrict__ qk8, const float* __restrict__ amax_prev) {
  constexpr bool Amax = Mode != kNormInPlace;
  const int64_t row = row0 + blockIdx.x;
  const int s = static_cast<int>(row % S);
  const int f = s / (H * W), y = (s / W) % H, x = s % W;
  const int nchunks = D >> 3;
  uint16_t* qrow = qkv + row * (3 * (int64_t)D);
  uint16_t* krow = qrow + D;

  // The token's 64 rotary (cos, sin) pairs (22 frame, 21 row, 21 column), gathered once by the
  // first wave into LDS; published by the barrier of the reduction below.
  __shared__ __attribute__((aligned(16))) float2 rot[64];
  if (threadIdx.x < 64) {
    const int p = threadIdx.x;
    rot[p] = p < kPairsT ? tab[f * kPairsT + p]
                         : (p < kPairsT + kPairsH ? tab[offH + y * kPairsH + (p - kPairsT)]
                                                  : tab[offW + x * kPairsW + (p - kPairsT - kPairsH)]);
  }
  u32x4_t qv[CPT], kv[CPT];
  float sq = 0.f, sk = 0.f, mq = 0.f, mk = 0.f, mv = 0.f;
  float sq8 = 1.f, sk8 = 1.f;  // kNormFp8Delayed: e4m3 scales of Q and K from the earlier amax
  if constexpr (Mode == kNormFp8Delayed) {
    sq8 = fp8_scale_of(amax_prev[0]);
    sk8 = fp8_scale_of(amax_prev[1]);
  }
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
      if constexpr (Mode == kNormAmax)
        mv = absmax8(mv, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(krow + D + 8 * c)));
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

  // Chunk c holds pairs 4 (c % 16) .. +3 of its head; c = threadIdx.x + i * blockDim.x with
  // blockDim a multiple of 64, so all chunks of this thread use the same four pairs.
  float2 cs4[4];
  {
    const float4* r = reinterpret_cast<const float4*>(rot) + 2 * (threadIdx.x & 15);
    const float4 a0 = r[0], a1 = r[1];
    cs4[0] = make_float2(a0.x, a0.y);
    cs4[1] = make_float2(a0.z, a0.w);
    cs4[2] = make_float2(a1.x, a1.y);
    cs4[3] = make_float2(a1.z, a1.w);
  }

#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * blockDim.x;
    if (c < nchunks) {
      const u32x4_t g1 = *reinterpret_cast<const u32x4_t*>(gq + 8 * c);
      const u32x4_t g2 = *reinterpret_cast<const u32x4_t*>(gk + 8 * c);
      u32x4_t qo, ko;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float2 cs = cs4[j];
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
      if constexpr (Amax) {
        mq = absmax8(mq, qo);
        mk = absmax8(mk, ko);
      }
      if constexpr (Mode == kNormFp8Delayed) {
        uint8_t* orow = qk8 + row * (2 * (int64_t)D);
        __builtin_nontemporal_store(quant8_e4m3(qo, sq8), reinterpret_cast<u32x2_t*>(orow + 8 * c));
        __builtin_nontemporal_store(quant8_e4m3(ko, sk8), reinterpret_cast<u32x2_t*>(orow + D + 8 * c));
      } else {
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
  if constexpr (Amax) {
    // Block maxima, then one atomic maximum per tensor (non-negative floats
    // order like their bits). Most blocks find the running value already
    // larger and skip the atomic.
    __shared__ float pmax[32][3];
    mq = wave_max(mq);
    mk = wave_max(mk);
    mv = wave_max(mv);
    if ((threadIdx.x & 63) == 0) {
      pmax[wave][0] = mq;
      pmax[wave][1] = mk;
      pmax[wave][2] = mv;
    }
    __syncthreads();
    constexpr int kTensors = Mode == kNormAmax ? 3 : 2;  // the delayed mode leaves V to the V pass
    if (threadIdx.x < kTensors) {
      float m = 0.f;
      for (int w = 0; w < nwaves; ++w) m = fmaxf(m, pmax[w][threadIdx.x]);
      unsigned* p = reinterpret_cast<unsigned*>(amax) + threadIdx.x;
      const unsigned bits = __float_as_uint(m);
      if (bits > __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(p, bits);
    }
  }
}

// The fp32 (cos, sin) tables of the three rotary axes: entry (pos, j) of an
// axis with np pairs holds cos / sin of pos * theta^(-2j / (2 np)), computed in
// double and rounded once to fp32. Layout: frame axis [T][22], row axis
// [H][21], column axis [W][21], one after the other.
__global__ void __launch_bounds__(256) rope_table_kernel(float2* __restrict__ tab, int T, int H, int W, double theta) {
  const int n = T * kPairsT + H * kPairsH + W * kPairsW;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  int pos, j, np;
  if (e < T * kPairsT) {
    pos = e / kPairsT, j = e % kPairsT, np = kPairsT;
  } else if (e < T * kPairsT + H * kPairsH) {
    const int r = e - T * kPairsT;
    pos = r / kPairsH, j = r % kPairsH, np = kPairsH;
  } else {
    const int r = e - T * kPairsT - H * kPairsH;
    pos = r / kPairsW, j = r % kPairsW, np = kPairsW;
  }
  const double omega = pow(theta, -2.0 * j / (2.0 * np));
  const double phi = static_cast<double>(pos) * omega;
  tab[e] = make_float2(static_cast<float>(cos(phi)), static_cast<float>(sin(phi)));
}

}  // namespace

int64_t rope_table_entries(int64_t T, int64_t H, int64_t W) { return T * kPairsT + H * kPairsH + W * kPairsW; }

hipError_t launch_rope_table(float2* tab, int T, int H, int W, float theta, hipStream_t stream) {
  const int64_t n = rope_table_entries(T, H, W);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, tab, T, H,
                     W, static_cast<double>(theta));
  return hipGetLastError();
}

hipError_t launch_qknorm_rope(void* qkv, const void* gq, const void* gk, const float2* tab,
                              int64_t row0, int64_t rows, int S, int T, int H, int W, int D,
                              float eps, float* amax, hipStream_t stream, uint8_t* qk8, const float* amax_prev) {
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
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, q, a, b, tab, row0, S, H, W, D, offH, offW, inv_d, eps,
                       amax, qk8, amax_prev);
  };
  auto pick = [&](auto mode) {
    constexpr int M = decltype(mode)::value;
    if (cpt == 1) go(qknorm_rope_kernel<1, M>);
    else if (cpt == 2) go(qknorm_rope_kernel<2, M>);
    else go(qknorm_rope_kernel<4, M>);
  };
  if (qk8) pick(std::integral_constant<int, kNormFp8Delayed>{});
  else if (amax) pick(std::integral_constant<int, kNormAmax>{});
  else pick(std::integral_constant<int, kNormInPlace>{});
  return hipGetLastError();
}

}  // namespace wan
