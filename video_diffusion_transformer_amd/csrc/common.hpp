// Device-side helpers shared by the HIP kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wan {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16). Within each group of 16
// lanes, lane i receives element i%4 of the four 16-bit values that lane
// 4*j + i/4 of the group addressed, as its element j.
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
__device__ __forceinline__ s16x4_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

// Fold of two partial attentions over disjoint key sets (natural-log LSEs la of
// the accumulator, lc of the chunk): L = log(e^la + e^lc), and the accumulator
// becomes wa * acc + wc * chunk with wa = e^(la - L), wc = e^(lc - L). An LSE of
// -inf is an empty side (weight 0; an empty accumulator is not read). Shared by
// the merge kernel and the merging epilogue of the chunk attention, so the two
// give the same bits.
struct LseFold {
  float L, wa, wc;
  bool acc_empty;
};
__device__ __forceinline__ LseFold lse_fold(float la, float lc) {
  const float mx = fmaxf(la, lc);
  LseFold f;
  f.L = mx == -INFINITY ? -INFINITY : mx + log1pf(expf(-fabsf(la - lc)));
  f.acc_empty = la == -INFINITY;
  f.wa = f.acc_empty ? 0.f : expf(la - f.L);
  f.wc = lc == -INFINITY ? 0.f : expf(lc - f.L);
  return f;
}
__device__ __forceinline__ float lse_fold_value(const LseFold& f, float a, float c) {
  return fmaf(f.wa, f.acc_empty ? 0.f : a, f.wc * c);
}

// Per-tensor e4m3 scale from an amax: 448 / amax (IEEE fp32 division), or 1
// for an all-zero tensor.
__device__ __forceinline__ float fp8_scale_of(float amax) { return amax > 0.f ? 448.0f / amax : 1.0f; }

// Eight bf16 values (one 16-byte chunk) -> eight OCP e4m3 bytes of x * s:
// fp32 product, clamped to +-448 (saturation), round to nearest even.
__device__ __forceinline__ u32x2_t quant8_e4m3(const u32x4_t v, float s) {
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float x0 = fminf(fmaxf(bf16_lo(v[2 * h]) * s, -448.f), 448.f);
    const float x1 = fminf(fmaxf(bf16_hi(v[2 * h]) * s, -448.f), 448.f);
    const float x2 = fminf(fmaxf(bf16_lo(v[2 * h + 1]) * s, -448.f), 448.f);
    const float x3 = fminf(fmaxf(bf16_hi(v[2 * h + 1]) * s, -448.f), 448.f);
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, p, true);
    w[h] = static_cast<uint32_t>(p);
  }
  return u32x2_t{w[0], w[1]};
}

// max |x| over eight bf16 values, folded into m.
__device__ __forceinline__ float absmax8(float m, const u32x4_t v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(bf16_lo(v[j])), fabsf(bf16_hi(v[j]))));
  return m;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Block-wide max of non-negative per-thread values folded into *target with one
// atomic maximum on the float bits (non-negative floats order like their bits);
// skipped when the running value is already larger. red: LDS of >= waves floats.
__device__ __forceinline__ void block_atomic_max(float v, float* target, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6, nwaves = (blockDim.x + 63) >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = 0.f;
    for (int w = 0; w < nwaves; ++w) m = fmaxf(m, red[w]);
    unsigned* p = reinterpret_cast<unsigned*>(target);
    const unsigned bits = __float_as_uint(m);
    if (bits > __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(p, bits);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace wan
