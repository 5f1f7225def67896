// Bidirectional multi-head attention with fp8 (OCP e4m3) operands and fp32
// accumulation on the gfx950 v_mfma_scale_f32_16x16x128_f8f6f4 (unit block
// scales), the fp8 configuration of the Wan2.2 720p step. The TensorRT-LLM pull
// request "Optimize Wan2.2 Dataflow" runs this attention in FP8 through a cuDNN
// flash SDPA kernel (Isolated Operator Results); this kernel is written from the
// definition, not from that one.
//
// Inputs come from the quantisation pass: Q and K in a packed [B, S, 2D] e4m3
// buffer, V transposed per head [B, heads, 128, S_pad] e4m3, and the three
// per-tensor scales (x8 = x * scale). Scores are q8 . k8 / (scale_q scale_k)
// * softmax_scale; the softmax is fp32 (base 2, scale folded in); P is
// quantised to e4m3 at a fixed scale of 2^8 (folded into the exponent:
// p8 = e4m3(exp2(s - m + 8))) and the output is (sum p8 v8) / (scale_v * l8),
// with l8 = sum p8 accumulated by the MFMA itself: one extra 16x16x128 MFMA per
// query tile multiplies P by a constant operand whose first row is all ones,
// which costs 1/16 more MFMA work and removes a VALU add per score (the
// softmax, not the MFMA, bounds this kernel), and normalises by exactly the
// quantised weights used in PV.
//
// Work decomposition (same skeleton as the bf16 kernel):
//   * workgroup = 8 waves = 256 queries of one (b, h), one workgroup per CU;
//     each wave owns 32 queries (two 16-column MFMA tiles);
//   * keys stream in units of 128 (one K = 128 MFMA step for PV) through two LDS
//     stages, filled straight from global memory by global_load_lds_dwordx4 (no
//     staging registers): the next unit is requested at the top of the
//     iteration that consumes the current one, and one wait + barrier per unit
//     publishes it;
//   * S^T = K Q^T: one 16x16x128 MFMA covers all 128 channels of a 16-key tile.
//     The K rows are fed in a permuted order -- tile t, A-row m takes key
//     32*(m/4) + 4t + m%4 -- so that after the 8 tiles lane group g holds the
//     scores of keys 32g .. 32g+31 in order, which is exactly the k layout of the
//     B operand of O^T = V^T P^T: the quantised probabilities need no shuffle;
//   * K and V^T tiles are 128 x 128 bytes in LDS with an XOR swizzle of the
//     16-byte chunk (below) so every group of 8 and of 16 lanes reads distinct
//     bank slots;
//   * the running max moves only when a unit's max exceeds it by more than 0.75
//     (log2 units): p <= 2^0.75, so p * 2^8 <= 431 stays inside e4m3.
#include "common.hpp"
#include "kernels.hpp"

namespace wan {

namespace {

constexpr int kD = 128;
constexpr int kBN = 128;                 // keys per unit
#ifndef WAN_FP8_WAVES
#define WAN_FP8_WAVES 8
#endif
constexpr int kWaves = WAN_FP8_WAVES;
constexpr int kThreads = 64 * kWaves;
static_assert(16 % kWaves == 0, "the 16 blocks of a K or V^T tile must split evenly over the waves");
constexpr int kBM = 32 * kWaves;
constexpr int kTile = 128 * 128;         // bytes of one K or V^T tile
constexpr int kStage = 2 * kTile;
constexpr float kPLog2Scale = 8.0f;      // P is quantised as e4m3(p * 2^8)
constexpr float kRescaleSlack = 0.75f;   // keeps p * 2^8 <= 2^8.75 < 448
constexpr int kE4m3One = 0x38383838;     // four e4m3 1.0 bytes

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid & 7, j = bid >> 3;
  const int q = nb >> 3, r = nb & 7;
  return xcd * q + (xcd < r ? xcd : r) + j;
}

// Chunk swizzles: logical 16-byte chunk ch of row r sits at physical chunk
// ch ^ xor(r). Rows are 128 bytes. Measured with the LDS bank-conflict counter
// on single-pattern probes, a 16-byte-per-lane read on gfx950 is conflict-free
// when each half-wave (32 lanes) covers 32 distinct 16-byte slots of a 512-byte
// window (slot = 8 (row % 4) + physical chunk); the swizzles below also keep
// every 8 and 16 consecutive lanes on distinct slots of 128 and 256 bytes.
// K: lane (l16, g) reads row 32a + 4t + b (a = l16/4, b = l16%4) at logical
// chunk 2g (+1): xor = a0 | b1 << 1 | (a1 ^ b0) << 2. V^T: lane (l16, g) reads
// row 16dt + i (i = l16) at chunk 2g (+1): xor = i2 | i1 << 1 | (i0 ^ i3) << 2.
// (Rows shifted by ((r >> 5) & 3) | ((r >> 1) & 1) << 2 and (r >> 1) & 7 instead
// spent 19% of the kernel's cycles in bank conflicts.)
__device__ __forceinline__ int k_xor(int r) {
  return ((r >> 5) & 1) | (((r >> 1) & 1) << 1) | ((((r >> 6) ^ r) & 1) << 2);
}
__device__ __forceinline__ int v_xor(int r) {
  return ((r >> 2) & 1) | (((r >> 1) & 1) << 1) | ((((r >> 3) ^ r) & 1) << 2);
}
__device__ __forceinline__ int k_swz(int r, int ch) { return r * 128 + 16 * (ch ^ k_xor(r)); }
__device__ __forceinline__ int v_swz(int r, int ch) { return r * 128 + 16 * (ch ^ v_xor(r)); }

// s_waitcnt with vmcnt = 0 and the other counters at their maximum (no wait).
constexpr int kWaitVmem0 = 0x0f70;

__device__ __forceinline__ f32x4_t mfma_fp8(const i32x8_t& a, const i32x8_t& b, const f32x4_t& c) {
  // e4m3 x e4m3 (format code 0 for both), block scales 2^(127-127) = 1.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ExactSum (the instance that returns the LSE): each lane also adds up its fp32
// probabilities before the e4m3 rounding, so the log-sum-exp is that of the
// scores up to fp32 rounding, not of the quantised weights.
template <bool ExactSum>
__global__ void __launch_bounds__(kThreads, kWaves > 4 ? 1 : 2)
attn_fwd_fp8_kernel(const uint8_t* __restrict__ qk8, const uint8_t* __restrict__ vt8,
                    const float* __restrict__ scales, uint16_t* __restrict__ out, float* __restrict__ lse, int S,
                    int S_pad, int heads, int nqt, float softmax_scale) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStage];

  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = lid % nqt;
  const int bh = lid / nqt;
  const int h = bh % heads, b = bh / heads;
  const int D = heads * kD;
  const int rs = 2 * D;  // bytes per token row of qk8
  const uint8_t* qkb = qk8 + (int64_t)b * S * rs + h * kD;
  const uint8_t* vtb = vt8 + (int64_t)bh * kD * S_pad;

  const float dq = 1.0f / scales[0], dk = 1.0f / scales[1], dv = 1.0f / scales[2];
  const float c_log2 = dq * dk * softmax_scale * 1.4426950408889634f;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, grp = lane >> 4;

  // Q fragments: query 16u + l16, channels 32*grp .. +31 (32 bytes).
  const int q0 = qt * kBM + wave * 32;
  i32x8_t qf[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    int q = q0 + 16 * u + l16;
    q = q < S ? q : S - 1;
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(qkb + (int64_t)q * rs + 32 * grp);
    const u32x4_t x0 = qp[0], x1 = qp[1];
    qf[u] = i32x8_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  }

  f32x4_t acc_o[8][2], acc_l[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc_o[i][0] = acc_o[i][1] = f32x4_t{};
  acc_l[0] = acc_l[1] = f32x4_t{};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l32[2] = {0.f, 0.f};  // ExactSum: this lane's fp32 sum of 2^8 p
  // A operand whose row 0 is all ones (rows 1..15 zero): row 0 of ones x P^T is
  // the column sum of P, i.e. l for each query, in lane (grp 0, l16), register 0.
  const int one = l16 == 0 ? kE4m3One : 0;
  const i32x8_t ones = {one, one, one, one, one, one, one, one};

  // Direct global -> LDS staging (global_load_lds_dwordx4: lane l of a wave
  // instruction lands at the wave-uniform LDS base + 16*l). Each wave fills four
  // 1 KB blocks (8 rows) of the K tile and of the V^T tile; lane l of a block
  // takes physical row 8*blk + l/8, physical chunk l%8, so it fetches the
  // logical chunk that the swizzle maps there.
  auto issue_unit = [&](int k0, int stage) {
    unsigned char* ks = smem + stage * kStage;
#pragma unroll
    for (int j = 0; j < 16 / kWaves; ++j) {
      const int blk = (16 / kWaves) * wave + j;
      const int r = 8 * blk + (lane >> 3), pc = lane & 7;
      const int key = min(k0 + r, S - 1);
      __builtin_amdgcn_global_load_lds(qkb + (int64_t)key * rs + D + 16 * (pc ^ k_xor(r)), ks + blk * 1024, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vtb + (int64_t)r * S_pad + k0 + 16 * (pc ^ v_xor(r)), ks + kTile + blk * 1024,
                                       16, 0, 0);
    }
  };

  const int nu = (S + kBN - 1) / kBN;
  // P of the current unit in e4m3. Each word is written as two halves by two
  // conversions; the first keeps the other half of the word it is given, so
  // it is given the word it replaces (kept across units: no zeroing moves).
  i32x8_t pf[2] = {};
  issue_unit(0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  __syncthreads();

  for (int un = 0; un < nu; ++un) {
    const int k0 = un * kBN;
    const unsigned char* ks = smem + (un & 1) * kStage;
    const unsigned char* vs = ks + kTile;
    // The other stage was last read in iteration un-1, which every wave has left.
    if (un + 1 < nu) issue_unit(k0 + kBN, (un + 1) & 1);

    // S^T for 8 key tiles; tile t, A-row l16 holds key 32*(l16/4) + 4t + l16%4.
    f32x4_t acc_s[8][2];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int r = 32 * (l16 >> 2) + 4 * t + (l16 & 3);
      const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(ks + k_swz(r, 2 * grp));
      const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(ks + k_swz(r, 2 * grp + 1));
      const i32x8_t a = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      acc_s[t][0] = mfma_fp8(a, qf[0], f32x4_t{});
      acc_s[t][1] = mfma_fp8(a, qf[1], f32x4_t{});
    }
    // Fragment reads issued two tiles ahead of their MFMAs (R0 R1 | M0 R2 | M1
    // R3 | ... | M7): grouped two reads then two MFMAs by the compiler, each
    // wait for a tile's reads also waited for the next tile's (+2%).
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      if (t + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }

    if (k0 + kBN > S) {  // keys past the end (last unit only): lane group grp holds keys 32grp + 4t + i
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k0 + 32 * grp + 4 * t + i >= S) acc_s[t][0][i] = acc_s[t][1][i] = -INFINITY;
    }

#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // Two chains of three-input maxima (v_max3_f32): 17 instructions for the
      // 32 scores; the empty asm keeps the compiler from re-balancing them into
      // a tree of two-input maxima (23 instructions).
      float m1 = fmaxf(acc_s[0][u][0], acc_s[0][u][1]), m2 = fmaxf(acc_s[0][u][2], acc_s[0][u][3]);
#pragma unroll
      for (int t = 1; t < 8; ++t) {
        m1 = fmaxf(m1, fmaxf(acc_s[t][u][0], acc_s[t][u][1]));
        m2 = fmaxf(m2, fmaxf(acc_s[t][u][2], acc_s[t][u][3]));
        asm("" : "+v"(m1), "+v"(m2));
      }
      float mx = fmaxf(m1, m2);
      // Lanes l, l^16, l^32, l^48 share the query and its m_run: testing each
      // lane's own max is the same as testing the column max, so the
      // cross-lane reduction runs only when the max moves.
      mx *= c_log2;
      if (__ballot(mx > m_run[u] + kRescaleSlack)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run[u], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[u] - m_new);
        m_run[u] = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_l[u][i] *= alpha;
        if constexpr (ExactSum) l32[u] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc_o[dt][u][i] *= alpha;
      }
      const float m_shift = m_run[u] - kPLog2Scale;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(acc_s[t][u][i], c_log2, -m_shift));
        if constexpr (ExactSum) l32[u] += (p[0] + p[1]) + (p[2] + p[3]);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pf[u][t], false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
        pf[u][t] = w;
      }
      acc_l[u] = mfma_fp8(ones, pf[u], acc_l[u]);
    }

    // O^T += V^T P^T: 8 channel tiles, K = the 128 keys of the unit.
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int r = 16 * dt + l16;
      const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(vs + v_swz(r, 2 * grp));
      const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(vs + v_swz(r, 2 * grp + 1));
      const i32x8_t a = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      acc_o[dt][0] = mfma_fp8(a, pf[0], acc_o[dt][0]);
      acc_o[dt][1] = mfma_fp8(a, pf[1], acc_o[dt][1]);
    }
    // The same two-ahead order for the V^T fragments.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 2);
      if (dt + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
    }

    __builtin_amdgcn_s_waitcnt(kWaitVmem0);  // this wave's part of the next unit has landed
    __syncthreads();                          // ... and every other wave's; this stage is free
  }

#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float l_tot = __shfl(acc_l[u][0], l16, 64);  // l8 of query l16 lives in lane l16
    const int q = q0 + 16 * u + l16;
    if (q < S) {
      const float inv = dv / l_tot;
      uint16_t* op = out + ((int64_t)b * S + q) * D + h * kD + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint2 w;
        w.x = pack_bf16x2(acc_o[dt][u][0] * inv, acc_o[dt][u][1] * inv);
        w.y = pack_bf16x2(acc_o[dt][u][2] * inv, acc_o[dt][u][3] * inv);
        *reinterpret_cast<uint2*>(op + 16 * dt) = w;
      }
      if constexpr (ExactSum) {
        // the four lanes of a query hold disjoint keys; their fp32 sum is
        // 2^8 * sum p, so ln(sum exp(s)) = (m + log2(l) - 8) * ln 2
        float l = l32[u];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        if (grp == 0) lse[(int64_t)bh * S + q] = (m_run[u] + __log2f(l) - kPLog2Scale) * 0.69314718055994531f;
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const void* qk8, const void* vt8, const float* scales, void* out, float* lse, int B,
                               int S, int heads, float softmax_scale, hipStream_t stream) {
  const int nqt = (S + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)nqt * heads * B;
  if (nblocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const int S_pad = (S + 127) / 128 * 128;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, stream,
                       static_cast<const uint8_t*>(qk8), static_cast<const uint8_t*>(vt8), scales,
                       static_cast<uint16_t*>(out), lse, S, S_pad, heads, nqt, softmax_scale);
  };
  if (lse)
    go(attn_fwd_fp8_kernel<true>);
  else
    go(attn_fwd_fp8_kernel<false>);
  return hipGetLastError();
}

}  // namespace wan
