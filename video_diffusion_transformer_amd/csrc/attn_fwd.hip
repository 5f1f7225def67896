// Bidirectional multi-head flash-attention forward on the packed [Q|K|V]
// buffer, bf16 MFMA with fp32 accumulation (gfx950 v_mfma_f32_16x16x32_bf16).
//
// What it computes: for every (batch, head) and every query row, softmax over
// ALL keys of (q . k) * scale, times V -- the unmasked attention of the Wan2.2
// DiT ("Optimizing High-Quality Offline Video Generation", Overview: the
// denoiser is bidirectional). The S x S score matrix never leaves registers.
//
// Work decomposition
//   * one workgroup = 8 wavefronts = 384 query rows of one (b, h), one
//     workgroup per CU (two waves per SIMD); each wave owns 48 rows (three
//     16-row MFMA column tiles) for the whole kernel, so every K/V fragment read
//     from LDS feeds three MFMAs (LDS bandwidth, not the MFMA rate, is the
//     tighter limit of this loop on gfx950), and each K/V tile staged in LDS
//     serves 384 queries;
//   * keys stream in tiles of 64 through two LDS stages, filled straight from
//     global memory by global_load_lds_dwordx4 (no staging registers): tile j+1
//     is requested at the top of the iteration that consumes tile j, and one
//     wait + barrier per tile publishes it;
//   * scores are computed transposed, S^T = K Q^T (16x16x32 MFMA: A = 16 keys x
//     32 channels from LDS, B = Q held in registers), so after the MFMA each
//     lane holds scores of ONE query column: the online-softmax max and sum are
//     lane-local plus two cross-lane steps (lanes l^16, l^32 share the query);
//   * the bf16 probabilities of two adjacent 16-key tiles are already the B
//     operand of O^T = V^T P^T (lane group g holds keys 4g..4g+3 of each tile);
//     the V^T A operand is read straight from the row-major V tile with the
//     gfx950 transposing LDS load ds_read_b64_tr_b16 (inside each 16-lane group,
//     lane i receives element i%4 of the 8 bytes lane 4j+i/4 addressed, so 16
//     lanes addressing 4 key rows x 16 channels each receive one channel with
//     its 4 keys), pointed at exactly those key rows;
//   * K and V rows (256 B) are stored unpadded with an XOR swizzle of the 16-byte
//     chunk index (K: chunk ^ (row % 16), V: chunk ^ 2*(row % 8)), so the 16 K
//     rows one lane group reads, and the 8 V rows x 32 B half a wave reads with
//     the transposing load, fall in distinct banks;
//   * the O^T accumulator keeps one query column per lane, so the rescale by
//     exp2(m_old - m_new) is lane-local, and the row sums of P are accumulated
//     by one extra MFMA against a row of ones. The running max only moves when a
//     tile's max exceeds it by more than 8 (log2 units): most tiles skip the
//     rescale; the stale max keeps p <= 2^8 (exact in fp32, far from bf16
//     overflow) and the final normalisation uses the same max, so the result is
//     unchanged;
//   * workgroups are numbered so that consecutive q-tiles of the same head land
//     on the same XCD (blocks are dispatched round-robin over the 8 XCDs), and
//     that XCD's L2 serves the head's K/V to all of them.
#include "common.hpp"
#include "kernels.hpp"

namespace wan {

namespace {

constexpr int kD = 128;                  // head dim
constexpr int kBN = 64;                  // keys per tile
#ifndef WAN_ATTN_QT
#define WAN_ATTN_QT 3
#endif
#ifndef WAN_ATTN_WAVES
#define WAN_ATTN_WAVES 8
#endif
constexpr int kQT = WAN_ATTN_QT;         // 16-query MFMA column tiles per wave
constexpr int kWaves = WAN_ATTN_WAVES;   // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 16 * kQT * kWaves;   // query rows per workgroup
constexpr int kRow = kD * 2;             // bytes per K or V row
constexpr int kTile = kBN * kRow;        // 16 KB
constexpr int kStage = 2 * kTile;        // K tile + V tile
constexpr float kRescaleSlack = 8.0f;    // log2 units the running max may lag behind the true max
constexpr int kWaitVmem0 = 0x0f70;       // s_waitcnt vmcnt(0), other counters unconstrained

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid & 7, j = bid >> 3;
  const int q = nb >> 3, r = nb & 7;
  return xcd * q + (xcd < r ? xcd : r) + j;
}

// Logical 16-byte chunk ch of row r sits at physical chunk ch ^ xor(r).
__device__ __forceinline__ int k_xor(int r) { return r & 15; }
__device__ __forceinline__ int v_xor(int r) { return 2 * (r & 7); }

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Per-kernel constants shared by the tile step below.
struct TileArgs {
  const uint16_t* base;  // K/V rows of this (b, h): element offset of channel 0 of row 0
  int S, rs, D, nkt, wave, lane, l16, grp, vr;
  float scale_log2;
};

// Direct global -> LDS staging of one 64-key tile: lane l of a wave
// instruction lands at the wave-uniform LDS base + 16*l. Each wave fills
// 16/kWaves 1 KB blocks (4 rows) of the K tile and of the V tile; lane l of a
// block takes physical row 4*blk + l/16, physical chunk l%16, and fetches the
// logical chunk the swizzle maps there. Rows past the end re-read row S-1
// (masked later).
__device__ __forceinline__ void issue_tile(const TileArgs& a, int k0, unsigned char* __restrict__ ks) {
#pragma unroll
  for (int j = 0; j < 16 / kWaves; ++j) {
    const int blk = (16 / kWaves) * a.wave + j;
    const int r = 4 * blk + (a.lane >> 4), pc = a.lane & 15;
    const uint16_t* rp = a.base + (int64_t)min(k0 + r, a.S - 1) * a.rs;
    __builtin_amdgcn_global_load_lds(rp + a.D + 8 * (pc ^ k_xor(r)), ks + blk * 1024, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(rp + 2 * a.D + 8 * (pc ^ v_xor(r)), ks + kTile + blk * 1024, 16, 0, 0);
  }
}

// One 64-key tile: scores, online softmax and PV from stage `cur`, while the
// next tile streams into stage `nxt`.
__device__ __forceinline__ void tile_step(const TileArgs& a, int kt, const unsigned char* __restrict__ cur,
                                          unsigned char* __restrict__ nxt, const bf16x8_t (&qf)[kQT][4],
                                          f32x4_t (&acc_o)[8][kQT], f32x4_t (&acc_l)[kQT], float (&m_run)[kQT],
                                          const bf16x8_t& ones) {
  const int k0 = kt * kBN;
  const unsigned char* ks = cur;
  const unsigned char* vs = cur + kTile;
  // The other stage was last read in iteration kt-1, which every wave has left.
  if (kt + 1 < a.nkt) issue_tile(a, k0 + kBN, nxt);

  // S^T: 4 key tiles (16 keys) x kQT query tiles, K over the 128 channels.
  f32x4_t acc_s[4][kQT];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int u = 0; u < kQT; ++u) acc_s[t][u] = f32x4_t{};
    const int r = 16 * t + a.l16;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(ks + r * kRow + 16 * ((4 * k + a.grp) ^ k_xor(r)));
#pragma unroll
      for (int u = 0; u < kQT; ++u) acc_s[t][u] = mfma16(av, qf[u][k], acc_s[t][u]);
    }
  }

  // Mask keys past the end (only the last tile can have them).
  if (k0 + kBN > a.S) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (k0 + 16 * t + 4 * a.grp + i >= a.S) {
#pragma unroll
          for (int u = 0; u < kQT; ++u) acc_s[t][u][i] = -INFINITY;
        }
  }

  // Online softmax per query column (base-2, scale folded in), lazily rescaled.
  bf16x8_t pf[kQT][2];
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    float mx = fmaxf(fmaxf(acc_s[0][u][0], acc_s[0][u][1]), fmaxf(acc_s[0][u][2], acc_s[0][u][3]));
#pragma unroll
    for (int t = 1; t < 4; ++t)
      mx = fmaxf(mx, fmaxf(fmaxf(acc_s[t][u][0], acc_s[t][u][1]), fmaxf(acc_s[t][u][2], acc_s[t][u][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * a.scale_log2;
    if (__ballot(mx > m_run[u] + kRescaleSlack)) {
      const float m_new = fmaxf(m_run[u], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[u] - m_new);
      m_run[u] = m_new;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_l[u][i] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_o[dt][u][i] *= alpha;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8_t v;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(acc_s[2 * c + (j >> 2)][u][j & 3], a.scale_log2, -m_run[u]));
      pf[u][c] = v;
      acc_l[u] = mfma16(ones, v, acc_l[u]);
    }
  }

  // Let the next tile's direct-to-LDS writes finish before the transposed V
  // reads: measured, the PV phase runs faster without those writes competing
  // for the LDS, and the loads have had the score and softmax phases to land.
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  // O^T (channels x queries) += V^T P^T: 8 channel tiles x 2 key steps of 32.
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const int ch = 2 * dt + ((a.l16 & 3) >> 1), sub = 8 * (a.l16 & 1);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int r0 = 32 * c + a.vr, r1 = r0 + 16;
      const s16x4_t lo = lds_read_tr16(vs + r0 * kRow + 16 * (ch ^ v_xor(r0)) + sub);
      const s16x4_t hi4 = lds_read_tr16(vs + r1 * kRow + 16 * (ch ^ v_xor(r1)) + sub);
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int u = 0; u < kQT; ++u) acc_o[dt][u] = mfma16(av, pf[u][c], acc_o[dt][u]);
    }
  }

  __builtin_amdgcn_s_waitcnt(kWaitVmem0);  // this wave's part of tile kt+1 has landed
  __syncthreads();                          // ... and every wave's; stage `cur` is free again
}

// Queries come from the Q part of one packed buffer (Sq rows per batch entry),
// keys and values from the K and V parts of another (Skv rows); for full
// attention both are the same buffer. F32Out selects an fp32 output (the
// chunked path, whose partial outputs are merged later) instead of bf16.
template <bool F32Out>
__global__ void __launch_bounds__(kThreads, (kQT >= 4 || kWaves > 4) ? 1 : 2)
attn_fwd_kernel(const uint16_t* __restrict__ qsrc, const uint16_t* __restrict__ kvsrc, void* __restrict__ out,
                float* __restrict__ lse, int Sq, int S, int heads, int nqt, float scale_log2) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStage];

  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = lid % nqt;
  const int bh = lid / nqt;
  const int h = bh % heads, b = bh / heads;
  const int D = heads * kD;
  const int rs = 3 * D;  // row stride in elements (< 2^17)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  TileArgs a;
  a.base = kvsrc + (int64_t)b * S * rs + h * kD;
  a.S = S;
  a.rs = rs;
  a.D = D;
  a.nkt = (S + kBN - 1) / kBN;
  a.wave = wave;
  a.lane = lane;
  a.l16 = l16;
  a.grp = grp;
  a.vr = 4 * grp + (l16 >> 2);  // V^T source row 4*grp + l16/4 (+32c, +16)
  a.scale_log2 = scale_log2;

  // Q fragments (B operand of S^T = K Q^T): query 16u + l16 of this wave,
  // channels 32k + 8*grp .. +7.
  const uint16_t* qbase = qsrc + (int64_t)b * Sq * rs + h * kD;
  const int q0 = qt * kBM + wave * 16 * kQT;
  bf16x8_t qf[kQT][4];
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    int q = q0 + 16 * u + l16;
    q = q < Sq ? q : Sq - 1;
    const uint16_t* qp = qbase + (int64_t)q * rs + 8 * grp;
#pragma unroll
    for (int k = 0; k < 4; ++k) qf[u][k] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * k);
  }
  // Complete the Q loads here: if they were still in flight at the loop head,
  // the wait for them would land inside the loop, where it would also wait for
  // the next tile's direct-to-LDS loads in every iteration. An empty asm that
  // reads every fragment pins the loads (and their wait) to this block.
#pragma unroll
  for (int u = 0; u < kQT; ++u)
#pragma unroll
    for (int k = 0; k < 4; ++k) asm volatile("" ::"v"(qf[u][k]));

  // Row sums of P come from the MFMA too: an A operand whose row 0 is all
  // bf16 ones (rows 1..15 zero) times P^T gives, in register 0 of lane l16 of
  // lane group 0, the sum of the bf16 probabilities of query l16 -- one extra
  // MFMA per 32 keys instead of a VALU add per score, and the normalisation uses
  // exactly the weights PV used.
  f32x4_t acc_o[8][kQT], acc_l[kQT];
  float m_run[kQT];
  const unsigned short one = l16 == 0 ? 0x3f80 : 0;
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, s16x8_t{(short)one, (short)one, (short)one, (short)one,
                                                              (short)one, (short)one, (short)one, (short)one});
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc_o[i][u] = f32x4_t{};
    acc_l[u] = f32x4_t{};
    m_run[u] = -INFINITY;
  }

  issue_tile(a, 0, smem);
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  __syncthreads();
  for (int kt = 0; kt < a.nkt; ++kt) {
    unsigned char* cur = smem + (kt & 1) * kStage;
    unsigned char* nxt = smem + ((kt + 1) & 1) * kStage;
    tile_step(a, kt, cur, nxt, qf, acc_o, acc_l, m_run, ones);
  }

  // Epilogue: O = O^T / l; lane holds 4 consecutive channels per (dt, u).
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    const float l_tot = __shfl(acc_l[u][0], l16, 64);  // sum of the bf16 P of query l16, in lane l16
    const int q = q0 + 16 * u + l16;
    if (q < Sq) {
      const float inv = 1.0f / l_tot;
      if constexpr (F32Out) {
        float* op = static_cast<float*>(out) + ((int64_t)b * Sq + q) * D + h * kD + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<f32x4_t*>(op + 16 * dt) = acc_o[dt][u] * inv;
      } else {
        uint16_t* op = static_cast<uint16_t*>(out) + ((int64_t)b * Sq + q) * D + h * kD + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          uint2 w;
          w.x = pack_bf16x2(acc_o[dt][u][0] * inv, acc_o[dt][u][1] * inv);
          w.y = pack_bf16x2(acc_o[dt][u][2] * inv, acc_o[dt][u][3] * inv);
          *reinterpret_cast<uint2*>(op + 16 * dt) = w;
        }
      }
      if (lse && grp == 0) lse[(int64_t)bh * Sq + q] = (m_run[u] + __log2f(l_tot)) * 0.69314718055994531f;
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd(const void* qkv, void* out, float* lse, int B, int S, int heads,
                           float softmax_scale, hipStream_t stream) {
  const int nqt = (S + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)nqt * heads * B;
  if (nblocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  const auto* src = static_cast<const uint16_t*>(qkv);
  hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, stream, src, src,
                     out, lse, S, S, heads, nqt, scale_log2);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_chunk(const void* q_src, int Sq, const void* kv_src, int Skv, float* out, float* lse, int B,
                                 int heads, float softmax_scale, hipStream_t stream) {
  const int nqt = (Sq + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)nqt * heads * B;
  if (nblocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q_src), static_cast<const uint16_t*>(kv_src), out, lse, Sq, Skv,
                     heads, nqt, scale_log2);
  return hipGetLastError();
}

}  // namespace wan
