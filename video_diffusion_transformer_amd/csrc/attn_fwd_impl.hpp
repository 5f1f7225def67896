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
//     global memory by buffer_load_dwordx4 ... lds (no staging registers): tile j+1
//     is requested during the score MFMAs of the iteration that consumes tile j, and one
//     wait + barrier per tile publishes it;
//   * scores are computed transposed, S^T = K Q^T (16x16x32 MFMA: A = 16 keys x
//     32 channels from LDS, B = Q held in registers), so after the MFMA each
//     lane holds scores of ONE query column: the online-softmax max is
//     lane-local, plus two cross-lane steps (lanes l^16, l^32 share the query)
//     only on the tiles where the running max moves;
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
//     exp2(m_old - m_new) is lane-local, and each lane sums its own bf16
//     probabilities (packed dot products with (1, 1); the instances that
//     return a log-sum-exp sum the fp32 probabilities instead, so the LSE is
//     exact up to fp32 rounding). The running max only moves when a
//     tile's max exceeds it by more than 8 (log2 units): most tiles skip the
//     rescale; the stale max keeps p <= 2^8 (exact in fp32, far from bf16
//     overflow) and the final normalisation uses the same max, so the result is
//     unchanged;
//   * workgroups are numbered so that consecutive q-tiles of the same head land
//     on the same XCD (blocks are dispatched round-robin over the 8 XCDs), and
//     that XCD's L2 serves the head's K/V to all of them.
//
// This header holds the kernel template; attn_fwd.hip instantiates the
// instances that normalise by the bf16 weights (the attention step and
// Skip-Softmax) and is compiled with the max-ILP machine scheduler,
// attn_fwd_exact.hip those that return a log-sum-exp (the fp32-sum instances:
// dense with LSE, the ring chunk and fold modes), compiled with the default
// scheduler, which measured faster for them (they spill a few registers).
#pragma once

#include <cmath>

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
constexpr int kStages = 2;               // LDS stages (K + V tile each)
constexpr float kRescaleSlack = 8.0f;    // log2 units the running max may lag behind the true max
constexpr float kSumLimit = 256.0f;      // 2^kRescaleSlack: bound on a lane's sum of one tile's probabilities
static_assert(kSumLimit == static_cast<float>(1 << static_cast<int>(kRescaleSlack)), "the sum limit is 2^slack");
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
  int S, rs, D, nkt, wave, lane, l16, grp;
  int kb, vb;  // per-lane byte offsets of the first K / V^T fragment read in a stage
  uint32_t gk[16 / kWaves], gv[16 / kWaves];  // per-lane byte offsets of the K / V chunks a lane stages
  float scale_log2;
};

// Direct global -> LDS staging of one 64-key tile (buffer_load_dwordx4 ...
// lds): lane l of a wave instruction lands at the wave-uniform LDS base +
// 16*l. Each wave fills kBlk 1 KB blocks (4 rows) of the K tile and of the V
// tile; lane l of a block takes physical row 4*blk + l/16, physical chunk
// l%16, and fetches the logical chunk the swizzle maps there. The per-lane byte
// offsets from the tile's first row are fixed (gk, gv). One buffer descriptor
// per tile covers the rows that exist, so rows past S read as zeros (masked
// later). (The global_load_lds form of the same copy measured 2% slower.)
constexpr int kBlk = 16 / kWaves;  // 1 KB blocks per wave per K or V tile
static_assert(16 % kWaves == 0, "the 16 blocks of a K or V tile must split evenly over the waves");

__device__ __forceinline__ int tile_row(const TileArgs& a, int j) { return 4 * (kBlk * a.wave + j) + (a.lane >> 4); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void issue_tile(const TileArgs& a, int k0, unsigned char* __restrict__ smem, int off) {
  const uint16_t* tb = a.base + (int64_t)k0 * a.rs;  // wave-uniform
  const int rows = min(kBN, a.S - k0);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(tb), (short)0, rows * a.rs * 2, 0x00020000);
  unsigned char* dst = smem + off + kBlk * a.wave * 1024;
#pragma unroll
  for (int j = 0; j < kBlk; ++j) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + j * 1024), 16, a.gk[j], 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + kTile + j * 1024), 16, a.gv[j], 0, 0, 0);
  }
}

// S^T for one 64-key tile: 4 key tiles (16 keys) x kQT query tiles, K over
// the 128 channels. A = 16 keys x 32 channels from LDS, B = Q in registers.
// Lane (l16, grp) reads row 16t + l16, logical chunk 4k + grp, at physical
// chunk (4k + grp) ^ l16: byte offset kb ^ 64k (kb = the k = 0 offset) plus
// 4096t. The stage offset (a multiple of 32 KB) is added before the XOR and
// hidden from the optimiser, so the four addresses cost one XOR each per tile
// instead of four registers held across the loop.
__device__ __forceinline__ void tile_scores(const TileArgs& a, const unsigned char* __restrict__ smem, int k_off,
                                            const bf16x8_t (&qf)[kQT][4], f32x4_t (&acc_s)[4][kQT]) {
  int x = k_off + a.kb;
  asm("" : "+v"(x));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int u = 0; u < kQT; ++u) acc_s[t][u] = f32x4_t{};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(smem + (x ^ (64 * k)) + 4096 * t);
#pragma unroll
      for (int u = 0; u < kQT; ++u) acc_s[t][u] = mfma16(av, qf[u][k], acc_s[t][u]);
    }
  }
}

// Max step of the online softmax of one tile (base-2, scale folded in): masks
// keys past the end, and moves the running max of a query column only when the
// tile's max exceeds it by more than the slack. The row sums are rescaled here;
// returns a bit per query tile whose max moved, with the factor alpha the
// output accumulator must be scaled by.
// Scales the output accumulator of the query tiles whose max moved.
__device__ __forceinline__ void tile_rescale(unsigned moved, const float (&alpha)[kQT], f32x4_t (&acc_o)[8][kQT]) {
#pragma unroll
  for (int u = 0; u < kQT; ++u)
    if (moved & (1u << u)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_o[dt][u][i] *= alpha[u];
    }
}

// p = 2^(s * scale_log2 - m) rounded to bf16, written in the B-operand layout
// of PV (two 32-key steps per query tile: lane group g holds keys 4g..4g+3 of
// 16-key tiles 2c and 2c+1); each lane sums its own keys. Without ExactSum the
// row sums add up exactly the bf16 weights PV multiplies (a dot product of each
// packed pair with (1, 1), fp32 sum: 4 instructions per 8 weights), so the
// normalisation matches what PV accumulated. With ExactSum they add the fp32
// probabilities before rounding (8 adds per 8 weights), so that ln of the sum is
// the log-sum-exp of the scores up to fp32 rounding: the instances that return
// an LSE use it.
template <bool ExactSum>
__device__ __forceinline__ float exp_pack8(const TileArgs& a, const f32x4_t (&acc_s)[4][kQT], float m, int u, int c,
                                           bf16x8_t& out, float l) {
  const bf16x2_t one2 = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  bf16x8_t v;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float e = __builtin_amdgcn_exp2f(fmaf(acc_s[2 * c + (j >> 2)][u][j & 3], a.scale_log2, -m));
    v[j] = (__bf16)e;
    if constexpr (ExactSum) l += e;
  }
  out = v;
  if constexpr (!ExactSum) {
    // Literal shuffles: extracting the pairs through a bit cast to 32-bit
    // lanes is miscompiled by this clang (every extraction read element 0).
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one2, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one2, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one2, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one2, l, false);
  }
  return l;
}

template <bool ExactSum>
__device__ __forceinline__ void tile_exp(const TileArgs& a, const f32x4_t (&acc_s)[4][kQT], const float (&m_run)[kQT],
                                         bf16x8_t (&pf)[kQT][2], float (&lt)[kQT]) {
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    lt[u] = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) lt[u] = exp_pack8<ExactSum>(a, acc_s, m_run[u], u, c, pf[u][c], lt[u]);
  }
}

// One query tile redone against a new running max (the rare path of tile_softmax).
template <bool ExactSum>
__device__ __forceinline__ void tile_exp_one(const TileArgs& a, const f32x4_t (&acc_s)[4][kQT], float m, int u,
                                             bf16x8_t (&pf)[kQT][2], float& lt) {
  lt = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) lt = exp_pack8<ExactSum>(a, acc_s, m, u, c, pf[u][c], lt);
}

// Softmax step with optimistic exponentials: all probabilities of the tile are
// computed against the running max first. If some lane's sum over its 16 keys
// of a query tile exceeds 2^slack (or is infinite: on the first tile the
// running max is the most negative float), a score passed the running max by
// more than the slack; that query tile is then redone against the new max (the
// column max of the tile's scores), with the running sum rescaled and the
// query tile marked for the output rescale. Each probability is at most its
// lane's sum, so p <= 2^slack on every kept tile: the bound a max test before
// the exponentials gives, without computing the max where it does not move.
template <bool ExactSum>
__device__ __forceinline__ unsigned tile_softmax(const TileArgs& a, int k0, f32x4_t (&acc_s)[4][kQT],
                                                 float (&m_run)[kQT], float (&acc_l)[kQT], float (&alpha)[kQT],
                                                 bf16x8_t (&pf)[kQT][2]) {
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
  float lt[kQT];
  tile_exp<ExactSum>(a, acc_s, m_run, pf, lt);
  bool over = false;
#pragma unroll
  for (int u = 0; u < kQT; ++u) over = over || lt[u] > kSumLimit;
  unsigned moved = 0;
#pragma unroll
  for (int u = 0; u < kQT; ++u) alpha[u] = 1.0f;
  if (__ballot(over)) {
#pragma unroll
    for (int u = 0; u < kQT; ++u)
      if (__ballot(lt[u] > kSumLimit)) {
        float mx = fmaxf(fmaxf(acc_s[0][u][0], acc_s[0][u][1]), fmaxf(acc_s[0][u][2], acc_s[0][u][3]));
#pragma unroll
        for (int t = 1; t < 4; ++t)
          mx = fmaxf(mx, fmaxf(fmaxf(acc_s[t][u][0], acc_s[t][u][1]), fmaxf(acc_s[t][u][2], acc_s[t][u][3])));
        mx *= a.scale_log2;
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run[u], mx);
        alpha[u] = __builtin_amdgcn_exp2f(m_run[u] - m_new);
        m_run[u] = m_new;
        acc_l[u] *= alpha[u];
        moved |= 1u << u;
        tile_exp_one<ExactSum>(a, acc_s, m_new, u, pf, lt[u]);
      }
  }
#pragma unroll
  for (int u = 0; u < kQT; ++u) acc_l[u] += lt[u];
  return moved;
}

// O^T (channels x queries) += V^T P^T over one tile: 8 channel tiles x 2 key
// steps of 32. The V^T fragment comes from two transposing LDS reads of the
// row-major V tile: lane (l16, grp) reads rows 32c + 4grp + l16/4 (+16),
// logical chunk 2dt + (l16%4)/2, half l16%2. The swizzle XORs the chunk with
// 2 (row % 8), so the byte offset is vb ^ 32dt (vb = the dt = 0 offset) plus
// 8192c (+4096); as for K, one XOR per address.
__device__ __forceinline__ void tile_pv(const TileArgs& a, const unsigned char* __restrict__ smem, int v_off,
                                        const bf16x8_t (&pf)[kQT][2], f32x4_t (&acc_o)[8][kQT]) {
  int x = v_off + a.vb;
  asm("" : "+v"(x));
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const unsigned char* p = smem + (x ^ (32 * dt));
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const s16x4_t lo = lds_read_tr16(p + 8192 * c);
      const s16x4_t hi4 = lds_read_tr16(p + 8192 * c + 4096);
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int u = 0; u < kQT; ++u) acc_o[dt][u] = mfma16(av, pf[u][c], acc_o[dt][u]);
    }
  }
}

// Skip-Softmax, threshold mode (the vLLM-Omni recipe "Wan2.2 Text-to-Video",
// Skip-Softmax controls: a direct skip threshold, no calibration). The rule
// (the pages give only the knob): keys go in tiles of 64 in increasing order;
// a tile's softmax and PV are skipped for a wave's 48 query rows when, for
// every one of them, exp(tile max - running max) < threshold, the running max
// being that of the softmax, i.e. of the tiles kept so far. The scores of
// every tile are computed (the decision needs them); a kept tile runs the
// softmax against the exact running max (no lazy rescale: p <= 1).
struct SkipArgs {
  float thr_log2;  // log2(threshold) in the scaled log2 units of the scores; -inf keeps every tile
  uint8_t* kept;   // optional decision map [B*heads][nqb][nkt] (1 = kept), or null
  int nqb;         // query blocks (of 48 rows) per (b, h)
};

// The decision for one tile: masks keys past the end, leaves the column
// max of each query tile in mx (scaled log2 units) and returns whether some
// query of the wave has exp(tile max - running max) >= threshold.
__device__ __forceinline__ bool skip_decide(const TileArgs& a, int k0, float thr_log2, f32x4_t (&acc_s)[4][kQT],
                                            const float (&m_run)[kQT], float (&mx)[kQT]) {
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
  bool need = false;
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    float m = fmaxf(fmaxf(acc_s[0][u][0], acc_s[0][u][1]), fmaxf(acc_s[0][u][2], acc_s[0][u][3]));
#pragma unroll
    for (int t = 1; t < 4; ++t) m = fmaxf(m, fmaxf(fmaxf(acc_s[t][u][0], acc_s[t][u][1]), fmaxf(acc_s[t][u][2], acc_s[t][u][3])));
    m *= a.scale_log2;
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));  // the column max: every lane of the query holds it
    mx[u] = m;
    need = need || (m - m_run[u] >= thr_log2);  // m_run = -inf before the first tile: always kept
  }
  return __ballot(need) != 0;
}

// Softmax of a kept tile against the exact running max: rescales the row sums
// and output accumulator of the query tiles whose max moved, leaves the bf16 P in pf.
template <bool ExactSum>
__device__ __forceinline__ void skip_softmax(const TileArgs& a, const f32x4_t (&acc_s)[4][kQT], const float (&mx)[kQT],
                                             float (&m_run)[kQT], float (&acc_l)[kQT], f32x4_t (&acc_o)[8][kQT],
                                             bf16x8_t (&pf)[kQT][2]) {
#pragma unroll
  for (int u = 0; u < kQT; ++u)
    if (__ballot(mx[u] > m_run[u])) {
      const float m_new = fmaxf(m_run[u], mx[u]);
      const float alpha = __builtin_amdgcn_exp2f(m_run[u] - m_new);  // 0 on the first tile
      m_run[u] = m_new;
      acc_l[u] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_o[dt][u][i] *= alpha;
    }
  float lt[kQT];
  tile_exp<ExactSum>(a, acc_s, m_run, pf, lt);
#pragma unroll
  for (int u = 0; u < kQT; ++u) acc_l[u] += lt[u];
}

// Queries come from the Q part of one packed buffer (Sq rows per batch entry),
// keys and values from the K and V parts of another (Skv rows); for full
// attention both are the same buffer. The output mode: bf16 O (full
// attention); fp32 O and the LSE of this key chunk (one ring round); or the
// chunk's result folded straight into an fp32 accumulator and its LSE (one ring
// round with the merge in the epilogue, out16 optionally receiving a bf16 copy).
enum OutMode { kOutBf16 = 0, kOutF32 = 1, kOutFold = 2 };

template <int Mode, bool ExactSum, bool Skip>
__global__ void __launch_bounds__(kThreads, (kQT >= 4 || kWaves > 4) ? 1 : 2)
attn_fwd_kernel(const uint16_t* __restrict__ qsrc, const uint16_t* __restrict__ kvsrc, void* __restrict__ out,
                float* __restrict__ lse, uint16_t* __restrict__ out16, int Sq, int S, int heads, int nqt,
                float scale_log2, SkipArgs sk) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * kStage];

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
  a.wave = __builtin_amdgcn_readfirstlane(wave);
  a.lane = lane;
  a.l16 = l16;
  a.grp = grp;
#pragma unroll
  for (int j = 0; j < kBlk; ++j) {
    const int r = tile_row(a, j), pc = lane & 15;
    a.gk[j] = 2 * (r * rs + D + 8 * (pc ^ k_xor(r)));
    a.gv[j] = 2 * (r * rs + 2 * D + 8 * (pc ^ v_xor(r)));
  }
  a.kb = l16 * kRow + 16 * ((grp ^ l16) & 3) + 64 * (l16 >> 2);
  {
    const int vr = 4 * grp + (l16 >> 2);  // V^T source row (+32c, +16)
    a.vb = kTile + vr * kRow + 32 * (vr & 7) + 16 * ((l16 & 3) >> 1) + 8 * (l16 & 1);
  }
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

  f32x4_t acc_o[8][kQT];
  float acc_l[kQT], m_run[kQT];  // per-lane partial row sums (this lane's keys), running max
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc_o[i][u] = f32x4_t{};
    acc_l[u] = 0.0f;
    m_run[u] = -3.0e38f;  // finite: s - m_run is +inf (or -inf for masked keys), never NaN
  }

  float alpha[kQT];
  if constexpr (Skip) {
#pragma unroll
    for (int u = 0; u < kQT; ++u) m_run[u] = -INFINITY;  // exact running max: no tile seen yet
  }
  const int qblock = qt * kWaves + wave;  // Skip: this wave's 48-row query block
  f32x4_t acc_s[4][kQT];
  bf16x8_t pf[kQT][2];
  issue_tile(a, 0, smem, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  __syncthreads();
  for (int kt = 0; kt < a.nkt; ++kt) {
    const int cur = (kt & 1) * kStage;
    // The copies of tile kt+1 (past the last tile: the last tile again, into
    // the stage nobody reads any more) go into the other stage, last read in
    // iteration kt-1, which every wave has left. They follow the score
    // fragment reads in program order and are spread over the score MFMAs, one
    // per 8 (+1% over issuing them in one burst at the top).
    tile_scores(a, smem, cur, qf, acc_s);
    issue_tile(a, min(kt + 1, a.nkt - 1) * kBN, smem, ((kt + 1) & 1) * kStage);
#pragma unroll
    for (int q = 0; q < 2 * kBlk; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // 8 MFMAs
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // 1 copy
    }
    if constexpr (Skip) {
      float mx[kQT];
      const bool keep = skip_decide(a, kt * kBN, sk.thr_log2, acc_s, m_run, mx);
      if (sk.kept && lane == 0 && qblock < sk.nqb) sk.kept[((int64_t)bh * sk.nqb + qblock) * a.nkt + kt] = keep;
      if (keep) {
        skip_softmax<ExactSum>(a, acc_s, mx, m_run, acc_l, acc_o, pf);
        __builtin_amdgcn_s_waitcnt(kWaitVmem0);
        tile_pv(a, smem, cur, pf, acc_o);
      }
    } else {
      const unsigned moved = tile_softmax<ExactSum>(a, kt * kBN, acc_s, m_run, acc_l, alpha, pf);
      if (moved) tile_rescale(moved, alpha, acc_o);
      // Let the next tile's direct-to-LDS writes finish before the transposed V
      // reads: measured, the PV phase runs faster without those writes competing
      // for the LDS, and the loads have had the score and softmax phases to land.
      __builtin_amdgcn_s_waitcnt(kWaitVmem0);
      tile_pv(a, smem, cur, pf, acc_o);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);  // this wave's part of tile kt+1 has landed
    __syncthreads();                          // ... and every wave's; this stage is free again
  }

  // Epilogue: O = O^T / l; lane holds 4 consecutive channels per (dt, u).
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    float l_tot = acc_l[u];  // the four lanes of a query column hold disjoint keys
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int q = q0 + 16 * u + l16;
    if (q < Sq) {
      const float inv = 1.0f / l_tot;
      if constexpr (Mode == kOutFold) {
        const int64_t li = (int64_t)bh * Sq + q;
        const LseFold fo = lse_fold(lse[li], (m_run[u] + __log2f(l_tot)) * 0.69314718055994531f);
        const int64_t o0 = ((int64_t)b * Sq + q) * D + h * kD + 4 * grp;
        float* op = static_cast<float*>(out) + o0;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const f32x4_t c = acc_o[dt][u] * inv;
          const f32x4_t av = fo.acc_empty ? f32x4_t{} : *reinterpret_cast<const f32x4_t*>(op + 16 * dt);
          f32x4_t r;
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = lse_fold_value(fo, av[i], c[i]);
          *reinterpret_cast<f32x4_t*>(op + 16 * dt) = r;
          if (out16) {
            uint2 w;
            w.x = pack_bf16x2(r[0], r[1]);
            w.y = pack_bf16x2(r[2], r[3]);
            *reinterpret_cast<uint2*>(out16 + o0 + 16 * dt) = w;
          }
        }
        // every lane of the query has read the old LSE above (same wave, earlier)
        if (grp == 0) lse[li] = fo.L;
        continue;
      }
      if constexpr (Mode == kOutF32) {
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

}  // namespace wan
