// Bidirectional multi-head flash-attention forward on the packed [Q|K|V]
// buffer, bf16 MFMA with fp32 accumulation (gfx950 v_mfma_f32_16x16x32_bf16).
//
// What it computes: for every (batch, head) and every query row, softmax over
// ALL keys of (q . k) * scale, times V -- the unmasked attention of the Wan2.2
// DiT ("Optimizing High-Quality Offline Video Generation", Overview: the
// denoiser is bidirectional). The S x S score matrix never leaves registers.
//
// Work decomposition
//   * one workgroup = 4 wavefronts = 128 query rows of one (b, h); each wave owns
//     32 rows (two 16-row MFMA column tiles) for the whole kernel;
//   * keys stream in units of 32 through a ring of four LDS stages. In the
//     iteration that consumes unit j, the scores of unit j+1 are computed (MFMA)
//     while the exponentials of unit j run (VALU), then PV of unit j; unit j+2,
//     loaded into registers one iteration earlier, is written to the stage unit
//     j-2 used, and one barrier per unit publishes it;
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
//   * the O^T accumulator keeps one query column per lane, so the rescale by
//     exp2(m_old - m_new) is lane-local. The running max only moves when a
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
constexpr int kBN = 32;                  // keys per pipeline unit
constexpr int kStages = 4;               // LDS ring of K/V units
constexpr int kWaves = 4;                // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;         // query rows per workgroup
#ifndef WAN_ATTN_KPAD
#define WAN_ATTN_KPAD 16
#endif
#ifndef WAN_ATTN_VPAD
#define WAN_ATTN_VPAD 32
#endif
constexpr int kKPitch = kD * 2 + WAN_ATTN_KPAD;  // K row pitch in LDS: 16 rows at distinct 4-bank offsets (b128 reads)
constexpr int kVPitch = kD * 2 + WAN_ATTN_VPAD;  // V row pitch: 8 rows x 32 B tile the 64 banks (transposed b64 reads)
constexpr int kKBytes = kBN * kKPitch;
constexpr int kVBytes = kBN * kVPitch;
constexpr int kStage = kKBytes + kVBytes;
constexpr int kChunks = kBN * 16 / kThreads;  // 16-byte chunks of K (and of V) per thread per unit
constexpr float kRescaleSlack = 8.0f;    // log2 units the running max may lag behind the true max

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid & 7, j = bid >> 3;
  const int q = nb >> 3, r = nb & 7;
  return xcd * q + (xcd < r ? xcd : r) + j;
}

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__global__ void __launch_bounds__(kThreads, 2)
attn_fwd_kernel(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ out, float* __restrict__ lse,
                int S, int heads, int nqt, float scale_log2) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * kStage];

  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = lid % nqt;
  const int bh = lid / nqt;
  const int h = bh % heads, b = bh / heads;
  const int D = heads * kD;
  const int rs = 3 * D;  // row stride in elements (< 2^17)
  const uint16_t* base = qkv + (int64_t)b * S * rs + h * kD;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, grp = lane >> 4;

  // Q fragments (B operand of S^T = K Q^T): query 16u + l16 of this wave,
  // channels 32k + 8*grp .. +7.
  const int q0 = qt * kBM + wave * 32;
  bf16x8_t qf[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    int q = q0 + 16 * u + l16;
    q = q < S ? q : S - 1;
    const uint16_t* qp = base + (int64_t)q * rs + 8 * grp;
#pragma unroll
    for (int k = 0; k < 4; ++k) qf[u][k] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * k);
  }

  f32x4_t acc_o[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc_o[i][0] = acc_o[i][1] = f32x4_t{};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  // Staging of one unit (32 keys) of K and V: chunk c = tid + 256 i -> key c/16,
  // channels 8*(c%16). Offsets are 32-bit element offsets from the unit's first row.
  int g_off[kChunks], sk_off[kChunks], sv_off[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int c = tid + i * kThreads;
    g_off[i] = (c >> 4) * rs + 8 * (c & 15);
    sk_off[i] = (c >> 4) * kKPitch + (c & 15) * 16;
    sv_off[i] = (c >> 4) * kVPitch + (c & 15) * 16;
  }
  u32x4_t kreg[kChunks], vreg[kChunks];
  auto load_unit = [&](int k0) {
    const uint16_t* ub = base + (int64_t)k0 * rs;
    if (k0 + kBN <= S) {
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        kreg[i] = *reinterpret_cast<const u32x4_t*>(ub + g_off[i] + D);
        vreg[i] = *reinterpret_cast<const u32x4_t*>(ub + g_off[i] + 2 * D);
      }
    } else {  // ragged last unit: rows past the end re-read row S-1 (masked later)
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const int c = tid + i * kThreads;
        const int r = min(c >> 4, S - 1 - k0);
        const uint16_t* rp = ub + r * rs + 8 * (c & 15);
        kreg[i] = *reinterpret_cast<const u32x4_t*>(rp + D);
        vreg[i] = *reinterpret_cast<const u32x4_t*>(rp + 2 * D);
      }
    }
  };
  auto store_unit = [&](int stage) {
    unsigned char* ks = smem + stage * kStage;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      *reinterpret_cast<u32x4_t*>(ks + sk_off[i]) = kreg[i];
      *reinterpret_cast<u32x4_t*>(ks + kKBytes + sv_off[i]) = vreg[i];
    }
  };

  // Per-lane LDS offsets: K A-operand row l16 at channel 8*grp; V^T source row
  // 4*grp + l16/4 at channel 4*(l16%4).
  const int k_off = l16 * kKPitch + 16 * grp;
  const int v_off = kKBytes + (4 * grp + (l16 >> 2)) * kVPitch + 8 * (l16 & 3);

  // S^T of one unit: 2 key tiles (16 keys) x 2 query tiles, over 128 channels.
  auto scores = [&](int stage, f32x4_t (&acc)[2][2]) {
    const unsigned char* ks = smem + stage * kStage + k_off;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      acc[t][0] = acc[t][1] = f32x4_t{};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ks + 16 * t * kKPitch + 64 * k);
        acc[t][0] = mfma16(a, qf[0][k], acc[t][0]);
        acc[t][1] = mfma16(a, qf[1][k], acc[t][1]);
      }
    }
  };

  const int nu = (S + kBN - 1) / kBN;
  load_unit(0);
  store_unit(0);
  if (nu > 1) {
    load_unit(kBN);
    store_unit(1);
  }
  __syncthreads();
  if (nu > 2) load_unit(2 * kBN);
  f32x4_t sc[2][2];
  scores(0, sc);

  for (int un = 0; un < nu; ++un) {
    const int k0 = un * kBN;
    // LDS holds units un and un+1 (stages un%4, (un+1)%4); unit un+2 is in registers.

    if (k0 + kBN > S) {  // mask keys past the end (last unit only)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k0 + 16 * t + 4 * grp + i >= S) sc[t][0][i] = sc[t][1][i] = -INFINITY;
    }

    // Running max per query column (base-2, scale folded in), lazily moved.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float mx = fmaxf(fmaxf(sc[0][u][0], sc[0][u][1]), fmaxf(sc[0][u][2], sc[0][u][3]));
      mx = fmaxf(mx, fmaxf(fmaxf(sc[1][u][0], sc[1][u][1]), fmaxf(sc[1][u][2], sc[1][u][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
      if (__ballot(mx > m_run[u] + kRescaleSlack)) {
        const float m_new = fmaxf(m_run[u], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[u] - m_new);
        m_run[u] = m_new;
        l_run[u] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc_o[dt][u][i] *= alpha;
      }
    }

    // Scores of the next unit (MFMA) overlap the exponentials of this one
    // (VALU). On the last unit the stage read is stale but in bounds and the
    // result is discarded; computing it unconditionally keeps the MFMAs and
    // the exponentials in one basic block so they can be interleaved.
    f32x4_t sn[2][2];
    scores((un + 1) % kStages, sn);

    bf16x8_t pf[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float psum = 0.f;
      bf16x8_t v;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[j >> 2][u][j & 3], scale_log2, -m_run[u]));
        psum += p;
        v[j] = (__bf16)p;
      }
      pf[u] = v;
      l_run[u] += psum;
    }
#if WAN_ATTN_SCHED
    // Issue order: the 8 K reads of the next unit, then each of its 16 MFMAs
    // followed by a share of the exponential / conversion VALU work.
#pragma unroll
    for (int i = 0; i < 8; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, WAN_ATTN_SCHED, 0);
    }
#endif

    // O^T (channels x queries) += V^T P^T: 8 channel tiles, one 32-key step.
    {
      const unsigned char* vp = smem + (un % kStages) * kStage + v_off;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const s16x4_t lo = lds_read_tr16(vp + 32 * dt);
        const s16x4_t hi4 = lds_read_tr16(vp + 16 * kVPitch + 32 * dt);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        acc_o[dt][0] = mfma16(a, pf[0], acc_o[dt][0]);
        acc_o[dt][1] = mfma16(a, pf[1], acc_o[dt][1]);
      }
    }

    // Stage (un+2)%4 last held unit un-2, which every wave finished in an
    // earlier iteration (barrier below), so unit un+2 can be written now.
    store_unit((un + 2) % kStages);  // past the end: stale registers into a stage no longer read
    __syncthreads();
    if (un + 3 < nu) load_unit((un + 3) * kBN);
#pragma unroll
    for (int t = 0; t < 2; ++t) sc[t][0] = sn[t][0], sc[t][1] = sn[t][1];
  }

  // Epilogue: O = O^T / l in bf16; lane holds 4 consecutive channels per (dt, u).
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    float l_tot = l_run[u] + __shfl_xor(l_run[u], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int q = q0 + 16 * u + l16;
    if (q < S) {
      const float inv = 1.0f / l_tot;
      uint16_t* op = out + ((int64_t)b * S + q) * D + h * kD + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint2 w;
        w.x = pack_bf16x2(acc_o[dt][u][0] * inv, acc_o[dt][u][1] * inv);
        w.y = pack_bf16x2(acc_o[dt][u][2] * inv, acc_o[dt][u][3] * inv);
        *reinterpret_cast<uint2*>(op + 16 * dt) = w;
      }
      if (lse && grp == 0) lse[(int64_t)bh * S + q] = (m_run[u] + __log2f(l_tot)) * 0.69314718055994531f;
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
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(qkv), static_cast<uint16_t*>(out), lse, S, heads, nqt,
                     scale_log2);
  return hipGetLastError();
}

}  // namespace wan
