// Bidirectional multi-head flash-attention forward on the packed [Q|K|V]
// buffer, bf16 MFMA with fp32 accumulation (gfx950 v_mfma_f32_32x32x16_bf16).
//
// What it computes: for every (batch, head) and every query row, softmax over
// ALL keys of (q . k) * scale, times V -- the unmasked attention of the Wan2.2
// DiT ("Optimizing High-Quality Offline Video Generation", Overview: the
// denoiser is bidirectional). The S x S score matrix never leaves registers.
//
// Work decomposition
//   * one workgroup = 4 wavefronts = 128 query rows of one (b, h); each wave owns
//     32 rows for the whole kernel;
//   * keys stream in tiles of 64; each tile's K (row-major) and V (transposed to
//     [channel][key]) are staged in LDS, the next tile is prefetched into
//     registers while the current one is consumed;
//   * scores are computed transposed, S^T = K Q^T, so that after the MFMA every
//     lane holds 32 key scores of ONE query row: the running max / sum of the
//     online softmax stay lane-local (one cross-lane max with the partner lane
//     l^32 per tile), and the bf16 probabilities are already in the register
//     layout of the B operand of O^T = V^T P^T. The K rows are fed to the MFMA
//     in a permuted order (bits 2 and 3 of the row swapped) so that the
//     accumulator's key order matches the operand's k order exactly;
//   * the output accumulator O^T keeps one query column per lane, so the
//     per-row rescale by exp2(m_old - m_new) is lane-local too;
//   * workgroups are numbered so that consecutive q-tiles of the same head land
//     on the same XCD (blocks are dispatched round-robin over the 8 XCDs), and
//     that XCD's L2 serves the head's K/V to all of them.
#include "common.hpp"
#include "kernels.hpp"

namespace wan {

namespace {

constexpr int kD = 128;                  // head dim
constexpr int kBN = 64;                  // keys per tile
constexpr int kWaves = 4;                // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;         // query rows per workgroup
constexpr int kKPitch = kD * 2 + 16;     // bytes per K row in LDS (16 B pad: conflict-free b128 reads)
constexpr int kVPitch = kBN * 2 + 16;    // bytes per V^T row in LDS
constexpr int kKBytes = kBN * kKPitch;
constexpr int kVBytes = kD * kVPitch;

// Row of the 32-key sub-tile that the MFMA A-operand lane m must load so that
// accumulator register 4g+r of lane l holds key 16*(g/2) + 8*(l/32) + 4*(g%2) + r.
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid & 7, j = bid >> 3;
  const int q = nb >> 3, r = nb & 7;
  return xcd * q + (xcd < r ? xcd : r) + j;
}

__global__ void __launch_bounds__(kThreads, 2)
attn_fwd_kernel(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ out, float* __restrict__ lse,
                int S, int heads, int nqt, float scale_log2) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kKBytes + kVBytes];
  unsigned char* ks = smem;
  unsigned char* vs = smem + kKBytes;

  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = lid % nqt;
  const int bh = lid / nqt;
  const int h = bh % heads, b = bh / heads;
  const int D = heads * kD;
  const int64_t rs = 3 * (int64_t)D;  // row stride in elements
  const uint16_t* base = qkv + (int64_t)b * S * rs + h * kD;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // Q fragment (B operand of S^T = K Q^T): query row l32 of this wave, channels 16k + 8*hi.
  const int qrow = qt * kBM + wave * 32 + l32;
  const int qrow_c = qrow < S ? qrow : S - 1;
  bf16x8_t qf[8];
  {
    const uint16_t* qp = base + (int64_t)qrow_c * rs + 8 * hi;
#pragma unroll
    for (int k = 0; k < 8; ++k) qf[k] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * k);
  }

  f32x16_t acc_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc_o[i] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  // Global -> register staging of one K/V tile. K: 4 x 16 B per thread, key = c/16, chunk c%16.
  // V: key = tid%64, channel group 8*(tid/64 + 4i).
  u32x4_t kreg[4], vreg[4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * kThreads;
      int key = k0 + (c >> 4);
      key = key < S ? key : S - 1;
      kreg[i] = *reinterpret_cast<const u32x4_t*>(base + (int64_t)key * rs + D + 8 * (c & 15));
    }
    int key = k0 + lane;
    key = key < S ? key : S - 1;
    const uint16_t* vp = base + (int64_t)key * rs + 2 * D;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vreg[i] = *reinterpret_cast<const u32x4_t*>(vp + 8 * (wave + 4 * i));
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * kThreads;
      *reinterpret_cast<u32x4_t*>(ks + (c >> 4) * kKPitch + (c & 15) * 16) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 8 * (wave + 4 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<uint16_t*>(vs + (d0 + 2 * j) * kVPitch + lane * 2) = static_cast<uint16_t>(vreg[i][j]);
        *reinterpret_cast<uint16_t*>(vs + (d0 + 2 * j + 1) * kVPitch + lane * 2) = static_cast<uint16_t>(vreg[i][j] >> 16);
      }
    }
  };

  const int nkt = (S + kBN - 1) / kBN;
  load_tile(0);
  store_tile();
  __syncthreads();

  const int prow0 = perm_row(l32);
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * kBN;
    if (kt + 1 < nkt) load_tile(k0 + kBN);

    // S^T (keys x queries) for two 32-key sub-tiles.
    f32x16_t acc_s[2];
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      acc_s[sg] = f32x16_t{};
      const unsigned char* kp = ks + (32 * sg + prow0) * kKPitch + 16 * hi;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kp + 32 * k);
        acc_s[sg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[k], acc_s[sg], 0, 0, 0);
      }
    }

    // Mask keys past the end (only the last tile can have them).
    if (k0 + kBN > S) {
#pragma unroll
      for (int sg = 0; sg < 2; ++sg)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int g = i >> 2, r = i & 3;
          const int key = k0 + 32 * sg + 16 * (g >> 1) + 8 * hi + 4 * (g & 1) + r;
          if (key >= S) acc_s[sg][i] = -INFINITY;
        }
    }

    // Online softmax (base-2, scale folded in).
    float mx = acc_s[0][0];
#pragma unroll
    for (int sg = 0; sg < 2; ++sg)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc_s[sg][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8_t pf[4];
#pragma unroll
    for (int sg = 0; sg < 2; ++sg)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8_t v;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(acc_s[sg][8 * half + j], scale_log2, -m_new));
          psum += p;
          v[j] = (__bf16)p;
        }
        pf[2 * sg + half] = v;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[dt][i] *= alpha;

    // O^T (channels x queries) += V^T P^T over the 64 keys of the tile.
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const unsigned char* vp = vs + (32 * dt + l32) * kVPitch + 16 * hi;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vp + 32 * k);
        acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[k], acc_o[dt], 0, 0, 0);
      }
    }

    __syncthreads();
    if (kt + 1 < nkt) {
      store_tile();
      __syncthreads();
    }
  }

  // Epilogue: O = O^T / l, bf16; lane holds 4 consecutive channels per (dt, g).
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qrow < S) {
    const float inv = 1.0f / l_tot;
    uint16_t* op = out + ((int64_t)b * S + qrow) * D + h * kD + 4 * hi;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack_bf16x2(acc_o[dt][4 * g + 0] * inv, acc_o[dt][4 * g + 1] * inv);
        w.y = pack_bf16x2(acc_o[dt][4 * g + 2] * inv, acc_o[dt][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(op + 32 * dt + 8 * g) = w;
      }
    if (lse && hi == 0) lse[(int64_t)bh * S + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
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
