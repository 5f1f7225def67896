// QKV projection of the DiT self-attention block: packed [Q|K|V] = x W^T + b,
// the linear layer whose output the norm + RoPE and attention steps read in
// place ("Optimize Wan2.2 Dataflow", change 1: one fused QKV allocation; the
// qkv_cte kernel of "Optimizing High-Quality Offline Video Generation", NKI
// kernels). bf16 operands, fp32 accumulation on gfx950 16x16x32 MFMA, bf16 out.
//
// Design (gfx950):
//   * workgroup = 8 waves, output tile 256 tokens x 256 features, K in steps of
//     64 through two LDS stages of 64 KB, filled straight from global memory
//     by buffer_load_dwordx4 ... lds (no staging registers). The buffer form
//     takes one descriptor per operand tile and a 32-bit offset per lane, and
//     rows past the end of the matrix read as zeros. (The global_load_lds form
//     of the same copy measured slower: its requests queue behind the LDS
//     commands of the fragment reads.)
//   * the tile is computed transposed, C^T = W X^T (A = 16 features x 32
//     channels of W, B = 32 channels x 16 tokens of x), so each lane ends with 4
//     consecutive features of one token;
//   * waves are 2 (features) x 4 (tokens), each owning 128 x 64 outputs = 32
//     MFMA tiles; per 32-channel half step a wave reads 8 W and 4 x fragments
//     (16 B per lane) and issues 32 MFMAs;
//   * the copies of the next step are spread over the first half's MFMAs, one
//     per two MFMAs: issued in one burst, the copies of all waves fill the
//     texture unit's queues and the in-order wave stalls with its MFMAs behind
//     them (+5%);
//   * 128-byte LDS rows (64 channels) with the 16-byte chunk XOR-swizzled by
//     the row (p_swz): conflict-free fragment reads;
//   * epilogue through LDS: the tile is written to LDS and stored as whole
//     256-byte row segments (8-byte stores straight from the MFMA layout touch
//     16 rows per store and stall the texture unit's write path: +6%);
//   * workgroups are numbered XCD-major and then in groups of 8 token tiles
//     sweeping the feature tiles, so the ~32 workgroups an XCD runs at once
//     share 8 x tiles and 4 W tiles in its L2 (groups of 16 or 32 token tiles
//     measured 10% and 20% slower).
#include "common.hpp"
#include "kernels.hpp"

namespace wan {

namespace {

constexpr int kPM = 256, kPN = 256, kPK = 64;  // tile: tokens, features, channels per step
constexpr int kPWaves = 8, kPThreads = 64 * kPWaves;
constexpr int kPRow = kPK * 2;                 // bytes per LDS row
constexpr int kPTile = kPM * kPRow;            // 32 KB per operand tile
constexpr int kPStage = 2 * kPTile;            // W tile + x tile
constexpr int kPGroup = 8;                     // token tiles per ordering group
constexpr int kPBlk = kPTile / 1024 / kPWaves;  // 1 KB blocks (8 rows) per wave per operand tile (4)
constexpr int kPLoads = 2 * kPBlk;             // copies per wave per step (8)
static_assert(kPM == kPN, "one staging layout serves both operands");
static_assert(kPWaves * 64 * 256 <= 2 * kPStage, "the epilogue needs 16 KB per wave");
constexpr int kWaitVm0 = 0x0f70;               // s_waitcnt vmcnt(0), other counters unconstrained

// XOR swizzle of the 16-byte chunk of a 128-byte row: r1 | r2 << 1 | (r0 ^ r3)
// << 2. Each half-wave's 32 fragment reads land on 32 distinct 16-byte slots
// of a 512-byte window (and every 8 or 16 consecutive lanes on distinct slots
// of 128 or 256 bytes), which the gfx950 LDS serves without bank conflicts.
__device__ __forceinline__ int p_swz(int r) { return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r ^ (r >> 3)) & 1) << 2); }

__device__ __forceinline__ int p_xcd_remap(int bid, int nb) {
  const int xcd = bid & 7, j = bid >> 3;
  const int q = nb >> 3, r = nb & 7;
  return xcd * q + (xcd < r ? xcd : r) + j;
}

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__global__ void __launch_bounds__(kPThreads, 1)
qkv_proj_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias,
                uint16_t* __restrict__ out, int M, int N, int K, int ntm, int ntn) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kPStage];

  // Tile order: XCD-major, then groups of kPGroup token tiles x all feature tiles.
  const int lid = p_xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = kPGroup * ntn;
  const int group = lid / per_group;
  const int first_tm = group * kPGroup;
  const int gm = min(ntm - first_tm, kPGroup);
  const int rr = lid - group * per_group;
  const int tm = first_tm + rr % gm, tn = rr / gm;
  const int m0 = tm * kPM, n0 = tn * kPN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;  // 2 x 4 waves: features 128 wn.., tokens 64 wm..

  // Staging: each wave fills kPBlk 1 KB blocks (8 rows of 128 B) of the W tile
  // and of the x tile; lane l of a block takes physical row 8 blk + l/8,
  // physical chunk l%8, i.e. logical chunk (l%8) ^ swz(row). One buffer
  // descriptor per operand tile, sized to the rows that exist: rows past N or
  // M read as zeros (and are never stored).
  const uint32_t wbytes = (uint32_t)(min(N - n0, kPN) * K * 2), xbytes = (uint32_t)(min(M - m0, kPM) * K * 2);
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(w + (int64_t)n0 * K), (short)0, (int)wbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + (int64_t)m0 * K), (short)0, (int)xbytes, 0x00020000);
  uint32_t goff[kPBlk];
#pragma unroll
  for (int j = 0; j < kPBlk; ++j) {
    const int r = 8 * (kPBlk * wave + j) + (lane >> 3);
    goff[j] = (uint32_t)(r * K * 2 + 16 * ((lane & 7) ^ p_swz(r)));
  }
  auto issue = [&](int kt, int stage) {
    unsigned char* dst = smem + stage * kPStage + kPBlk * wave * 1024;
#pragma unroll
    for (int j = 0; j < kPBlk; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr_t)(dst + j * 1024), 16, goff[j], kt * kPRow, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_ptr_t)(dst + kPTile + j * 1024), 16, goff[j], kt * kPRow, 0, 0);
    }
  };

  // Fragment reads: lane (l16, grp) reads row 16 t + l16 at logical chunk 4 s +
  // grp; the swizzle depends on the row only through l16, so the per-lane byte
  // offset of a read is fixed for each 32-channel half s.
  int roff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) roff[s] = l16 * kPRow + 16 * ((4 * s + grp) ^ p_swz(l16));

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{};

  // Step kt lives in stage kt & 1. Iteration kt copies step kt + 1 (past the
  // last step: the last step again, into the stage nobody reads any more), so
  // the loop body is one basic block the schedule below can arrange.
  const int nk = K / kPK;
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    // This wave's copies of step kt have landed; past the barrier, every
    // wave's, and every wave has finished reading step kt - 1, whose stage is
    // refilled below. A bare barrier: the fence of __syncthreads() adds nothing
    // the explicit wait does not.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    asm volatile("s_barrier" ::: "memory");
    const unsigned char* st = smem + (kt & 1) * kPStage;
    bf16x8_t a[2][8], b[2][4];
    auto read = [&](int s) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        a[s][i] = *reinterpret_cast<const bf16x8_t*>(st + (128 * wn + 16 * i) * kPRow + roff[s]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[s][j] = *reinterpret_cast<const bf16x8_t*>(st + kPTile + (64 * wm + 16 * j) * kPRow + roff[s]);
    };
    auto mfmas = [&](int s) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a[s][i], b[s][j], acc[i][j]);
    };
    // The copies follow the first half's fragment reads in program order (the
    // compiler cannot tell the stages apart and keeps LDS reads and LDS-writing
    // copies in order) and interleave with its MFMAs; the second half's reads
    // follow the copies.
    read(0);
    issue(min(kt + 1, nk - 1), (kt + 1) & 1);
    mfmas(0);
    read(1);
    mfmas(1);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // 12 fragment reads
#pragma unroll
    for (int q = 0; q < kPLoads; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMAs
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // 1 copy
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 64 - 2 * kPLoads, 0);
    __builtin_amdgcn_sched_barrier(0);  // nothing moves past the next iteration's wait
  }
  // The last copies (a reload) land, and every wave leaves the stages, before
  // the epilogue reuses the LDS.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  // Epilogue through LDS (free after the last barrier): each wave writes its
  // 64 tokens x 128 features, bias added and rounded to bf16, into its own 16 KB
  // (one 256-byte row per token), then stores whole 16-byte pieces of rows, so
  // a store instruction covers 4 tokens x 256 contiguous bytes instead of 16
  // tokens x 32 bytes. Lane (l16, grp) of tile (i, j) holds features
  // 16 i + 4 grp .. +3 of token 16 j + l16. The 8-byte unit u of a row is
  // stored at u ^ f(row), f(row) = 2 ((row >> 1) & 15): even, so 16-byte
  // pieces stay whole, and the writes of a half-wave (16 rows x 2 units) and
  // the reads (2 rows x 256 bytes) both cover distinct banks.
  unsigned char* ep = smem + wave * (64 * 256);
  const int nb = n0 + 128 * wn;  // first feature of this wave's tile
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    const int n = nb + 16 * i + 4 * grp;
    if (bias && n < N) {
      const uint2 bw = *reinterpret_cast<const uint2*>(bias + n);
      bv[0] = bf16_lo(bw.x);
      bv[1] = bf16_hi(bw.x);
      bv[2] = bf16_lo(bw.y);
      bv[3] = bf16_hi(bw.y);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * j + l16;
      const int u = (4 * i + grp) ^ (((row >> 1) & 15) << 1);
      uint2 o;
      o.x = pack_bf16x2(acc[i][j][0] + bv[0], acc[i][j][1] + bv[1]);
      o.y = pack_bf16x2(acc[i][j][2] + bv[2], acc[i][j][3] + bv[3]);
      *reinterpret_cast<uint2*>(ep + row * 256 + u * 8) = o;
    }
  }
  // Each wave reads back only what it wrote: the compiler's LDS waits order it.
  const int k = lane & 15;  // 16-byte piece: features nb + 8 k .. +7
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int row = 4 * t + (lane >> 4);
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ep + row * 256 + ((2 * k) ^ (((row >> 1) & 15) << 1)) * 8);
    const int m = m0 + 64 * wm + row, n = nb + 8 * k;
    if (m < M && n < N) *reinterpret_cast<u32x4_t*>(out + (int64_t)m * N + n) = v;
  }
}

}  // namespace

hipError_t launch_qkv_proj(const void* x, const void* w, const void* bias, void* out, int64_t M, int N, int K,
                           hipStream_t stream) {
  const int64_t ntm = (M + kPM - 1) / kPM;
  const int ntn = (N + kPN - 1) / kPN;
  const int64_t nblocks = ntm * ntn;
  if (nblocks > INT32_MAX || ntm > INT32_MAX / kPGroup / ntn) return hipErrorInvalidConfiguration;
  // A buffer descriptor covers one operand tile: 256 rows of K bf16 must stay
  // within its 32-bit byte range.
  if ((int64_t)kPM * K * 2 > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(qkv_proj_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(kPThreads), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                     static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(out), static_cast<int>(M), N, K,
                     static_cast<int>(ntm), ntn);
  return hipGetLastError();
}

}  // namespace wan
