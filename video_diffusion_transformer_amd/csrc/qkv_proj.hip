// QKV projection of the DiT self-attention block: packed [Q|K|V] = x W^T + b,
// the linear layer whose output the norm + RoPE and attention steps read in
// place ("Optimize Wan2.2 Dataflow", change 1: one fused QKV allocation; the
// qkv_cte kernel of "Optimizing High-Quality Offline Video Generation", NKI
// kernels). bf16 operands, fp32 accumulation on gfx950 16x16x32 MFMA, bf16 out.
//
// Design (gfx950):
//   * workgroup = 8 waves, output tile 256 tokens x 256 features, K in steps of
//     64 channels; the x tiles (32 KB per step) go through three LDS stages and
//     are copied two steps ahead, the W tiles through two, one step ahead (all
//     160 KB of the CU's LDS). The stages are filled straight from global
//     memory by buffer_load_dwordx4 ... lds (no staging registers), one buffer
//     descriptor per operand tile and a 32-bit offset per lane; rows past the
//     end of the matrix read as zeros. The copies are inline asm, waited for
//     only by the loop's explicit vmcnt waits (the compiler's own tracking of
//     them added waits that cancelled the deeper prefetch). (The
//     global_load_lds form of the copy measured slower: its requests queue
//     behind the LDS commands of the fragment reads.)
//   * the tile is computed transposed, C^T = W X^T (A = 16 features x 32
//     channels of W, B = 32 channels x 16 tokens of x), so each lane ends with 4
//     consecutive features of one token;
//   * waves are 2 (features) x 4 (tokens), each owning 128 x 64 outputs = 32
//     MFMA tiles; per 32-channel half step a wave reads 8 W and 4 x fragments
//     (16 B per lane) and issues 32 MFMAs;
//   * the copies (W of the next step, x of the one after) are spread over the
//     first half's MFMAs, one per four: issued in one burst, the copies of all
//     waves fill the texture unit's queues and the in-order wave stalls with
//     its MFMAs behind them;
//   * 128-byte LDS rows (64 channels) with the 16-byte chunk XOR-swizzled by
//     the row (p_swz): conflict-free fragment reads;
//   * epilogue through LDS: the tile is written to LDS and stored as whole
//     256-byte row segments (8-byte stores straight from the MFMA layout touch
//     16 rows per store and stall the texture unit's write path: +6%);
//   * a persistent grid (one workgroup per CU slot) takes output tiles from
//     per-XCD queues (next_tile_xcd) where the feature tiles form 8 bands,
//     else, and always in the fused kernel, from one atomic counter in
//     token-block order (token block, then feature tile):
//     the ~4 token blocks in flight share their x tiles in L2 while W (157 MB
//     at D = 5120) streams from the 256 MB last-level cache. Measured against
//     one workgroup per tile in an XCD-grouped order (interleaved calls, both
//     with two stages per operand): 480p (10.3 TFLOP) 7.90 against 7.80 ms,
//     720p (23.8 TFLOP) 18.2 against 18.9 ms; the fused norm + RoPE epilogue
//     below needs the persistent grid.
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace wan {

namespace {

constexpr int kPM = 256, kPN = 256, kPK = 64;  // tile: tokens, features, channels per step
static_assert(kPM == kFusedTileTokens && kPN == kFusedTileFeatures, "workspace layout follows the tile");
constexpr int kPWaves = 8, kPThreads = 64 * kPWaves;
constexpr int kPRow = kPK * 2;                 // bytes per LDS row
constexpr int kPTile = kPM * kPRow;            // 32 KB per operand tile
constexpr int kXStages = 3, kWStages = 2;      // x tiles are copied two steps ahead, W tiles one
constexpr int kWOff = kXStages * kPTile;       // the W stages follow the x stages
constexpr int kSmem = (kXStages + kWStages) * kPTile;  // 160 KB: all of a CU's LDS
constexpr int kPBlk = kPTile / 1024 / kPWaves;  // 1 KB blocks (8 rows) per wave per operand tile (4)
constexpr int kPLoads = 2 * kPBlk;             // copies per wave per step (8)
// Between two tiles the stages are free: the epilogue's LDS tile takes the
// first 128 KB, the fused epilogue's exchange area and the tile index sit in the
// last W stage (first written by step 0's copies, after every wave has read the
// tile index).
constexpr int kAuxOff = 4 * kPTile;
constexpr int kTileShOff = kSmem - 16;
static_assert(kPM == kPN, "one staging layout serves both operands");
static_assert(kPWaves * 64 * 256 <= kAuxOff, "the epilogue needs 16 KB per wave below the exchange area");
static_assert(kAuxOff + (kPWaves * 64 + 1) * 4 <= kTileShOff, "exchange area and tile index apart");
static_assert(kWOff + (kWStages - 1) * kPTile <= kAuxOff, "exchange area and tile index in the last W stage");
constexpr int kWaitVm0 = 0x0f70;               // s_waitcnt vmcnt(0), other counters unconstrained

// XOR swizzle of the 16-byte chunk of a 128-byte row: r1 | r2 << 1 | (r0 ^ r3)
// << 2. Each half-wave's 32 fragment reads land on 32 distinct 16-byte slots
// of a 512-byte window (and every 8 or 16 consecutive lanes on distinct slots
// of 128 or 256 bytes), which the gfx950 LDS serves without bank conflicts.
__device__ __forceinline__ int p_swz(int r) { return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r ^ (r >> 3)) & 1) << 2); }

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Buffer descriptor of `bytes` bytes from base (raw buffer, no stride): reads
// past the end return zeros. Wave-uniform.
__device__ __forceinline__ u32x4_t buf_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4_t d;
  d[0] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  d[1] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xffffu);
  d[2] = __builtin_amdgcn_readfirstlane(bytes);
  d[3] = 0x00020000u;
  return d;
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const unsigned char*)p));
}

// One direct global -> LDS copy, 16 bytes per lane (lane l lands at lds + 16 l).
// Written as inline asm so that the compiler does not track it: for its own
// form of this copy the compiler cannot tell one stage from another and waits
// for every copy in flight before the next LDS read, which undoes a prefetch
// distance of two steps (measured at 480p: the three-stage loop 12% slower
// than two stages with the builtin, 3.5% faster with this, 5% with the copies
// spread as below). The only waits for these copies are the explicit vmcnt
// waits of the K loop.
__device__ __forceinline__ void dma16(const u32x4_t& desc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(desc), "s"(soff), "{m0}"(lds));
}

// The 256 x 256 tile (m0, n0) of x W^T (no bias) into acc: each lane ends with
// 4 consecutive features of one token per MFMA tile (i, j) -- features
// n0 + 128 wn + 16 i + 4 grp .. +3 of token m0 + 64 wm + 16 j + l16. On return
// every wave has left the LDS stages (the caller may reuse the LDS).
__device__ __forceinline__ void gemm_tile(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int M, int N,
                                          int K, int m0, int n0, unsigned char* __restrict__ smem, int wave, int lane,
                                          f32x4_t (&acc)[8][4]) {
  const int l16 = lane & 15, grp = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;  // 2 x 4 waves: features 128 wn.., tokens 64 wm..

  // Staging: each wave fills kPBlk 1 KB blocks (8 rows of 128 B) of the W tile
  // and of the x tile; lane l of a block takes physical row 8 blk + l/8,
  // physical chunk l%8, i.e. logical chunk (l%8) ^ swz(row). One buffer
  // descriptor per operand tile, sized to the rows that exist: rows past N or
  // M read as zeros (and are never stored).
  const uint32_t wbytes = (uint32_t)(min(N - n0, kPN) * K * 2), xbytes = (uint32_t)(min(M - m0, kPM) * K * 2);
  const u32x4_t wrs = buf_desc(w + (int64_t)n0 * K, wbytes), xrs = buf_desc(x + (int64_t)m0 * K, xbytes);
  uint32_t goff[kPBlk];
#pragma unroll
  for (int j = 0; j < kPBlk; ++j) {
    const int r = 8 * (kPBlk * wave + j) + (lane >> 3);
    goff[j] = (uint32_t)(r * K * 2 + 16 * ((lane & 7) ^ p_swz(r)));
  }
  const int nk = K / kPK;
  const uint32_t lds0 = lds_addr(smem);
  // Block j of step kt (clamped to the last step: past it, the copies reload
  // the last step into a stage nobody reads any more) into the x or W stage.
  auto copy_x = [&](int j, int kt, int stage) {
    dma16(xrs, goff[j], (uint32_t)(min(kt, nk - 1) * kPRow),
          __builtin_amdgcn_readfirstlane(lds0 + stage * kPTile + (kPBlk * wave + j) * 1024));
  };
  auto copy_w = [&](int j, int kt, int stage) {
    dma16(wrs, goff[j], (uint32_t)(min(kt, nk - 1) * kPRow),
          __builtin_amdgcn_readfirstlane(lds0 + kWOff + stage * kPTile + (kPBlk * wave + j) * 1024));
  };

  // Fragment reads: lane (l16, grp) reads row 16 t + l16 at logical chunk 4 s +
  // grp; the swizzle depends on the row only through l16, so the per-lane byte
  // offset of a read is fixed for each 32-channel half s.
  int roff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) roff[s] = l16 * kPRow + 16 * ((4 * s + grp) ^ p_swz(l16));

#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{};

  // Step kt reads x from stage kt % 3 and W from stage kt % 2, and copies x of
  // step kt + 2 and W of step kt + 1 into the stages step kt - 1 read. (x two
  // steps ahead and W one measured 3.5% faster than one step for both, W two
  // and x one 2.8%; two steps for both would need 192 KB.) Each wave copies W
  // first: loads complete in order, so at the top of step kt everything but its
  // last kPBlk copies (x of step kt + 1) has landed -- x and W of step kt.
#pragma unroll
  for (int j = 0; j < kPBlk; ++j) copy_w(j, 0, 0);
#pragma unroll
  for (int j = 0; j < kPBlk; ++j) copy_x(j, 0, 0);
#pragma unroll
  for (int j = 0; j < kPBlk; ++j) copy_x(j, 1, 1);

  auto step = [&](int kt, auto u_c) {
    constexpr int u = decltype(u_c)::value;  // kt % 6: the stages are constants
    constexpr int xc = u % kXStages, xn = (u + 2) % kXStages, wc = u % kWStages, wn1 = (u + 1) % kWStages;
    // This wave's copies of step kt have landed; past the barrier, every
    // wave's, and every wave has finished step kt - 1, whose stages are
    // refilled below. A bare barrier: the fence of __syncthreads() adds nothing
    // the explicit wait does not.
    __builtin_amdgcn_s_waitcnt(kWaitVm0 | kPBlk);
    asm volatile("s_barrier" ::: "memory");
    const unsigned char* stx = smem + xc * kPTile;
    const unsigned char* stw = smem + kWOff + wc * kPTile;
    bf16x8_t a[2][8], b[2][4];
    auto read = [&](int s) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        a[s][i] = *reinterpret_cast<const bf16x8_t*>(stw + (128 * wn + 16 * i) * kPRow + roff[s]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[s][j] = *reinterpret_cast<const bf16x8_t*>(stx + (64 * wm + 16 * j) * kPRow + roff[s]);
    };
    // Order, pinned by scheduling barriers: the first half's fragment reads,
    // its 32 MFMAs with one copy after every four (W, then x; measured 2-4%
    // faster than one copy per two, three, five or eight MFMAs), the second
    // half's reads after the first half's 16th MFMA, then the second half's
    // 32 MFMAs.
    read(0);
#pragma unroll
    for (int m = 0; m < 64; ++m) {
      const int sh = m >> 5, i = (m & 31) >> 2, j = m & 3;
      acc[i][j] = mfma16(a[sh][i], b[sh][j], acc[i][j]);
      if (m == 15) {
        __builtin_amdgcn_sched_barrier(0);
        read(1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (m % 4 == 3 && m < 4 * kPLoads) {
        const int q = m / 4;
        __builtin_amdgcn_sched_barrier(0);
        if (q < kPBlk)
          copy_w(q, kt + 1, wn1);
        else
          copy_x(q - kPBlk, kt + 2, xn);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // nothing moves past the next step's wait
  };
  for (int kt = 0; kt < nk; kt += 6) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>{});
    if (kt + 2 < nk) step(kt + 2, std::integral_constant<int, 2>{});
    if (kt + 3 < nk) step(kt + 3, std::integral_constant<int, 3>{});
    if (kt + 4 < nk) step(kt + 4, std::integral_constant<int, 4>{});
    if (kt + 5 < nk) step(kt + 5, std::integral_constant<int, 5>{});
  }
  // Every copy (the last ones reload the last step) lands, and every wave
  // leaves the stages, before the epilogue reuses the LDS.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
}

// Epilogue through LDS (free after gemm_tile): each wave writes its 64 tokens x
// 128 features, as the packed bf16 pairs pk(i, j) returns for MFMA tile (i, j),
// into its own 16 KB (one 256-byte row per token), then stores whole 16-byte
// pieces of rows, so a store instruction covers 4 tokens x 256 contiguous bytes
// instead of 16 tokens x 32 bytes. The 8-byte unit u of a row is stored at
// u ^ f(row), f(row) = 2 ((row >> 1) & 15): even, so 16-byte pieces stay whole,
// and the writes of a half-wave (16 rows x 2 units) and the reads (2 rows x 256
// bytes) both cover distinct banks.
//
// The lane index passes through an empty asm statement so that the LDS
// addresses derived from it are computed here and not hoisted out of a
// persistent kernel's tile loop: hoisted, 16 of them would stay live across the
// GEMM, spill, and every store would first wait (vmcnt) for its reload -- and
// with it for all earlier stores.
template <class Pack>
__device__ __forceinline__ void store_tile(uint16_t* __restrict__ out, int M, int N, int m0, int n0,
                                           unsigned char* __restrict__ smem, int wave, int lane_in, Pack pk) {
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const int l16 = lane & 15, grp = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;
  unsigned char* ep = smem + wave * (64 * 256);
  const int nb = n0 + 128 * wn;  // first feature of this wave's tile
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * j + l16;
      const int u = (4 * i + grp) ^ (((row >> 1) & 15) << 1);
      *reinterpret_cast<uint2*>(ep + row * 256 + u * 8) = pk(i, j);
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

// Bias of the 4 features n .. n+3 (zero without bias or past N).
__device__ __forceinline__ void load_bias4(const uint16_t* __restrict__ bias, int n, int N, float (&bv)[4]) {
  bv[0] = bv[1] = bv[2] = bv[3] = 0.f;
  if (bias && n < N) {
    const uint2 bw = *reinterpret_cast<const uint2*>(bias + n);
    bv[0] = bf16_lo(bw.x);
    bv[1] = bf16_hi(bw.x);
    bv[2] = bf16_lo(bw.y);
    bv[3] = bf16_hi(bw.y);
  }
}

// ---------------------------------------------------------------------------
// The projection with the Q/K RMSNorm and 3-D RoPE in its epilogue (the qkv_cte
// kernel of "Optimizing High-Quality Offline Video Generation", NKI kernels: QKV
// projection, distributed QK RMSNorm and RoPE in one kernel). A token's norm
// spans all D channels of its Q (and of its K): `heads` wave columns of 128
// features each, spread over heads / 2 output tiles. As the pages distribute
// the norm over the tensor-parallel ranks that hold the head shards, the tiles
// of one token block exchange per-token partial sums of squares: each tile
// rounds its outputs to bf16 (the projection's own rounding point), publishes
// every token's sum of squares over each of its 128-feature wave columns, waits
// until all columns of its part (Q, or K) of its token block have published,
// and then normalises, rotates and rounds its tile in registers. The
// unnormalised Q and K never reach memory.
//
// Scheduling: a persistent grid (one workgroup per CU slot) takes tiles from an
// atomic counter in token-block order (token block, then feature tile: the Q
// tiles of a block, then its K tiles, then V). A workgroup publishes before it
// waits and waits only for the tiles of its own (token block, part) unit.
// Taking the units in order, waiting workgroups hold tiles of the lowest
// unfinished unit only (every tile of a lower unit has been taken and
// published), so fewer wait than the unit has tiles (some tile of it is still
// untaken): at most about heads / 2. With room on the device for `heads`
// workgroups, some workgroup is always free to take the missing tiles, and
// every wait ends. A bounded spin guards the rest (e.g. the device held by
// other work): past the limit the wave sets the error word of the workspace
// and stores NaN bits for its Q and K outputs. Counting Q and K apart halves
// the span of tiles a wait covers (with one count per token block, publishing
// and waiting took 6.9% of the kernel at 480p; counted apart, 0.05 ms less).
// ---------------------------------------------------------------------------
constexpr int kPairsT = 22, kPairsH = 21, kPairsW = 21;  // rotary pairs per axis (44/42/42 channels)
constexpr unsigned kSpinLimit = 1u << 20;                // polls of a token block's arrival count (about 1 s)
constexpr unsigned kReadLimit = 1u << 16;                // re-reads of partial sums whose marker is not yet visible

struct NormRopeArgs {
  const uint16_t* gq;  // RMSNorm weights of Q and of K, [D] bf16
  const uint16_t* gk;
  const float2* tab;   // rotary (cos, sin): frame [T][22], row [H][21], column [W][21]
  int S, H, W, offH, offW, heads;
  float inv_d, eps;
  unsigned spin_limit, read_limit;  // bounds of the two waits (kSpinLimit, kReadLimit)
  unsigned* ctl;       // [0] tile counter, [1] error word (a wait hit the spin limit); plain: [0..7] XCD queues
  int xcd_queues;      // plain projection: take tiles from the per-XCD queues (next_tile_xcd)
  unsigned* arrive;    // [ntm][2] published Q and K wave columns per token block
  uint64_t* partial;   // [2 heads][M] (1 << 32 | sum-of-squares bits) per wave column (Q heads, then K heads) and token
};

// Per-XCD tile queues of the plain projection, used when the feature tiles
// form 8 bands of 8 (the last band may be partial; 57..64 feature tiles, as at
// D = 5120) and the grid has at least 8 workgroups. Workgroup i runs on XCD
// i % 8 (dispatch is round-robin over the XCDs) and takes tiles from queue
// i % 8. Tiles come in blocks of 4 token tiles x 8 feature tiles (one band);
// for block row bm, queue k takes band (k + bm) % 8, so the 8 queues share
// every block row equally and, at any time, the ~32 tiles in flight on an XCD
// share 4 x tiles and 8 W tiles in its L2: at 480p the traffic beyond L2
// drops from ~44 to ~16 GB per call and the call takes 1.2% less time than
// with one queue in token-block order. (Band k for queue k, unbalanced since
// the last band is half as wide, was 1% slower.) Every queue is drained by
// its own workgroups; each tile is taken once: queue (tn / 8 - tm / 4) % 8 at
// index 32 (tm / 4) + (tm % 4) + 4 (tn % 8).
__device__ __forceinline__ int next_tile_xcd(unsigned* ctl, int ntm, int ntn, int ntiles) {
  const int k = blockIdx.x & 7;
  const int nbm = (ntm + 3) / 4;
  for (;;) {
    const unsigned idx = atomicAdd(ctl + k, 1u);
    const int bm = static_cast<int>(idx >> 5);
    if (bm >= nbm) return ntiles;
    const int q = static_cast<int>(idx & 31u);
    const int tm = 4 * bm + (q & 3), tn = 8 * ((k + bm) & 7) + (q >> 2);
    if (tm < ntm && tn < ntn) return tm * ntn + tn;  // else a ragged edge: take the next
  }
}

// Zero n 16-byte words (grid-stride).
__global__ void __launch_bounds__(256) zero16_kernel(u32x4_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = u32x4_t{0u, 0u, 0u, 0u};
}

// Norm = false: the plain projection (bias, bf16 rounding, store); only
// na.ctl (the tile counter) is used.
template <bool Norm>
__global__ void __launch_bounds__(kPThreads, 1)
qkv_proj_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias,
                uint16_t* __restrict__ out, int M, int N, int K, int ntm, int ntn, NormRopeArgs na) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmem];
  int& tile_sh = *reinterpret_cast<int*>(smem + kTileShOff);  // the tile taken
  // Fused epilogue only: sums of squares passed between the two waves of a
  // row, and whether the arrival wait timed out.
  float(&xsum)[kPWaves][64] = *reinterpret_cast<float(*)[kPWaves][64]>(smem + kAuxOff);
  int& late_sh = *reinterpret_cast<int*>(smem + kAuxOff + sizeof(xsum));

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;
  const int D = na.heads * 128;
  const int ntiles = ntm * ntn;

  for (;;) {
    // The barrier at the end of the previous tile orders this write after every read of tile_sh.
    if (tid == 0)
      tile_sh = (!Norm && na.xcd_queues) ? next_tile_xcd(na.ctl, ntm, ntn, ntiles)
                                         : static_cast<int>(atomicAdd(na.ctl, 1u));
    __syncthreads();
    const int t = tile_sh;
    if (t >= ntiles) break;
    const int tm = t / ntn, tn = t - tm * ntn;
    const int m0 = tm * kPM, n0 = tn * kPN;

    f32x4_t acc[8][4];
    gemm_tile(x, w, M, N, K, m0, n0, smem, wave, lane, acc);

    // y = bf16(x W^T + b): the values the packed buffer of the plain projection holds.
    const int nb = n0 + 128 * wn;  // this wave's first feature (a multiple of 128: inside one of Q, K, V)
    const int part = nb / D;       // 0 Q, 1 K, 2 V
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float bv[4];
      load_bias4(bias, nb + 16 * i + 4 * grp, N, bv);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = static_cast<float>(static_cast<__bf16>(acc[i][j][e] + bv[e]));
    }

    // The tile's Q and its K wave columns (0, 1 or 2 of each); whether this wave holds one.
    int cols_q = 0, cols_k = 0;
    if (Norm) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int f = n0 + 128 * h;
        cols_q += f < N && f / D == 0;
        cols_k += f < N && f / D == 1;
      }
    }
    const int qk_cols = cols_q + cols_k;
    const bool qk = Norm && nb < N && part < 2;
    // Publish, then wait. The partial sums travel as 64-bit words (value bits,
    // 1 above them) written and read with device-scope atomic accesses: a
    // reader that finds the marker has the value of the same word, so the
    // exchange needs no device-wide fence (those write back and invalidate the
    // XCD's L2, which the GEMM operands live in). The arrival count only tells
    // the workgroup when to start reading; a word not yet visible is re-read.
    // Layout [column][token]: one wave's 64 tokens of a column are 512
    // contiguous bytes, read by one load instruction.
    bool bad = false;  // this wave's wait timed out: its Q/K outputs are stored as NaN bits
    float ssum = 0.f;  // reader: sum of squares over all Q (or K) channels of token m0 + 64 wm + lane
    if (qk_cols > 0) {
      if (qk) {
        // Sum of squares of each of the wave's 64 tokens over its 128 features.
        const int col = part * na.heads + (nb - part * D) / 128;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float ss = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += acc[i][j][e] * acc[i][j][e];
          ss += __shfl_xor(ss, 16, 64);
          ss += __shfl_xor(ss, 32, 64);
          const int m = m0 + 64 * wm + 16 * j + l16;
          if (grp == 0 && m < M)
            __hip_atomic_store(na.partial + (int64_t)col * M + m, (uint64_t(1) << 32) | __float_as_uint(ss),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // The stores have completed before the arrival below is counted, so a
        // reader that sees the count complete finds the words (re-reads stay rare).
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      }
      __syncthreads();
      if (tid == 0) {
        // Q and K of a token block are counted apart: a tile waits only for
        // the columns of the part(s) it holds.
        int late = 0;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int cols = p == 0 ? cols_q : cols_k;
          if (cols == 0) continue;
          unsigned* cnt = na.arrive + 2 * tm + p;
          atomicAdd(cnt, static_cast<unsigned>(cols));
          unsigned spins = 0;
          while (!late && __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                              static_cast<unsigned>(na.heads)) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins > na.spin_limit) late = 1;
          }
        }
        late_sh = late;
      }
      __syncthreads();
      bad = qk && late_sh != 0;

      // Both wave columns of the tile in Q (or both in K): the two waves of a
      // row read alternate columns and add each other's sums (through LDS).
      const bool split = qk_cols == 2 && n0 / D == (n0 + 128) / D;
      if (qk) {
        const int mrow = min(m0 + 64 * wm + lane, M - 1);  // rows past M: any row of the block (not stored)
        const uint64_t* pr = na.partial + (int64_t)(part * na.heads) * M + mrow;
        const int c0 = split ? wn : 0, cstep = split ? 2 : 1;
        for (unsigned tries = 0; !bad; ++tries) {
          bool ready = true;
          float sc = 0.f;
          for (int c = c0; c < na.heads; c += cstep) {
            const uint64_t v = __hip_atomic_load(pr + (int64_t)c * M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ready = ready && (v >> 32) != 0;
            sc += __uint_as_float(static_cast<uint32_t>(v));
          }
          ssum = sc;
          if (__all(ready)) break;
          if (tries > na.read_limit) bad = true;
          __builtin_amdgcn_s_sleep(2);
        }
        if (bad && lane == 0) atomicOr(na.ctl + 1, 1u);
      }
      if (split) {
        xsum[wave][lane] = ssum;
        __syncthreads();
        ssum += xsum[wave ^ 1][lane];  // same sum in both waves: fp32 addition commutes
      }
    }

    if (qk) {
      const uint16_t* g = part == 0 ? na.gq : na.gk;
      const int cbase = nb - part * D;  // channel of this wave's first feature within Q or K
      float r[4];                       // (mean square + eps)^-1/2 of the wave's tokens 16 j + l16
      int tb[4][3];                     // their rotary table rows (frame, row, column axis), minus the axis' first pair
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float ss = __shfl(ssum, 16 * j + l16, 64);
        r[j] = rsqrtf(ss * na.inv_d + na.eps);
        const int s = min(m0 + 64 * wm + 16 * j + l16, M - 1) % na.S;
        tb[j][0] = (s / (na.H * na.W)) * kPairsT;
        tb[j][1] = na.offH + ((s / na.W) % na.H) * kPairsH - kPairsT;
        tb[j][2] = na.offW + (s % na.W) * kPairsW - (kPairsT + kPairsH);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = cbase + 16 * i + 4 * grp;  // channels c .. c+3 of Q (or K): rotary pairs p0, p0 + 1
        const uint2 gw = *reinterpret_cast<const uint2*>(g + c);
        const float gv[4] = {bf16_lo(gw.x), bf16_hi(gw.x), bf16_lo(gw.y), bf16_hi(gw.y)};
        const int p0 = (c & 127) >> 1;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int p = p0 + h;
          const int ax = p < kPairsT ? 0 : (p < kPairsT + kPairsH ? 1 : 2);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float2 cs = na.tab[p + (ax == 0 ? tb[j][0] : (ax == 1 ? tb[j][1] : tb[j][2]))];
            // norm, x gamma, bf16 rounding point; rotation in fp32 (bf16 at the store)
            const uint32_t nv = pack_bf16x2(acc[i][j][2 * h] * r[j] * gv[2 * h], acc[i][j][2 * h + 1] * r[j] * gv[2 * h + 1]);
            const float a = bf16_lo(nv), b = bf16_hi(nv);
            acc[i][j][2 * h] = a * cs.x - b * cs.y;
            acc[i][j][2 * h + 1] = a * cs.y + b * cs.x;
          }
        }
      }
    }
    store_tile(out, M, N, m0, n0, smem, wave, lane, [&](int i, int j) {
      uint2 o;
      o.x = bad ? 0x7fc07fc0u : pack_bf16x2(acc[i][j][0], acc[i][j][1]);
      o.y = bad ? 0x7fc07fc0u : pack_bf16x2(acc[i][j][2], acc[i][j][3]);
      return o;
    });
    __syncthreads();  // the epilogue's LDS is the next tile's staging, and tile_sh is rewritten
  }
}

// Workgroups of the persistent kernel the device holds at once (cached per device).
static int proj_capacity(int dev) {
  static std::mutex mu;
  static int cap[64] = {};
  if (dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!cap[dev]) {
    int cus = 0, per_cu = 0, per_cu_norm = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, qkv_proj_kernel<false>, kPThreads, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_norm, qkv_proj_kernel<true>, kPThreads, 0) !=
            hipSuccess)
      return 0;
    cap[dev] = cus * (per_cu < per_cu_norm ? per_cu : per_cu_norm);
  }
  return cap[dev];
}

// Tile counts of M x N; false if they (or an operand tile's byte range, which a
// buffer descriptor addresses with 32 bits) do not fit the kernel's int32 math.
static bool proj_tiles(int64_t M, int N, int K, int64_t* ntm, int* ntn) {
  *ntm = (M + kPM - 1) / kPM;
  *ntn = (N + kPN - 1) / kPN;
  return *ntm <= INT32_MAX / 2 / *ntn && (int64_t)kPM * K * 2 <= (int64_t)INT32_MAX;
}

static hipError_t clear_words(void* p, int64_t bytes, hipStream_t stream) {
  const int64_t nz = bytes / 16;
  const int64_t blocks = (nz + 255) / 256;
  hipLaunchKernelGGL(zero16_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream,
                     static_cast<u32x4_t*>(p), nz);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_proj(const void* x, const void* w, const void* bias, void* out, int64_t M, int N, int K,
                           unsigned* counter, hipStream_t stream) {
  int64_t ntm;
  int ntn;
  if (!proj_tiles(M, N, K, &ntm, &ntn)) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int cap = proj_capacity(dev);
  if (cap < 1) return hipErrorInvalidConfiguration;
  const int ntiles = static_cast<int>(ntm * ntn);
  const int grid = cap < ntiles ? cap : ntiles;
  NormRopeArgs na = {};
  na.heads = K / 128;
  na.ctl = counter;
  na.xcd_queues = (ntn + 7) / 8 == 8 && grid >= 8;
  e = clear_words(counter, 32, stream);  // the tile counters start at zero
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(qkv_proj_kernel<false>, dim3(grid), dim3(kPThreads), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                     static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(out), static_cast<int>(M), N, K,
                     static_cast<int>(ntm), ntn, na);
  return hipGetLastError();
}

hipError_t launch_qkv_proj_norm_rope(const void* x, const void* w, const void* bias, const void* gq, const void* gk,
                                     const float2* tab, void* out, void* workspace, int64_t M, int heads, int S, int T,
                                     int H, int W, float eps, hipStream_t stream) {
  const int D = heads * 128, N = 3 * D, K = D;
  int64_t ntm;
  int ntn;
  if (!proj_tiles(M, N, K, &ntm, &ntn)) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int cap = proj_capacity(dev);
  // At most heads - 1 workgroups wait at once; one more must fit for every wait to end.
  if (cap < heads) return hipErrorInvalidConfiguration;
  const int ntiles = static_cast<int>(ntm * ntn);
  FusedWorkspace fw;
  if (!fused_workspace(M, heads, &fw)) return hipErrorInvalidValue;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  NormRopeArgs na;
  na.gq = static_cast<const uint16_t*>(gq);
  na.gk = static_cast<const uint16_t*>(gk);
  na.tab = tab;
  na.S = S;
  na.H = H;
  na.W = W;
  na.offH = T * kPairsT;
  na.offW = na.offH + H * kPairsH;
  na.heads = heads;
  na.inv_d = 1.0f / static_cast<float>(D);
  na.eps = eps;
  // The waits' bounds; WAN_PROJ_NORM_SPIN_LIMIT overrides both (tests force the
  // time-out path with it; every wait still ends).
  na.spin_limit = kSpinLimit;
  na.read_limit = kReadLimit;
  if (const char* env = std::getenv("WAN_PROJ_NORM_SPIN_LIMIT")) {
    const unsigned long v = std::strtoul(env, nullptr, 10);
    na.spin_limit = na.read_limit = static_cast<unsigned>(v < kSpinLimit ? v : kSpinLimit);
  }
  na.ctl = reinterpret_cast<unsigned*>(ws);
  na.xcd_queues = 0;  // the fused kernel takes its units in order (one queue)
  na.arrive = reinterpret_cast<unsigned*>(ws + fw.arrive_off);
  na.partial = reinterpret_cast<uint64_t*>(ws + fw.partial_off);
  // Counters, error word and the markers of the partial sums start at zero: a
  // fill kernel over the whole workspace (no memset node if the call is
  // captured in a graph).
  e = clear_words(ws, fw.bytes, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(qkv_proj_kernel<true>, dim3(cap < ntiles ? cap : ntiles), dim3(kPThreads), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                     static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(out), static_cast<int>(M), N, K,
                     static_cast<int>(ntm), ntn, na);
  return hipGetLastError();
}

}  // namespace wan
