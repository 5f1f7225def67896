// Attention instances that return a log-sum-exp (fp32 sums of the
// probabilities): dense attention with LSE, and the ring-attention chunk and
// fold modes (384 queries per workgroup; the 256-query forms are in
// attn_fwd_ring_small.hip). The kernel is in attn_fwd_impl.hpp.
#include <mutex>

#include "attn_fwd_ring.hpp"

namespace wan {

hipError_t launch_attn_fwd_lse(const void* qkv, void* out, float* lse, int B, int S, int heads, float softmax_scale,
                               hipStream_t stream) {
  const int nqt = (S + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)nqt * heads * B;
  if (nblocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  const auto* src = static_cast<const uint16_t*>(qkv);
  hipLaunchKernelGGL((attn_fwd_kernel<kOutBf16, true, false>), dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0,
                     stream, src, src, out, lse, nullptr, S, S, heads, nqt, scale_log2, SkipArgs{-INFINITY, nullptr, 0});
  return hipGetLastError();
}

// Ring chunks hold a shard of the queries (S / cp per rank), so their grids
// can fill the CUs badly: at 480p and cp = 8, 4095 queries per (b, h) make
// 880 workgroups of 384 queries on 256 CUs (3.4 rounds, the last 44% full).
// The same instances with 256 queries per workgroup (attn_fwd_ring_small.hip)
// cost 7% more per query (fewer MFMAs per staged K/V fragment: dense
// attention with LSE at 480p 36.9 against 34.2 ms) but make 1280 workgroups
// (5 full rounds): the ring share at 480p, cp = 8, took 5.43-5.49 ms against
// 5.68-5.74. Each launch takes the size whose grid, weighted by that cost,
// fills the CUs better; the results are the same bits either way (a query's
// arithmetic does not depend on the workgroup size).
static int device_cus() {
  static std::mutex mu;
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!cus[dev] && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus[dev] = 0;
  return cus[dev];
}

static bool ring_small_tiles(int Sq, int B, int heads) {
  const int64_t cus = device_cus();
  if (cus <= 0) return false;
  auto fill = [&](int64_t bm) {  // workgroups over workgroup slots (one per CU), whole rounds
    const int64_t n = (Sq + bm - 1) / bm * heads * B;
    return static_cast<double>(n) / static_cast<double>((n + cus - 1) / cus * cus);
  };
  return 0.93 * fill(256) > fill(kBM);
}

hipError_t launch_attn_fwd_chunk(const void* q_src, int Sq, const void* kv_src, int Skv, float* out, float* lse, int B,
                                 int heads, float softmax_scale, hipStream_t stream) {
  if (ring_small_tiles(Sq, B, heads))
    return launch_attn_fwd_chunk_q256(q_src, Sq, kv_src, Skv, out, lse, B, heads, softmax_scale, stream);
  return ring_chunk_launch(q_src, Sq, kv_src, Skv, out, lse, B, heads, softmax_scale, stream);
}

hipError_t launch_attn_fwd_chunk_fold(const void* q_src, int Sq, const void* kv_src, int Skv, float* acc,
                                      float* acc_lse, void* out16, int B, int heads, float softmax_scale,
                                      hipStream_t stream) {
  if (ring_small_tiles(Sq, B, heads))
    return launch_attn_fwd_chunk_fold_q256(q_src, Sq, kv_src, Skv, acc, acc_lse, out16, B, heads, softmax_scale,
                                           stream);
  return ring_fold_launch(q_src, Sq, kv_src, Skv, acc, acc_lse, out16, B, heads, softmax_scale, stream);
}

}  // namespace wan
