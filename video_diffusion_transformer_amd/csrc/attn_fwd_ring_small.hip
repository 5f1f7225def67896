// The ring-attention chunk and fold instances with two 16-query tiles per wave
// (256 queries per workgroup; built with WAN_ATTN_QT=2), for query shards whose
// grids fill the CUs better that way (launch_attn_fwd_chunk and
// launch_attn_fwd_chunk_fold in attn_fwd_exact.hip choose). The kernel is in
// attn_fwd_impl.hpp.
#include "attn_fwd_ring.hpp"

static_assert(wan::kBM == 256, "this file is built with two query tiles per wave");

namespace wan {

hipError_t launch_attn_fwd_chunk_q256(const void* q_src, int Sq, const void* kv_src, int Skv, float* out, float* lse,
                                      int B, int heads, float softmax_scale, hipStream_t stream) {
  return ring_chunk_launch(q_src, Sq, kv_src, Skv, out, lse, B, heads, softmax_scale, stream);
}

hipError_t launch_attn_fwd_chunk_fold_q256(const void* q_src, int Sq, const void* kv_src, int Skv, float* acc,
                                           float* acc_lse, void* out16, int B, int heads, float softmax_scale,
                                           hipStream_t stream) {
  return ring_fold_launch(q_src, Sq, kv_src, Skv, acc, acc_lse, out16, B, heads, softmax_scale, stream);
}

}  // namespace wan
