// Launch helpers of the ring-attention instances of attn_fwd_kernel, compiled
// into each translation unit that includes this header with that unit's tile
// size (attn_fwd_exact.hip: 384 queries per workgroup; attn_fwd_ring_small.hip:
// 256).
#pragma once

#include "attn_fwd_impl.hpp"

namespace wan {

namespace {

// The ring-attention launches (chunk: fp32 O and LSE of one key chunk; fold:
// the chunk merged into an accumulator), with this translation unit's tile
// size.
inline hipError_t ring_chunk_launch(const void* q_src, int Sq, const void* kv_src, int Skv, float* out, float* lse,
                                    int B, int heads, float softmax_scale, hipStream_t stream) {
  const int nqt = (Sq + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)nqt * heads * B;
  if (nblocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  hipLaunchKernelGGL((attn_fwd_kernel<kOutF32, true, false>), dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(q_src), static_cast<const uint16_t*>(kv_src), out, lse,
                     nullptr, Sq, Skv, heads, nqt, scale_log2, SkipArgs{-INFINITY, nullptr, 0});
  return hipGetLastError();
}

inline hipError_t ring_fold_launch(const void* q_src, int Sq, const void* kv_src, int Skv, float* acc, float* acc_lse,
                                   void* out16, int B, int heads, float softmax_scale, hipStream_t stream) {
  const int nqt = (Sq + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)nqt * heads * B;
  if (nblocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  hipLaunchKernelGGL((attn_fwd_kernel<kOutFold, true, false>), dim3(static_cast<unsigned>(nblocks)), dim3(kThreads),
                     0, stream, static_cast<const uint16_t*>(q_src), static_cast<const uint16_t*>(kv_src), acc, acc_lse,
                     static_cast<uint16_t*>(out16), Sq, Skv, heads, nqt, scale_log2, SkipArgs{-INFINITY, nullptr, 0});
  return hipGetLastError();
}

}  // namespace

}  // namespace wan
