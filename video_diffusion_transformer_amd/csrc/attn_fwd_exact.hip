// Attention instances that return a log-sum-exp (fp32 sums of the
// probabilities): dense attention with LSE, and the ring-attention chunk and
// fold modes. The kernel is in attn_fwd_impl.hpp.
#include "attn_fwd_impl.hpp"

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

hipError_t launch_attn_fwd_chunk(const void* q_src, int Sq, const void* kv_src, int Skv, float* out, float* lse, int B,
                                 int heads, float softmax_scale, hipStream_t stream) {
  const int nqt = (Sq + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)nqt * heads * B;
  if (nblocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  hipLaunchKernelGGL((attn_fwd_kernel<kOutF32, true, false>), dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(q_src), static_cast<const uint16_t*>(kv_src), out, lse,
                     nullptr, Sq, Skv, heads, nqt, scale_log2, SkipArgs{-INFINITY, nullptr, 0});
  return hipGetLastError();
}

hipError_t launch_attn_fwd_chunk_fold(const void* q_src, int Sq, const void* kv_src, int Skv, float* acc,
                                      float* acc_lse, void* out16, int B, int heads, float softmax_scale,
                                      hipStream_t stream) {
  const int nqt = (Sq + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)nqt * heads * B;
  if (nblocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  hipLaunchKernelGGL((attn_fwd_kernel<kOutFold, true, false>), dim3(static_cast<unsigned>(nblocks)), dim3(kThreads),
                     0, stream, static_cast<const uint16_t*>(q_src), static_cast<const uint16_t*>(kv_src), acc, acc_lse,
                     static_cast<uint16_t*>(out16), Sq, Skv, heads, nqt, scale_log2, SkipArgs{-INFINITY, nullptr, 0});
  return hipGetLastError();
}

}  // namespace wan
