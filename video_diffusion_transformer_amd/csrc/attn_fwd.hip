// Attention instances that normalise by the bf16 weights: the attention step
// (no log-sum-exp) and Skip-Softmax. The kernel is in attn_fwd_impl.hpp.
#include "attn_fwd_impl.hpp"

namespace wan {

hipError_t launch_attn_fwd(const void* qkv, void* out, float* lse, int B, int S, int heads,
                           float softmax_scale, hipStream_t stream) {
  const int nqt = (S + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)nqt * heads * B;
  if (nblocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  const auto* src = static_cast<const uint16_t*>(qkv);
  // The LSE-free instance (the attention step) normalises by the sum of the
  // bf16 weights; the one that also returns the LSE sums the fp32 weights
  // (attn_fwd_exact.hip).
  if (lse) return launch_attn_fwd_lse(qkv, out, lse, B, S, heads, softmax_scale, stream);
  hipLaunchKernelGGL((attn_fwd_kernel<kOutBf16, false, false>), dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0,
                     stream, src, src, out, nullptr, nullptr, S, S, heads, nqt, scale_log2,
                     SkipArgs{-INFINITY, nullptr, 0});
  return hipGetLastError();
}

hipError_t launch_attn_fwd_skip(const void* qkv, void* out, float* lse, uint8_t* kept, int B, int S, int heads,
                                float softmax_scale, float threshold, hipStream_t stream) {
  static_assert(kQT * 16 == kSkipBlockQ && kBN == kSkipBlockK, "skip blocks are a wave's rows and one key tile");
  const int nqt = (S + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)nqt * heads * B;
  if (nblocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  // exp(d) < threshold <=> d * log2(e) < log2(threshold), d in natural units;
  // the kernel's scores are already in scaled log2 units
  const SkipArgs sk{threshold > 0.f ? static_cast<float>(std::log2(static_cast<double>(threshold))) : -INFINITY, kept,
                    (S + kSkipBlockQ - 1) / kSkipBlockQ};
  const auto* src = static_cast<const uint16_t*>(qkv);
  if (lse)
    hipLaunchKernelGGL((attn_fwd_kernel<kOutBf16, true, true>), dim3(static_cast<unsigned>(nblocks)), dim3(kThreads),
                       0, stream, src, src, out, lse, nullptr, S, S, heads, nqt, scale_log2, sk);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<kOutBf16, false, true>), dim3(static_cast<unsigned>(nblocks)), dim3(kThreads),
                       0, stream, src, src, out, nullptr, nullptr, S, S, heads, nqt, scale_log2, sk);
  return hipGetLastError();
}

}  // namespace wan
