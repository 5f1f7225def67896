// Host-side launchers of the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wan {

// Q/K RMSNorm + bf16 + 3-D RoPE, in place, rows [row0, row0 + rows) of the
// packed buffer. `tab` holds the fp32 (cos, sin) pairs: frame axis [T][22],
// then row axis [H][21], then column axis [W][21].
// With amax non-null the kernel also folds max |x| of the rounded Q and K it
// writes and of V into amax[0..2] (atomic maxima on the float bits; the caller
// clears them first).
hipError_t launch_qknorm_rope(void* qkv, const void* gq, const void* gk, const float2* tab,
                              int64_t row0, int64_t rows, int S, int T, int H, int W, int D,
                              float eps, float* amax, hipStream_t stream);

// bf16 attention forward over the packed buffer.
hipError_t launch_attn_fwd(const void* qkv, void* out, float* lse, int B, int S, int heads,
                           float softmax_scale, hipStream_t stream);

// Attention of the queries of q_src (Sq rows per batch entry) against the
// keys/values of kv_src (Skv rows), fp32 output and log-sum-exp.
hipError_t launch_attn_fwd_chunk(const void* q_src, int Sq, const void* kv_src, int Skv, float* out, float* lse, int B,
                                 int heads, float softmax_scale, hipStream_t stream);

// In-place log-sum-exp merge of a chunk result into an accumulator.
hipError_t launch_attn_fwd_chunk_fold(const void* q_src, int Sq, const void* kv_src, int Skv, float* acc,
                                      float* acc_lse, void* out16, int B, int heads, float softmax_scale,
                                      hipStream_t stream);
hipError_t launch_attn_merge(float* acc, float* acc_lse, const float* chunk, const float* chunk_lse, void* out16,
                             int B, int Sq, int heads, hipStream_t stream);

// fp8: per-tensor amax + e4m3 quantisation into qk8 [B, S, 2D] and
// vt8 [B, heads, 128, S_pad] (V transposed per head, zero past S).
hipError_t launch_qkv_quant_fp8(const void* qkv, void* qk8, void* vt8, float* scales, float* amax, int B, int S,
                                int heads, hipStream_t stream);
// The two halves of it: clearing amax, and the quantisation given amax.
hipError_t launch_amax_clear(float* amax, hipStream_t stream);
hipError_t launch_quant_fp8(const void* qkv, void* qk8, void* vt8, float* scales, const float* amax, int B, int S,
                            int heads, hipStream_t stream);

// QKV projection out[M, N] = x[M, K] w[N, K]^T (+ bias), bf16; K a multiple of
// 64, N a multiple of 4.
hipError_t launch_qkv_proj(const void* x, const void* w, const void* bias, void* out, int64_t M, int N, int K,
                           hipStream_t stream);

// fp8 attention forward from the quantised buffers.
hipError_t launch_attn_fwd_fp8(const void* qk8, const void* vt8, const float* scales, void* out, float* lse, int B,
                               int S, int heads, float softmax_scale, hipStream_t stream);

}  // namespace wan
