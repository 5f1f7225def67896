// Host-side launchers of the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wan_attn.h"

namespace wan {

// Q/K RMSNorm + bf16 + 3-D RoPE, in place, rows [row0, row0 + rows) of the
// packed buffer. `tab` holds the fp32 (cos, sin) pairs: frame axis [T][22],
// then row axis [H][21], then column axis [W][21].
// With amax non-null the kernel also folds max |x| of the rounded Q and K it
// writes and of V into amax[0..2] (atomic maxima on the float bits; the caller
// clears them first).
// With qk8 non-null (and amax_prev) the rotated Q and K are not stored in
// place but quantised to e4m3 into qk8 [rows, 2D] at the scales 448 /
// amax_prev[0..1], and max |x| of Q and K goes to amax[0..1].
hipError_t launch_qknorm_rope(void* qkv, const void* gq, const void* gk, const float2* tab,
                              int64_t row0, int64_t rows, int S, int T, int H, int W, int D,
                              float eps, float* amax, hipStream_t stream, uint8_t* qk8 = nullptr,
                              const float* amax_prev = nullptr);

// The rotary tables `tab` the norm kernel reads, built on the device (fp32
// roundings of double cos/sin) on `stream`; rope_table_entries() float2 entries.
int64_t rope_table_entries(int64_t T, int64_t H, int64_t W);
hipError_t launch_rope_table(float2* tab, int T, int H, int W, float theta, hipStream_t stream);

// bf16 attention forward over the packed buffer.
hipError_t launch_attn_fwd(const void* qkv, void* out, float* lse, int B, int S, int heads,
                           float softmax_scale, hipStream_t stream);
// The instance of launch_attn_fwd that also writes the log-sum-exp (lse != NULL).
hipError_t launch_attn_fwd_lse(const void* qkv, void* out, float* lse, int B, int S, int heads, float softmax_scale,
                               hipStream_t stream);

// Skip-Softmax (threshold mode) variant of it; kept (optional) receives the
// per-(query block, key tile) decisions.
constexpr int kSkipBlockQ = WAN_SKIP_BLOCK_Q;
constexpr int kSkipBlockK = WAN_SKIP_BLOCK_K;
hipError_t launch_attn_fwd_skip(const void* qkv, void* out, float* lse, uint8_t* kept, int B, int S, int heads,
                                float softmax_scale, float threshold, hipStream_t stream);

// Attention of the queries of q_src (Sq rows per batch entry) against the
// keys/values of kv_src (Skv rows), fp32 output and log-sum-exp.
hipError_t launch_attn_fwd_chunk(const void* q_src, int Sq, const void* kv_src, int Skv, float* out, float* lse, int B,
                                 int heads, float softmax_scale, hipStream_t stream);

// In-place log-sum-exp merge of a chunk result into an accumulator.
hipError_t launch_attn_fwd_chunk_fold(const void* q_src, int Sq, const void* kv_src, int Skv, float* acc,
                                      float* acc_lse, void* out16, int B, int heads, float softmax_scale,
                                      hipStream_t stream);

// The same two launches with 256 queries per workgroup (attn_fwd_ring_small.hip).
hipError_t launch_attn_fwd_chunk_q256(const void* q_src, int Sq, const void* kv_src, int Skv, float* out, float* lse,
                                      int B, int heads, float softmax_scale, hipStream_t stream);
hipError_t launch_attn_fwd_chunk_fold_q256(const void* q_src, int Sq, const void* kv_src, int Skv, float* acc,
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
// V only, at the scale 448 / amax_prev[2]: vt8, scales[0..2] (all three from
// amax_prev), max |v| into amax[2].
hipError_t launch_quant_v_delayed(const void* qkv, void* vt8, const float* amax_prev, float* scales, float* amax,
                                  int B, int S, int heads, hipStream_t stream);

// QKV projection out[M, N] = x[M, K] w[N, K]^T (+ bias), bf16; K a multiple of
// 128, N a multiple of 4. A persistent grid takes output tiles from *counter
// (16 bytes of device memory, cleared by the launch); launches that share a
// counter must not overlap.
hipError_t launch_qkv_proj(const void* x, const void* w, const void* bias, void* out, int64_t M, int N, int K,
                           unsigned* counter, hipStream_t stream);

// The projection of M = B * S tokens with the Q/K RMSNorm and 3-D RoPE in its
// epilogue (D = heads * 128; out [M, 3D] holds normalised, rotated Q and K and
// plain V). workspace: fused_workspace(M, heads) bytes (validate.hpp), its
// counters cleared by the launch itself (word 1 is nonzero afterwards if a
// token block's wait hit its spin limit). Fails with
// hipErrorInvalidConfiguration when the device cannot hold `heads` workgroups
// of the kernel at once.
hipError_t launch_qkv_proj_norm_rope(const void* x, const void* w, const void* bias, const void* gq, const void* gk,
                                     const float2* tab, void* out, void* workspace, int64_t M, int heads, int S, int T,
                                     int H, int W, float eps, hipStream_t stream);

// fp8 attention forward from the quantised buffers.
hipError_t launch_attn_fwd_fp8(const void* qk8, const void* vt8, const float* scales, void* out, float* lse, int B,
                               int S, int heads, float softmax_scale, hipStream_t stream);

}  // namespace wan
