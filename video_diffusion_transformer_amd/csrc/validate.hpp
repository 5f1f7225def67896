// Argument validation of the C ABI. Pure C++ (no HIP types or calls), so the
// same checks compile into the library and into a host-only test program.
//
// Every entry point validates before it touches memory or the HIP runtime, and
// returns a negative wan_status on the first failed check. The preconditions
// mirror the ones the TensorRT-LLM pull request "Optimize Wan2.2 Dataflow"
// lists for its packed QKV path (section "Fallback Behavior": self-attention,
// fused QKV, bf16 Q and K, matching head dims, rotary embeddings available,
// compatible norm weights) -- except that an unsupported case is an error here,
// never a silent fallback (the vLLM-Omni "Wan2.2 Text-to-Video" recipe, Notes:
// raise rather than degrade).
#pragma once

#include <cstdint>
#include <cstring>

#include "wan_attn.h"

namespace wan {

constexpr int64_t kHeadDim = 128;
constexpr int64_t kMaxHeads = 256;
constexpr int64_t kMaxTokens = INT32_MAX;  // token indices are 32-bit inside the kernels

// a*b with overflow detection for non-negative operands.
inline bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// Finite test on the bit pattern (exponent field not all ones): unlike
// std::isfinite it cannot be folded away by a compiler told that NaNs do not
// occur.
inline bool finite(float x) {
  uint32_t u;
  std::memcpy(&u, &x, sizeof u);
  return (u & 0x7f800000u) != 0x7f800000u;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Half-open byte ranges [a, a+na) and [b, b+nb) intersect.
inline bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + static_cast<uintptr_t>(nb) && y < x + static_cast<uintptr_t>(na);
}

struct Sizes {
  int64_t B = 0, S = 0, heads = 0, D = 0;
  int64_t rows = 0;       // B*S
  int64_t qkv_elems = 0;  // B*S*3D
  int64_t out_elems = 0;  // B*S*D
  int64_t lse_bytes = 0;  // B*heads*S*4
  bool empty = false;
};

// Shared shape checks. Returns WAN_OK and fills `z`, or an error.
inline int check_sizes(int64_t B, int64_t S, int64_t heads, int64_t head_dim, Sizes* z) {
  if (B < 0 || S < 0) return WAN_E_SHAPE;
  if (head_dim != kHeadDim) return WAN_E_UNSUPPORTED;
  if (heads < 1 || heads > kMaxHeads) return heads < 1 ? WAN_E_SHAPE : WAN_E_UNSUPPORTED;
  if (S > kMaxTokens) return WAN_E_OVERFLOW;
  z->B = B;
  z->S = S;
  z->heads = heads;
  z->D = heads * head_dim;
  if (!mul_ok(B, S, &z->rows)) return WAN_E_OVERFLOW;
  int64_t t;
  if (!mul_ok(z->rows, 3 * z->D, &z->qkv_elems)) return WAN_E_OVERFLOW;
  if (!mul_ok(z->qkv_elems, 2, &t)) return WAN_E_OVERFLOW;  // bytes
  if (!mul_ok(z->rows, z->D, &z->out_elems)) return WAN_E_OVERFLOW;
  int64_t lse_elems;
  if (!mul_ok(z->rows, heads, &lse_elems) || !mul_ok(lse_elems, 4, &z->lse_bytes)) return WAN_E_OVERFLOW;
  z->empty = (z->rows == 0);
  return WAN_OK;
}

inline int validate_qknorm_rope(const void* qkv, const void* gq, const void* gk, int64_t B, int64_t T,
                                int64_t H, int64_t W, int64_t heads, int64_t head_dim, float eps,
                                float theta, Sizes* z) {
  if (T < 0 || H < 0 || W < 0) return WAN_E_SHAPE;
  int64_t hw, S;
  if (!mul_ok(H, W, &hw) || !mul_ok(hw, T, &S)) return WAN_E_OVERFLOW;
  int rc = check_sizes(B, S, heads, head_dim, z);
  if (rc != WAN_OK) return rc;
  if (!finite(eps) || eps < 0.f) return WAN_E_VALUE;
  if (!finite(theta) || theta <= 0.f) return WAN_E_VALUE;
  if (z->empty) return WAN_OK;
  if (!qkv || !gq || !gk) return WAN_E_NULL;
  if (!aligned(qkv, 16) || !aligned(gq, 16) || !aligned(gk, 16)) return WAN_E_ALIGN;
  const int64_t qkv_bytes = z->qkv_elems * 2, g_bytes = z->D * 2;
  if (overlaps(qkv, qkv_bytes, gq, g_bytes) || overlaps(qkv, qkv_bytes, gk, g_bytes)) return WAN_E_ALIAS;
  return WAN_OK;
}

inline int validate_attn(const void* qkv, const void* out, const void* lse, int64_t B, int64_t S,
                         int64_t heads, int64_t head_dim, float scale, int64_t in_elem_bytes,
                         Sizes* z) {
  int rc = check_sizes(B, S, heads, head_dim, z);
  if (rc != WAN_OK) return rc;
  if (!finite(scale) || scale <= 0.f) return WAN_E_VALUE;
  if (z->empty) return WAN_OK;
  if (!qkv || !out) return WAN_E_NULL;
  if (!aligned(qkv, 16) || !aligned(out, 16) || (lse && !aligned(lse, 4))) return WAN_E_ALIGN;
  const int64_t in_bytes = z->qkv_elems * in_elem_bytes, out_bytes = z->out_elems * 2;
  const int64_t lse_bytes = z->lse_bytes;
  if (overlaps(qkv, in_bytes, out, out_bytes)) return WAN_E_ALIAS;
  if (lse && (overlaps(lse, lse_bytes, qkv, in_bytes) || overlaps(lse, lse_bytes, out, out_bytes)))
    return WAN_E_ALIAS;
  return WAN_OK;
}

// Bytes of a packed bf16 [B, Skv, 3D] buffer; false on overflow.
inline bool kv_chunk_bytes(int64_t B, int64_t Skv, int64_t D, int64_t* out) {
  int64_t t;
  return mul_ok(B, Skv, &t) && mul_ok(t, 3 * D, &t) && mul_ok(t, 2, out);
}

// Bytes of the Skip-Softmax decision map: B * heads * ceil(S/BQ) * ceil(S/BK).
inline bool skip_map_bytes(int64_t B, int64_t S, int64_t heads, int64_t* out) {
  if (S < 0 || S > INT64_MAX - WAN_SKIP_BLOCK_Q) return false;
  const int64_t nqb = (S + WAN_SKIP_BLOCK_Q - 1) / WAN_SKIP_BLOCK_Q, nkb = (S + WAN_SKIP_BLOCK_K - 1) / WAN_SKIP_BLOCK_K;
  int64_t t;
  return mul_ok(B, heads, &t) && mul_ok(t, nqb, &t) && mul_ok(t, nkb, out);
}

// Attention with Skip-Softmax: the checks of validate_attn, a finite
// threshold >= 0, and the optional decision map distinct from the other buffers.
inline int validate_attn_skip(const void* qkv, const void* out, const void* lse, const void* kept, int64_t B,
                              int64_t S, int64_t heads, int64_t head_dim, float scale, float threshold, Sizes* z) {
  int rc = validate_attn(qkv, out, lse, B, S, heads, head_dim, scale, 2, z);
  if (rc != WAN_OK) return rc;
  if (!finite(threshold) || threshold < 0.f) return WAN_E_VALUE;
  if (z->empty || !kept) return WAN_OK;
  int64_t map_bytes;
  if (!skip_map_bytes(B, S, heads, &map_bytes)) return WAN_E_OVERFLOW;
  if (overlaps(kept, map_bytes, qkv, z->qkv_elems * 2) || overlaps(kept, map_bytes, out, z->out_elems * 2) ||
      (lse && overlaps(kept, map_bytes, lse, z->lse_bytes)))
    return WAN_E_ALIAS;
  return WAN_OK;
}

inline int validate_attn_chunk(const void* q_src, const void* kv_src, const void* out, const void* lse, int64_t B,
                               int64_t Sq, int64_t Skv, int64_t heads, int64_t head_dim, float scale, Sizes* z) {
  if (Skv < 0) return WAN_E_SHAPE;
  if (Skv > kMaxTokens) return WAN_E_OVERFLOW;
  int rc = check_sizes(B, Sq, heads, head_dim, z);
  if (rc != WAN_OK) return rc;
  if (!finite(scale) || scale <= 0.f) return WAN_E_VALUE;
  if (z->empty) return WAN_OK;
  if (Skv == 0) return WAN_E_SHAPE;  // attention over no keys is undefined
  if (!q_src || !kv_src || !out || !lse) return WAN_E_NULL;
  if (!aligned(q_src, 16) || !aligned(kv_src, 16) || !aligned(out, 16) || !aligned(lse, 4)) return WAN_E_ALIGN;
  int64_t kv_elems;
  if (!kv_chunk_bytes(B, Skv, z->D, &kv_elems)) return WAN_E_OVERFLOW;
  const int64_t q_bytes = z->qkv_elems * 2, out_bytes = z->out_elems * 4, lse_bytes = z->lse_bytes;
  if (overlaps(out, out_bytes, q_src, q_bytes) || overlaps(out, out_bytes, kv_src, kv_elems) ||
      overlaps(lse, lse_bytes, q_src, q_bytes) || overlaps(lse, lse_bytes, kv_src, kv_elems) ||
      overlaps(lse, lse_bytes, out, out_bytes))
    return WAN_E_ALIAS;
  return WAN_OK;
}

inline int validate_attn_merge(const void* acc, const void* acc_lse, const void* chunk, const void* chunk_lse,
                               const void* out16, int64_t B, int64_t Sq, int64_t heads, int64_t head_dim, Sizes* z) {
  int rc = check_sizes(B, Sq, heads, head_dim, z);
  if (rc != WAN_OK) return rc;
  if (z->empty) return WAN_OK;
  if (!acc || !acc_lse || !chunk || !chunk_lse) return WAN_E_NULL;
  if (!aligned(acc, 16) || !aligned(chunk, 16) || !aligned(acc_lse, 4) || !aligned(chunk_lse, 4) ||
      (out16 && !aligned(out16, 16)))
    return WAN_E_ALIGN;
  const int64_t o_bytes = z->out_elems * 4, l_bytes = z->lse_bytes, h_bytes = z->out_elems * 2;
  const void* p[5] = {acc, acc_lse, chunk, chunk_lse, out16};
  const int64_t n[5] = {o_bytes, l_bytes, o_bytes, l_bytes, h_bytes};
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(p[i], n[i], p[j], n[j])) return WAN_E_ALIAS;
  return WAN_OK;
}

// One ring round folded into the accumulator: the chunk checks for the inputs,
// and acc, acc_lse, out16 (optional) distinct from the inputs and each other.
inline int validate_attn_chunk_fold(const void* q_src, const void* kv_src, const void* acc, const void* acc_lse,
                                    const void* out16, int64_t B, int64_t Sq, int64_t Skv, int64_t heads,
                                    int64_t head_dim, float scale, Sizes* z) {
  int rc = validate_attn_chunk(q_src, kv_src, acc, acc_lse, B, Sq, Skv, heads, head_dim, scale, z);
  if (rc != WAN_OK || z->empty) return rc;
  if (out16 && !aligned(out16, 16)) return WAN_E_ALIGN;
  int64_t kv_bytes;
  if (!kv_chunk_bytes(B, Skv, z->D, &kv_bytes)) return WAN_E_OVERFLOW;
  const int64_t h_bytes = z->out_elems * 2;
  if (overlaps(out16, h_bytes, q_src, z->qkv_elems * 2) || overlaps(out16, h_bytes, kv_src, kv_bytes) ||
      overlaps(out16, h_bytes, acc, z->out_elems * 4) || overlaps(out16, h_bytes, acc_lse, z->lse_bytes))
    return WAN_E_ALIAS;
  return WAN_OK;
}

// QKV projection: x [B, S, D], w [3D, D], bias [3D] (optional), out [B, S, 3D];
// out must not overlap an input.
inline int validate_qkv_proj(const void* x, const void* w, const void* bias, const void* out, int64_t B, int64_t S,
                             int64_t heads, int64_t head_dim, Sizes* z) {
  int rc = check_sizes(B, S, heads, head_dim, z);
  if (rc != WAN_OK || z->empty) return rc;
  if (z->rows > kMaxTokens - 256) return WAN_E_OVERFLOW;  // token rows and tile offsets are 32-bit in the GEMM
  if (!x || !w || !out) return WAN_E_NULL;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(out, 16) || (bias && !aligned(bias, 16))) return WAN_E_ALIGN;
  const int64_t x_bytes = z->out_elems * 2, w_bytes = 3 * z->D * z->D * 2, b_bytes = 3 * z->D * 2,
                o_bytes = z->qkv_elems * 2;
  if (overlaps(out, o_bytes, x, x_bytes) || overlaps(out, o_bytes, w, w_bytes) || overlaps(out, o_bytes, bias, b_bytes))
    return WAN_E_ALIAS;
  return WAN_OK;
}

// Workspace of the projection with the norm + RoPE epilogue, for `rows` tokens
// and `heads` heads: 256 bytes of control words (tile counter, error word), two
// 32-bit arrival counts (Q, K) per 256-token block (the span rounded up to 256 bytes),
// then rows x 2 heads 64-bit words (a partial sum of squares and its marker).
// False on overflow.
struct FusedWorkspace {
  int64_t arrive_off, partial_off, bytes;
};
constexpr int64_t kFusedTileTokens = 256, kFusedTileFeatures = 256;
inline bool fused_workspace(int64_t rows, int64_t heads, FusedWorkspace* f) {
  if (rows < 0 || heads < 1 || rows > INT64_MAX / 4 - kFusedTileTokens) return false;
  const int64_t ntm = (rows + kFusedTileTokens - 1) / kFusedTileTokens;
  int64_t part;
  if (!mul_ok(rows, 16 * heads, &part)) return false;
  f->arrive_off = 256;
  f->partial_off = 256 + (8 * ntm + 255) / 256 * 256;
  if (part > INT64_MAX - f->partial_off) return false;
  f->bytes = f->partial_off + part;
  return true;
}

// Projection + norm + RoPE: the norm checks on the output buffer (grid, eps,
// theta, gammas), the projection checks (x, w, bias against the output), a
// workspace of at least fused_workspace() bytes, 16-byte aligned, overlapping
// no other buffer, and a tile count within 32 bits.
inline int validate_qkv_proj_norm_rope(const void* x, const void* w, const void* bias, const void* gq, const void* gk,
                                       const void* out, const void* ws, int64_t ws_bytes, int64_t B, int64_t T,
                                       int64_t H, int64_t W, int64_t heads, int64_t head_dim, float eps, float theta,
                                       Sizes* z) {
  int rc = validate_qknorm_rope(out, gq, gk, B, T, H, W, heads, head_dim, eps, theta, z);
  if (rc != WAN_OK) return rc;
  rc = validate_qkv_proj(x, w, bias, out, B, z->S, heads, head_dim, z);
  if (rc != WAN_OK || z->empty) return rc;
  if (T > INT32_MAX / 22 || H > INT32_MAX / 21 || W > INT32_MAX / 21) return WAN_E_OVERFLOW;
  const int64_t ntm = (z->rows + kFusedTileTokens - 1) / kFusedTileTokens;
  const int64_t ntn = (3 * z->D + kFusedTileFeatures - 1) / kFusedTileFeatures;
  if (ntm > INT32_MAX / 2 / ntn) return WAN_E_OVERFLOW;
  FusedWorkspace f;
  if (!fused_workspace(z->rows, heads, &f)) return WAN_E_OVERFLOW;
  if (!ws) return WAN_E_NULL;
  if (!aligned(ws, 16)) return WAN_E_ALIGN;
  if (ws_bytes < f.bytes) return WAN_E_SHAPE;
  const void* p[6] = {x, w, bias, gq, gk, out};
  const int64_t n[6] = {z->out_elems * 2, 3 * z->D * z->D * 2, 3 * z->D * 2, z->D * 2, z->D * 2, z->qkv_elems * 2};
  for (int i = 0; i < 6; ++i)
    if (overlaps(ws, f.bytes, p[i], n[i])) return WAN_E_ALIAS;
  // the gammas are read while the output is written
  if (overlaps(gq, z->D * 2, out, z->qkv_elems * 2) || overlaps(gk, z->D * 2, out, z->qkv_elems * 2))
    return WAN_E_ALIAS;
  return WAN_OK;
}

// Bytes of the transposed fp8 V buffer: B * heads * 128 * S_pad, S_pad = S rounded up to 128.
inline bool fp8_vt_bytes(int64_t B, int64_t S, int64_t heads, int64_t* out) {
  if (S < 0 || S > INT64_MAX - 127) return false;
  const int64_t s_pad = (S + 127) / 128 * 128;
  int64_t t;
  return mul_ok(B, heads, &t) && mul_ok(t, kHeadDim, &t) && mul_ok(t, s_pad, out);
}

constexpr int64_t kMaxGridYZ = 65535;

inline int validate_quant_fp8(const void* qkv, const void* qk8, const void* vt8, const void* scales,
                              const void* amax, int64_t B, int64_t S, int64_t heads, int64_t head_dim,
                              Sizes* z) {
  int rc = check_sizes(B, S, heads, head_dim, z);
  if (rc != WAN_OK) return rc;
  if (B > kMaxGridYZ) return WAN_E_OVERFLOW;
  if (z->empty) return WAN_OK;
  if (!qkv || !qk8 || !vt8 || !scales || !amax) return WAN_E_NULL;
  if (!aligned(qkv, 16) || !aligned(qk8, 16) || !aligned(vt8, 16) || !aligned(scales, 4) || !aligned(amax, 4))
    return WAN_E_ALIGN;
  int64_t vt_bytes;
  if (!fp8_vt_bytes(B, S, heads, &vt_bytes)) return WAN_E_OVERFLOW;
  const int64_t in_bytes = z->qkv_elems * 2, qk_bytes = z->rows * 2 * z->D;
  const void* outs[4] = {qk8, vt8, scales, amax};
  const int64_t sizes[4] = {qk_bytes, vt_bytes, 12, 12};
  for (int i = 0; i < 4; ++i) {
    if (overlaps(outs[i], sizes[i], qkv, in_bytes)) return WAN_E_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], sizes[i], outs[j], sizes[j])) return WAN_E_ALIAS;
  }
  return WAN_OK;
}

// Norm + RoPE in place followed by the fp8 quantisation of the result: the
// checks of both calls, plus the gammas must not overlap an fp8 output.
inline int validate_qknorm_rope_fp8(const void* qkv, const void* gq, const void* gk, int64_t B, int64_t T,
                                    int64_t H, int64_t W, int64_t heads, int64_t head_dim, float eps, float theta,
                                    const void* qk8, const void* vt8, const void* scales, const void* amax, Sizes* z) {
  int rc = validate_qknorm_rope(qkv, gq, gk, B, T, H, W, heads, head_dim, eps, theta, z);
  if (rc != WAN_OK) return rc;
  rc = validate_quant_fp8(qkv, qk8, vt8, scales, amax, B, z->S, heads, head_dim, z);
  if (rc != WAN_OK || z->empty) return rc;
  int64_t vt_bytes;
  if (!fp8_vt_bytes(B, z->S, heads, &vt_bytes)) return WAN_E_OVERFLOW;
  const void* outs[4] = {qk8, vt8, scales, amax};
  const int64_t sizes[4] = {z->rows * 2 * z->D, vt_bytes, 12, 12};
  for (int i = 0; i < 4; ++i)
    if (overlaps(outs[i], sizes[i], gq, z->D * 2) || overlaps(outs[i], sizes[i], gk, z->D * 2)) return WAN_E_ALIAS;
  return WAN_OK;
}

// Norm + RoPE + e4m3 at a delayed scale: the norm checks (qkv is only read),
// the quantisation outputs distinct from qkv, the gammas and each other, and
// amax_prev (read while amax is cleared and written) distinct from every output.
inline int validate_qknorm_rope_fp8_delayed(const void* qkv, const void* gq, const void* gk, int64_t B, int64_t T,
                                            int64_t H, int64_t W, int64_t heads, int64_t head_dim, float eps,
                                            float theta, const void* amax_prev, const void* qk8, const void* vt8,
                                            const void* scales, const void* amax, Sizes* z) {
  int rc = validate_qknorm_rope_fp8(qkv, gq, gk, B, T, H, W, heads, head_dim, eps, theta, qk8, vt8, scales, amax, z);
  if (rc != WAN_OK || z->empty) return rc;
  if (!amax_prev) return WAN_E_NULL;
  if (!aligned(amax_prev, 4)) return WAN_E_ALIGN;
  int64_t vt_bytes;
  if (!fp8_vt_bytes(B, z->S, heads, &vt_bytes)) return WAN_E_OVERFLOW;
  const void* outs[4] = {qk8, vt8, scales, amax};
  const int64_t sizes[4] = {z->rows * 2 * z->D, vt_bytes, 12, 12};
  for (int i = 0; i < 4; ++i)
    if (overlaps(outs[i], sizes[i], amax_prev, 12)) return WAN_E_ALIAS;
  return WAN_OK;
}

inline int validate_attn_fp8(const void* qk8, const void* vt8, const void* scales, const void* out,
                             const void* lse, int64_t B, int64_t S, int64_t heads, int64_t head_dim, float scale,
                             Sizes* z) {
  int rc = check_sizes(B, S, heads, head_dim, z);
  if (rc != WAN_OK) return rc;
  if (!finite(scale) || scale <= 0.f) return WAN_E_VALUE;
  if (z->empty) return WAN_OK;
  if (!qk8 || !vt8 || !scales || !out) return WAN_E_NULL;
  if (!aligned(qk8, 16) || !aligned(vt8, 16) || !aligned(scales, 4) || !aligned(out, 16) ||
      (lse && !aligned(lse, 4)))
    return WAN_E_ALIGN;
  int64_t vt_bytes;
  if (!fp8_vt_bytes(B, S, heads, &vt_bytes)) return WAN_E_OVERFLOW;
  const int64_t qk_bytes = z->rows * 2 * z->D, out_bytes = z->out_elems * 2, lse_bytes = z->lse_bytes;
  const void* ins[3] = {qk8, vt8, scales};
  const int64_t in_sizes[3] = {qk_bytes, vt_bytes, 12};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(out, out_bytes, ins[i], in_sizes[i])) return WAN_E_ALIAS;
    if (lse && overlaps(lse, lse_bytes, ins[i], in_sizes[i])) return WAN_E_ALIAS;
  }
  if (lse && overlaps(lse, lse_bytes, out, out_bytes)) return WAN_E_ALIAS;
  return WAN_OK;
}

}  // namespace wan
