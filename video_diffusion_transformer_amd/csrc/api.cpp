// extern "C" entry points of libwan_attn.so: validate -> (tables) -> launch.
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "kernels.hpp"
#include "validate.hpp"
#include "wan_attn.h"

namespace {

// ---------------------------------------------------------------- RoPE tables
// fp32 (cos, sin) of pos * theta^(-2j/d_a) for the frame axis (d_a = 44, 22
// pairs), the row axis (42, 21 pairs) and the column axis (42, 21 pairs) --
// Wan2.2's 3-D rotary split of a 128-channel head -- computed in double and
// rounded once to fp32 by a device kernel (the one the allocation-free entry
// point also uses). One device allocation per (device, T, H, W, theta), kept
// until the process ends; built on the caller's stream, which is synchronised
// once so that calls on other streams find it complete.
using TabKey = std::tuple<int, int64_t, int64_t, int64_t, uint32_t>;
std::mutex g_tab_mu;
std::map<TabKey, float2*> g_tabs;

int rope_table(int64_t T, int64_t H, int64_t W, float theta, hipStream_t stream, const float2** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return WAN_E_HIP;
  uint32_t tbits;
  std::memcpy(&tbits, &theta, 4);
  const TabKey key{dev, T, H, W, tbits};
  std::lock_guard<std::mutex> lock(g_tab_mu);
  auto it = g_tabs.find(key);
  if (it != g_tabs.end()) {
    *out = it->second;
    return WAN_OK;
  }
  const int64_t n = wan::rope_table_entries(T, H, W);
  float2* dptr = nullptr;
  if (hipMalloc(&dptr, (n > 0 ? n : 1) * sizeof(float2)) != hipSuccess) return WAN_E_NOMEM;
  if (wan::launch_rope_table(dptr, static_cast<int>(T), static_cast<int>(H), static_cast<int>(W), theta, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipFree(dptr);
    return WAN_E_HIP;
  }
  g_tabs.emplace(key, dptr);
  *out = dptr;
  return WAN_OK;
}

// --------------------------------------------------- projection tile counters
// The persistent projection takes its tiles from a 32-byte block of device
// counters (one per XCD queue) that the launch clears first. Each call takes
// the next slot of a ring of 65,536 per device (2 MB, allocated on the first
// call on the device and
// kept until the process ends), so calls on different streams, or on a stream
// handle reused after a destroy, never share a counter unless 65,536 calls
// are in flight at once.
constexpr int kCounterSlots = 1 << 16;
constexpr int kMaxDevices = 64;
std::mutex g_cnt_mu;
unsigned char* g_counter_ring[kMaxDevices] = {};
uint32_t g_counter_next[kMaxDevices] = {};

int proj_counter(unsigned** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WAN_E_HIP;
  std::lock_guard<std::mutex> lock(g_cnt_mu);
  if (!g_counter_ring[dev]) {
    void* p = nullptr;
    if (hipMalloc(&p, static_cast<size_t>(kCounterSlots) * 32) != hipSuccess) return WAN_E_NOMEM;
    g_counter_ring[dev] = static_cast<unsigned char*>(p);
  }
  const uint32_t slot = g_counter_next[dev]++ % kCounterSlots;
  *out = reinterpret_cast<unsigned*>(g_counter_ring[dev] + static_cast<size_t>(slot) * 32);
  return WAN_OK;
}

constexpr int64_t kMaxRowsPerLaunch = 1 << 21;  // rows * threads per launch stays below 2^32

}  // namespace

extern "C" {

int wan_abi_version(void) { return WAN_ABI_VERSION; }

const char* wan_status_str(int status) {
  switch (status) {
    case WAN_OK: return "ok";
    case WAN_E_NULL: return "a required pointer is NULL";
    case WAN_E_SHAPE: return "invalid size (negative, zero where it must not be, or inconsistent)";
    case WAN_E_UNSUPPORTED: return "unsupported configuration (head_dim must be 128, heads 1..256)";
    case WAN_E_ALIGN: return "a pointer is not aligned as required (16 bytes; 4 for fp32 vectors)";
    case WAN_E_ALIAS: return "an output overlaps an input";
    case WAN_E_OVERFLOW: return "a size product overflows, or S exceeds 2^31-1";
    case WAN_E_HIP: return "HIP runtime error or kernel launch failure";
    case WAN_E_NOMEM: return "device allocation of a library table failed";
    case WAN_E_VALUE: return "a scalar argument is out of range";
    case WAN_E_LIMIT: return "beyond the fixed capacity of the allocation-free entry point (rotary table entries)";
    default: return "unknown status";
  }
}

int wan_token_grid(int64_t width, int64_t height, int64_t num_frames, int64_t* T, int64_t* H, int64_t* W) {
  if (!T || !H || !W) return WAN_E_NULL;
  if (width < 0 || height < 0 || num_frames < 1 || (num_frames - 1) % 4 != 0) return WAN_E_SHAPE;
  // Pixels rounded down to a multiple of 16, then 8x VAE compression and 2x
  // patchify per spatial axis: 16 pixels per token. 4x temporal compression
  // with the first frame kept: (F - 1) / 4 + 1 latent frames.
  const int64_t t = (num_frames - 1) / 4 + 1, h = (height / 16) * 16 / 8 / 2, w = (width / 16) * 16 / 8 / 2;
  int64_t hw, s;
  if (!wan::mul_ok(h, w, &hw) || !wan::mul_ok(hw, t, &s)) return WAN_E_OVERFLOW;
  *T = t;
  *H = h;
  *W = w;
  return WAN_OK;
}

int wan_qkv_proj(const void* x, const void* w_qkv, const void* bias, void* qkv, int64_t B, int64_t S, int64_t heads,
                 int64_t head_dim, void* stream) {
  wan::Sizes z;
  int rc = wan::validate_qkv_proj(x, w_qkv, bias, qkv, B, S, heads, head_dim, &z);
  if (rc != WAN_OK || z.empty) return rc;
  auto st = static_cast<hipStream_t>(stream);
  unsigned* counter = nullptr;
  rc = proj_counter(&counter);
  if (rc != WAN_OK) return rc;
  if (wan::launch_qkv_proj(x, w_qkv, bias, qkv, z.rows, static_cast<int>(3 * z.D), static_cast<int>(z.D), counter,
                           st) != hipSuccess)
    return WAN_E_HIP;
  return WAN_OK;
}

int64_t wan_qkv_proj_norm_rope_workspace_bytes(int64_t B, int64_t S, int64_t heads, int64_t head_dim) {
  wan::Sizes z;
  if (wan::check_sizes(B, S, heads, head_dim, &z) != WAN_OK) return -1;
  wan::FusedWorkspace f;
  if (!wan::fused_workspace(z.rows, heads, &f)) return -1;
  return f.bytes;
}

int wan_qkv_proj_norm_rope(const void* x, const void* w_qkv, const void* bias, const void* gamma_q,
                           const void* gamma_k, void* qkv, void* workspace, int64_t workspace_bytes, int64_t B,
                           int64_t T, int64_t H, int64_t W, int64_t heads, int64_t head_dim, float eps, float theta,
                           void* stream) {
  wan::Sizes z;
  int rc = wan::validate_qkv_proj_norm_rope(x, w_qkv, bias, gamma_q, gamma_k, qkv, workspace, workspace_bytes, B, T,
                                            H, W, heads, head_dim, eps, theta, &z);
  if (rc != WAN_OK || z.empty) return rc;
  auto st = static_cast<hipStream_t>(stream);
  const float2* tab = nullptr;
  rc = rope_table(T, H, W, theta, st, &tab);
  if (rc != WAN_OK) return rc;
  const hipError_t e = wan::launch_qkv_proj_norm_rope(
      x, w_qkv, bias, gamma_q, gamma_k, tab, qkv, workspace, z.rows, static_cast<int>(heads), static_cast<int>(z.S),
      static_cast<int>(T), static_cast<int>(H), static_cast<int>(W), eps, st);
  if (e == hipErrorInvalidConfiguration) return WAN_E_UNSUPPORTED;
  return e == hipSuccess ? WAN_OK : WAN_E_HIP;
}

int wan_qknorm_rope(void* qkv, const void* gamma_q, const void* gamma_k, int64_t B, int64_t T,
                    int64_t H, int64_t W, int64_t heads, int64_t head_dim, float eps, float theta,
                    void* stream) {
  wan::Sizes z;
  int rc = wan::validate_qknorm_rope(qkv, gamma_q, gamma_k, B, T, H, W, heads, head_dim, eps, theta, &z);
  if (rc != WAN_OK || z.empty) return rc;
  if (T > INT32_MAX / 22 || H > INT32_MAX / 21 || W > INT32_MAX / 21) return WAN_E_OVERFLOW;
  const float2* tab = nullptr;
  rc = rope_table(T, H, W, theta, static_cast<hipStream_t>(stream), &tab);
  if (rc != WAN_OK) return rc;
  auto st = static_cast<hipStream_t>(stream);
  for (int64_t r0 = 0; r0 < z.rows; r0 += kMaxRowsPerLaunch) {
    const int64_t n = z.rows - r0 < kMaxRowsPerLaunch ? z.rows - r0 : kMaxRowsPerLaunch;
    if (wan::launch_qknorm_rope(qkv, gamma_q, gamma_k, tab, r0, n, static_cast<int>(z.S), static_cast<int>(T),
                                static_cast<int>(H), static_cast<int>(W), static_cast<int>(z.D), eps, nullptr,
                                st) != hipSuccess)
      return WAN_E_HIP;
  }
  return WAN_OK;
}

int wan_qknorm_rope_quant_fp8(void* qkv, const void* gamma_q, const void* gamma_k, int64_t B, int64_t T, int64_t H,
                              int64_t W, int64_t heads, int64_t head_dim, float eps, float theta, void* qk8,
                              void* vt8, float* scales, float* amax, void* stream) {
  wan::Sizes z;
  int rc = wan::validate_qknorm_rope_fp8(qkv, gamma_q, gamma_k, B, T, H, W, heads, head_dim, eps, theta, qk8, vt8,
                                         scales, amax, &z);
  if (rc != WAN_OK || z.empty) return rc;
  if (T > INT32_MAX / 22 || H > INT32_MAX / 21 || W > INT32_MAX / 21) return WAN_E_OVERFLOW;
  const float2* tab = nullptr;
  rc = rope_table(T, H, W, theta, static_cast<hipStream_t>(stream), &tab);
  if (rc != WAN_OK) return rc;
  auto st = static_cast<hipStream_t>(stream);
  if (wan::launch_amax_clear(amax, st) != hipSuccess) return WAN_E_HIP;
  for (int64_t r0 = 0; r0 < z.rows; r0 += kMaxRowsPerLaunch) {
    const int64_t n = z.rows - r0 < kMaxRowsPerLaunch ? z.rows - r0 : kMaxRowsPerLaunch;
    if (wan::launch_qknorm_rope(qkv, gamma_q, gamma_k, tab, r0, n, static_cast<int>(z.S), static_cast<int>(T),
                                static_cast<int>(H), static_cast<int>(W), static_cast<int>(z.D), eps, amax,
                                st) != hipSuccess)
      return WAN_E_HIP;
  }
  if (wan::launch_quant_fp8(qkv, qk8, vt8, scales, amax, static_cast<int>(B), static_cast<int>(z.S),
                            static_cast<int>(heads), st) != hipSuccess)
    return WAN_E_HIP;
  return WAN_OK;
}

int wan_qknorm_rope_quant_fp8_delayed(const void* qkv, const void* gamma_q, const void* gamma_k, int64_t B, int64_t T,
                                      int64_t H, int64_t W, int64_t heads, int64_t head_dim, float eps, float theta,
                                      const float* amax_prev, void* qk8, void* vt8, float* scales, float* amax,
                                      void* stream) {
  wan::Sizes z;
  int rc = wan::validate_qknorm_rope_fp8_delayed(qkv, gamma_q, gamma_k, B, T, H, W, heads, head_dim, eps, theta,
                                                 amax_prev, qk8, vt8, scales, amax, &z);
  if (rc != WAN_OK || z.empty) return rc;
  if (T > INT32_MAX / 22 || H > INT32_MAX / 21 || W > INT32_MAX / 21) return WAN_E_OVERFLOW;
  const float2* tab = nullptr;
  rc = rope_table(T, H, W, theta, static_cast<hipStream_t>(stream), &tab);
  if (rc != WAN_OK) return rc;
  auto st = static_cast<hipStream_t>(stream);
  if (wan::launch_amax_clear(amax, st) != hipSuccess) return WAN_E_HIP;
  for (int64_t r0 = 0; r0 < z.rows; r0 += kMaxRowsPerLaunch) {
    const int64_t n = z.rows - r0 < kMaxRowsPerLaunch ? z.rows - r0 : kMaxRowsPerLaunch;
    // the kernel reads qkv and writes qk8 only (never the packed buffer) in this mode
    if (wan::launch_qknorm_rope(const_cast<void*>(qkv), gamma_q, gamma_k, tab, r0, n, static_cast<int>(z.S),
                                static_cast<int>(T), static_cast<int>(H), static_cast<int>(W), static_cast<int>(z.D),
                                eps, amax, st, static_cast<uint8_t*>(qk8), amax_prev) != hipSuccess)
      return WAN_E_HIP;
  }
  if (wan::launch_quant_v_delayed(qkv, vt8, amax_prev, scales, amax, static_cast<int>(B), static_cast<int>(z.S),
                                  static_cast<int>(heads), st) != hipSuccess)
    return WAN_E_HIP;
  return WAN_OK;
}

int wan_attn_fwd(const void* qkv, void* out, float* lse, int64_t B, int64_t S, int64_t heads,
                 int64_t head_dim, float softmax_scale, void* stream) {
  wan::Sizes z;
  int rc = wan::validate_attn(qkv, out, lse, B, S, heads, head_dim, softmax_scale, 2, &z);
  if (rc != WAN_OK || z.empty) return rc;
  if (B > INT32_MAX) return WAN_E_OVERFLOW;
  if (wan::launch_attn_fwd(qkv, out, lse, static_cast<int>(B), static_cast<int>(S), static_cast<int>(heads),
                           softmax_scale, static_cast<hipStream_t>(stream)) != hipSuccess)
    return WAN_E_HIP;
  return WAN_OK;
}

int wan_attn_fwd_skip(const void* qkv, void* out, float* lse, uint8_t* kept, int64_t B, int64_t S, int64_t heads,
                      int64_t head_dim, float softmax_scale, float threshold, void* stream) {
  wan::Sizes z;
  int rc = wan::validate_attn_skip(qkv, out, lse, kept, B, S, heads, head_dim, softmax_scale, threshold, &z);
  if (rc != WAN_OK || z.empty) return rc;
  if (B > INT32_MAX) return WAN_E_OVERFLOW;
  if (wan::launch_attn_fwd_skip(qkv, out, lse, kept, static_cast<int>(B), static_cast<int>(S),
                                static_cast<int>(heads), softmax_scale, threshold,
                                static_cast<hipStream_t>(stream)) != hipSuccess)
    return WAN_E_HIP;
  return WAN_OK;
}

int64_t wan_attn_skip_map_bytes(int64_t B, int64_t S, int64_t heads, int64_t head_dim) {
  if (B < 0 || S < 0 || heads < 0 || head_dim != wan::kHeadDim) return -1;
  int64_t n;
  return wan::skip_map_bytes(B, S, heads, &n) ? n : -1;
}

int wan_attn_fwd_chunk(const void* q_src, int64_t Sq, const void* kv_src, int64_t Skv, float* out, float* lse,
                       int64_t B, int64_t heads, int64_t head_dim, float softmax_scale, void* stream) {
  wan::Sizes z;
  int rc = wan::validate_attn_chunk(q_src, kv_src, out, lse, B, Sq, Skv, heads, head_dim, softmax_scale, &z);
  if (rc != WAN_OK || z.empty) return rc;
  if (B > INT32_MAX) return WAN_E_OVERFLOW;
  if (wan::launch_attn_fwd_chunk(q_src, static_cast<int>(Sq), kv_src, static_cast<int>(Skv), out, lse,
                                 static_cast<int>(B), static_cast<int>(heads), softmax_scale,
                                 static_cast<hipStream_t>(stream)) != hipSuccess)
    return WAN_E_HIP;
  return WAN_OK;
}

int wan_attn_fwd_chunk_merge(const void* q_src, int64_t Sq, const void* kv_src, int64_t Skv, float* acc_out,
                             float* acc_lse, void* out_bf16, int64_t B, int64_t heads, int64_t head_dim,
                             float softmax_scale, void* stream) {
  wan::Sizes z;
  int rc = wan::validate_attn_chunk_fold(q_src, kv_src, acc_out, acc_lse, out_bf16, B, Sq, Skv, heads, head_dim,
                                         softmax_scale, &z);
  if (rc != WAN_OK || z.empty) return rc;
  if (B > INT32_MAX) return WAN_E_OVERFLOW;
  if (wan::launch_attn_fwd_chunk_fold(q_src, static_cast<int>(Sq), kv_src, static_cast<int>(Skv), acc_out, acc_lse,
                                      out_bf16, static_cast<int>(B), static_cast<int>(heads), softmax_scale,
                                      static_cast<hipStream_t>(stream)) != hipSuccess)
    return WAN_E_HIP;
  return WAN_OK;
}

int wan_attn_merge(float* acc_out, float* acc_lse, const float* chunk_out, const float* chunk_lse, void* out_bf16,
                   int64_t B, int64_t Sq, int64_t heads, int64_t head_dim, void* stream) {
  wan::Sizes z;
  int rc = wan::validate_attn_merge(acc_out, acc_lse, chunk_out, chunk_lse, out_bf16, B, Sq, heads, head_dim, &z);
  if (rc != WAN_OK || z.empty) return rc;
  if (B > INT32_MAX) return WAN_E_OVERFLOW;
  if (wan::launch_attn_merge(acc_out, acc_lse, chunk_out, chunk_lse, out_bf16, static_cast<int>(B), static_cast<int>(Sq),
                             static_cast<int>(heads), static_cast<hipStream_t>(stream)) != hipSuccess)
    return WAN_E_HIP;
  return WAN_OK;
}

int wan_qkv_quant_fp8(const void* qkv, void* qk8, void* vt8, float* scales, float* amax, int64_t B, int64_t S,
                      int64_t heads, int64_t head_dim, void* stream) {
  wan::Sizes z;
  int rc = wan::validate_quant_fp8(qkv, qk8, vt8, scales, amax, B, S, heads, head_dim, &z);
  if (rc != WAN_OK || z.empty) return rc;
  if (wan::launch_qkv_quant_fp8(qkv, qk8, vt8, scales, amax, static_cast<int>(B), static_cast<int>(S),
                                static_cast<int>(heads), static_cast<hipStream_t>(stream)) != hipSuccess)
    return WAN_E_HIP;
  return WAN_OK;
}

int64_t wan_fp8_vt_bytes(int64_t B, int64_t S, int64_t heads, int64_t head_dim) {
  if (B < 0 || S < 0 || heads < 0 || head_dim != wan::kHeadDim) return -1;
  int64_t n;
  return wan::fp8_vt_bytes(B, S, heads, &n) ? n : -1;
}

int wan_attn_fwd_fp8(const void* qk8, const void* vt8, const float* scales, void* out, float* lse, int64_t B,
                     int64_t S, int64_t heads, int64_t head_dim, float softmax_scale, void* stream) {
  wan::Sizes z;
  int rc = wan::validate_attn_fp8(qk8, vt8, scales, out, lse, B, S, heads, head_dim, softmax_scale, &z);
  if (rc != WAN_OK || z.empty) return rc;
  if (B > INT32_MAX) return WAN_E_OVERFLOW;
  if (wan::launch_attn_fwd_fp8(qk8, vt8, scales, out, lse, static_cast<int>(B), static_cast<int>(S),
                               static_cast<int>(heads), softmax_scale, static_cast<hipStream_t>(stream)) != hipSuccess)
    return WAN_E_HIP;
  return WAN_OK;
}

}  // extern "C"
