// wan_qknorm_rope_noalloc: the in-place Q/K norm + RoPE of wan_qknorm_rope for
// callers that cannot allocate (code under HIP graph capture, tight serving
// loops). wan_qknorm_rope keeps its rotary (cos, sin) tables in device
// allocations it makes on the first call of each grid; this entry point keeps
// them instead in a fixed file-scope device array and rebuilds them on every
// call, with the same table kernel, so its output is bit-identical.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"
#include "validate.hpp"
#include "wan_attn.h"

namespace {

// Scratch for the rotary tables: T*22 + H*21 + W*21 float2 entries at most
// (64 Ki entries = 512 KiB per device, held until the process ends).
constexpr int64_t kScratchEntries = int64_t(1) << 16;
__device__ __align__(256) float2 scratch[kScratchEntries];

// The array's device address, per device. In host code `scratch` names a host
// stand-in; only the address hipGetSymbolAddress returns may reach a kernel.
constexpr int kMaxDevices = 64;
std::mutex g_mu;
float2* g_ptr[kMaxDevices] = {};

int scratch_ptr(float2** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WAN_E_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WAN_E_HIP;
    g_ptr[dev] = static_cast<float2*>(p);
  }
  *out = g_ptr[dev];
  return WAN_OK;
}

constexpr int64_t kMaxRowsPerLaunch = 1 << 21;  // as wan_qknorm_rope: rows * threads per launch below 2^32

}  // namespace

extern "C" int wan_qknorm_rope_noalloc(void* qkv, const void* gamma_q, const void* gamma_k, int64_t B, int64_t T,
                                       int64_t H, int64_t W, int64_t heads, int64_t head_dim, float eps, float theta,
                                       void* stream) {
  wan::Sizes z;
  int rc = wan::validate_qknorm_rope(qkv, gamma_q, gamma_k, B, T, H, W, heads, head_dim, eps, theta, &z);
  if (rc != WAN_OK || z.empty) return rc;
  if (T > INT32_MAX / 22 || H > INT32_MAX / 21 || W > INT32_MAX / 21) return WAN_E_OVERFLOW;
  if (wan::rope_table_entries(T, H, W) > kScratchEntries) return WAN_E_LIMIT;
  float2* tab = nullptr;
  rc = scratch_ptr(&tab);
  if (rc != WAN_OK) return rc;
  auto st = static_cast<hipStream_t>(stream);
  // Every call rebuilds the tables: the array is shared by all calls on this
  // device and holds whatever the last call left.
  if (wan::launch_rope_table(tab, static_cast<int>(T), static_cast<int>(H), static_cast<int>(W), theta, st) !=
      hipSuccess)
    return WAN_E_HIP;
  for (int64_t r0 = 0; r0 < z.rows; r0 += kMaxRowsPerLaunch) {
    const int64_t n = z.rows - r0 < kMaxRowsPerLaunch ? z.rows - r0 : kMaxRowsPerLaunch;
    if (wan::launch_qknorm_rope(qkv, gamma_q, gamma_k, tab, r0, n, static_cast<int>(z.S), static_cast<int>(T),
                                static_cast<int>(H), static_cast<int>(W), static_cast<int>(z.D), eps, nullptr,
                                st) != hipSuccess)
      return WAN_E_HIP;
  }
  return WAN_OK;
}
