// Host-side launchers of the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wan {

// Q/K RMSNorm + bf16 + 3-D RoPE, in place, rows [row0, row0 + rows) of the
// packed buffer. `tab` holds the fp32 (cos, sin) pairs: frame axis [T][22],
// then row axis [H][21], then column axis [W][21].
hipError_t launch_qknorm_rope(void* qkv, const void* gq, const void* gk, const float2* tab,
                              int64_t row0, int64_t rows, int S, int T, int H, int W, int D,
                              float eps, hipStream_t stream);

// bf16 attention forward over the packed buffer.
hipError_t launch_attn_fwd(const void* qkv, void* out, float* lse, int B, int S, int heads,
                           float softmax_scale, hipStream_t stream);

}  // namespace wan
