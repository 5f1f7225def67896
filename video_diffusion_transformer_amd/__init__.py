"""MI355X-native (gfx950) hot path of one Wan2.2 DiT self-attention step.

The computation lives in libwan_attn.so (hand-written HIP kernels behind the
C ABI in include/wan_attn.h); this package holds the ctypes binding, the build
script, the workload definitions and the seeded input generators.
"""

from .wan_attn import (Fp8QKV, WanError, attn_fwd, attn_fwd_chunk, attn_fwd_chunk_merge, attn_fwd_fp8, attn_fwd_skip,  # noqa: F401
                       attn_merge, fp8_buffers, lib, qknorm_rope, qknorm_rope_quant_fp8,
                       qknorm_rope_quant_fp8_delayed, qkv_proj, qkv_proj_norm_rope,
                       qkv_proj_norm_rope_workspace_bytes, qkv_quant_fp8, token_grid)
from .configs import WORKLOADS, Workload  # noqa: F401
