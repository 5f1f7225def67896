"""CPU checks of the boundary: the built library loads and exports every
symbol the header declares, the argument validation rejects every bad call
before touching memory (host-only C++ test), and the host-side token-grid
helper matches the pages' worked examples."""

import ctypes
import json
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wan_attn.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int64_t|int|const char \*)\s*(wan_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("wan_qknorm_rope", "wan_attn_fwd", "wan_status_str", "wan_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from video_diffusion_transformer_amd import wan_attn
    if not os.path.exists(wan_attn.LIB_PATH):
        pytest.skip("library not built")
    lib = ctypes.CDLL(wan_attn.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(wan_attn.SIGNATURES), "binding and header disagree"
    lib.wan_abi_version.restype = ctypes.c_int
    assert lib.wan_abi_version() == 1
    lib.wan_status_str.restype = ctypes.c_char_p
    assert lib.wan_status_str(-5) == b"an output overlaps an input"


@pytest.mark.parametrize("flags", [["-O1"], ["-O3", "-ffinite-math-only"]])
def test_validation_rejects_bad_calls_host_only(tmp_path, flags):
    """The host-only validation test, also built with finite-math assumptions
    (the NaN checks must survive them)."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "validate_test"
    src = os.path.join(ROOT, "tests", "csrc", "validate_test.cpp")
    subprocess.run([gxx, "-std=c++17", *flags, "-Wall", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "video_diffusion_transformer_amd", "csrc"), src, "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _built_lib():
    from video_diffusion_transformer_amd import wan_attn
    if not os.path.exists(wan_attn.LIB_PATH):
        pytest.skip("library not built")
    return wan_attn.lib()


def test_token_grid_through_the_c_abi_matches_worked_examples():
    """wan_token_grid (host arithmetic behind the C ABI) on the pages' worked
    examples, through the binding and through a raw ctypes call."""
    lib = _built_lib()
    from video_diffusion_transformer_amd.wan_attn import WanError, token_grid
    for c in json.load(open(os.path.join(ROOT, "tests", "golden", "output_spec.json")))["cases"]:
        assert token_grid(c["width"], c["height"], c["frames"]) == (c["T"], c["H"], c["W"])
        T, H, W = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        assert lib.wan_token_grid(c["width"], c["height"], c["frames"], ctypes.byref(T), ctypes.byref(H),
                                  ctypes.byref(W)) == 0
        assert T.value * H.value * W.value == c["S"]
    for bad in ((832, 480, 80), (832, 480, 0), (-16, 480, 81), (832, -1, 81)):
        with pytest.raises(WanError) as e:
            token_grid(*bad)
        assert e.value.status == -2, bad
    assert lib.wan_token_grid(832, 480, 81, None, None, None) == -1
    assert token_grid(15, 15, 1) == (1, 0, 0)  # below one token per axis: an empty grid


def test_nan_scalars_are_rejected_by_the_built_library():
    """The built library (not only the host test) refuses NaN eps, theta and
    softmax scale; B = 0 keeps every call free of device work."""
    lib = _built_lib()
    nan = float("nan")
    assert lib.wan_attn_fwd(None, None, None, 0, 16, 2, 128, nan, None) == -9
    assert lib.wan_attn_fwd_fp8(None, None, None, None, None, 0, 16, 2, 128, nan, None) == -9
    assert lib.wan_attn_fwd_chunk(None, 16, None, 16, None, None, 0, 2, 128, nan, None) == -9
    assert lib.wan_attn_fwd_chunk_merge(None, 16, None, 16, None, None, None, 0, 2, 128, nan, None) == -9
    assert lib.wan_qknorm_rope(None, None, None, 0, 2, 8, 8, 2, 128, nan, 1e4, None) == -9
    assert lib.wan_qknorm_rope(None, None, None, 0, 2, 8, 8, 2, 128, 1e-6, nan, None) == -9
    assert lib.wan_qknorm_rope_quant_fp8(None, None, None, 0, 2, 8, 8, 2, 128, 1e-6, nan, None, None, None, None,
                                         None) == -9
    assert lib.wan_attn_fwd(None, None, None, 0, 16, 2, 128, 0.088, None) == 0
    assert lib.wan_qkv_proj_norm_rope(None, None, None, None, None, None, None, 0, 0, 2, 8, 8, 2, 128, nan, 1e4,
                                      None) == -9
    assert lib.wan_qkv_proj_norm_rope(None, None, None, None, None, None, None, 0, 0, 2, 8, 8, 2, 128, 1e-6, nan,
                                      None) == -9
    assert lib.wan_qkv_proj_norm_rope(None, None, None, None, None, None, None, 0, 0, 2, 8, 8, 2, 128, 1e-6, 1e4,
                                      None) == 0


def test_fused_projection_workspace_size():
    """wan_qkv_proj_norm_rope_workspace_bytes (pure host arithmetic): 256
    control bytes, two arrival counts per 256-token block rounded up to 256
    bytes, then 2*heads 8-byte words per token; -1 for invalid sizes."""
    lib = _built_lib()
    f = lib.wan_qkv_proj_norm_rope_workspace_bytes
    assert f(1, 16, 2, 128) == 256 + 256 + 16 * 2 * 2 * 8
    assert f(2, 32760, 40, 128) == 256 + ((8 * 256 + 255) // 256) * 256 + 65520 * 80 * 8
    assert f(0, 0, 1, 128) == 256  # no token blocks: the control bytes only
    assert f(1, 16, 2, 64) == -1 and f(-1, 16, 2, 128) == -1 and f(1, 16, 0, 128) == -1
    assert f(1 << 40, 1 << 30, 40, 128) == -1  # overflow


def test_fp8_binding_checks_buffer_and_output_shapes():
    """The fp8 attention binding refuses short or mismatched buffers and
    outputs before any call into the library (meta tensors: shapes only)."""
    _built_lib()
    import torch
    from video_diffusion_transformer_amd import wan_attn
    B, S, heads = 2, 300, 3
    D = heads * 128

    def buffers(qk_n=B * S * 2 * D, vt_n=None, sc_n=3):
        vt_n = wan_attn.lib().wan_fp8_vt_bytes(B, S, heads, 128) if vt_n is None else vt_n
        m = dict(device="meta")
        return wan_attn.Fp8QKV(torch.empty(qk_n, dtype=torch.uint8, **m), torch.empty(vt_n, dtype=torch.uint8, **m),
                               torch.empty(sc_n, dtype=torch.float32, **m), torch.empty(3, dtype=torch.float32, **m),
                               B, S, heads)

    wan_attn.check_fp8_buffers(buffers(), B, S, heads)
    for bad in (buffers(qk_n=B * S * 2 * D - 1), buffers(vt_n=100), buffers(sc_n=2)):
        with pytest.raises(ValueError):
            wan_attn.check_fp8_buffers(bad, B, S, heads)
    with pytest.raises(ValueError):  # buffers made for other sizes
        wan_attn.check_fp8_buffers(buffers(), B, S + 1, heads)
    out = torch.empty((B, S, D), dtype=torch.bfloat16, device="meta")
    lse = torch.empty((B, heads, S), dtype=torch.float32, device="meta")
    wan_attn.check_attn_outputs(out, lse, B, S, heads)
    wan_attn.check_attn_outputs(out, None, B, S, heads)
    with pytest.raises(ValueError):
        wan_attn.check_attn_outputs(out[:, :S - 1], lse, B, S, heads)
    with pytest.raises(ValueError):
        wan_attn.check_attn_outputs(out, lse[:, :, :S - 1], B, S, heads)
    with pytest.raises(ValueError):
        wan_attn.check_attn_outputs(out.float(), lse, B, S, heads)
    with pytest.raises(ValueError, match="out must be"):  # the check inside attn_fwd_fp8 itself
        wan_attn.attn_fwd_fp8(buffers(), out=torch.empty((B, S - 1, D), dtype=torch.bfloat16, device="meta"))
    with pytest.raises(ValueError, match="qk8 must hold"):
        wan_attn.attn_fwd_fp8(buffers(qk_n=10))


def test_binding_refuses_cpu_tensors():
    import torch
    from video_diffusion_transformer_amd import wan_attn
    x = torch.zeros((1, 4, 768), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        wan_attn.attn_fwd(x, 2)
    with pytest.raises(ValueError):
        wan_attn.qknorm_rope(x, x[0, 0, :256], x[0, 0, :256], (1, 2, 2), 2)
