"""Python binding of libwan_attn.so (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/wan_attn.h. Tensors must already
live on the GPU; there is no CPU path. If the library is not built the first
call raises -- nothing falls back to another implementation.

The names follow the C ABI: ``token_grid`` -> wan_token_grid, ``qkv_proj`` -> wan_qkv_proj,
``qknorm_rope`` -> wan_qknorm_rope, ``qkv_proj_norm_rope`` -> wan_qkv_proj_norm_rope, ``attn_fwd`` -> wan_attn_fwd, ``attn_fwd_skip`` -> wan_attn_fwd_skip,
``attn_fwd_chunk`` -> wan_attn_fwd_chunk, ``attn_merge`` -> wan_attn_merge,
``attn_fwd_chunk_merge`` -> wan_attn_fwd_chunk_merge,
``qkv_quant_fp8`` -> wan_qkv_quant_fp8,
``qknorm_rope_quant_fp8`` -> wan_qknorm_rope_quant_fp8,
``qknorm_rope_quant_fp8_delayed`` -> wan_qknorm_rope_quant_fp8_delayed, ``attn_fwd_fp8`` -> wan_attn_fwd_fp8.
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwan_attn.so")

HEAD_DIM = 128
RMS_EPS = 1e-6
ROPE_THETA = 10000.0

_STATUS = {
    0: "WAN_OK", -1: "WAN_E_NULL", -2: "WAN_E_SHAPE", -3: "WAN_E_UNSUPPORTED", -4: "WAN_E_ALIGN",
    -5: "WAN_E_ALIAS", -6: "WAN_E_OVERFLOW", -7: "WAN_E_HIP", -8: "WAN_E_NOMEM", -9: "WAN_E_VALUE",
    -10: "WAN_E_LIMIT",
}

# (name, restype, argtypes) of every symbol the header declares.
_P, _I64, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
SIGNATURES = {
    "wan_abi_version": (ctypes.c_int, []),
    "wan_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "wan_token_grid": (ctypes.c_int, [_I64, _I64, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                                      ctypes.POINTER(_I64)]),
    "wan_qkv_proj": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]),
    "wan_qknorm_rope": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _F, _F, _P]),
    "wan_qkv_proj_norm_rope": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                              _F, _F, _P]),
    "wan_qkv_proj_norm_rope_workspace_bytes": (ctypes.c_int64, [_I64, _I64, _I64, _I64]),
    "wan_qknorm_rope_noalloc": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _F, _F, _P]),
    "wan_attn_fwd": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _F, _P]),
    "wan_attn_fwd_skip": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _F, _P]),
    "wan_attn_skip_map_bytes": (ctypes.c_int64, [_I64, _I64, _I64, _I64]),
    "wan_attn_fwd_chunk": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P, _I64, _I64, _I64, _F, _P]),
    "wan_attn_merge": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]),
    "wan_attn_fwd_chunk_merge": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _F, _P]),
    "wan_qkv_quant_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]),
    "wan_qknorm_rope_quant_fp8": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _F, _F,
                                                 _P, _P, _P, _P, _P]),
    "wan_qknorm_rope_quant_fp8_delayed": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _F, _F,
                                                         _P, _P, _P, _P, _P, _P]),
    "wan_fp8_vt_bytes": (ctypes.c_int64, [_I64, _I64, _I64, _I64]),
    "wan_attn_fwd_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _P]),
}


class WanError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} ({text})")
        self.status = status


_lib = None


def lib():
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m video_diffusion_transformer_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def _check(fn, status):
    if status != 0:
        raise WanError(fn, status, lib().wan_status_str(status).decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need_gpu(name, t, dtype):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def token_grid(width, height, num_frames):
    """(T, H, W) token grid of a clip of width x height pixels and num_frames
    frames, from wan_token_grid. Raises WanError on invalid sizes."""
    T, H, W = _I64(), _I64(), _I64()
    _check("wan_token_grid", lib().wan_token_grid(width, height, num_frames, ctypes.byref(T), ctypes.byref(H),
                                                  ctypes.byref(W)))
    return T.value, H.value, W.value


def qkv_proj(x, w_qkv, heads, bias=None, head_dim=HEAD_DIM, out=None, stream=None):
    """Packed [B, S, 3D] bf16 = x [B, S, D] w_qkv^T (+ bias), w_qkv [3D, D].
    Returns the output tensor (allocated unless ``out`` is given)."""
    D = heads * head_dim
    _need_gpu("x", x, torch.bfloat16)
    _need_gpu("w_qkv", w_qkv, torch.bfloat16)
    if bias is not None:
        _need_gpu("bias", bias, torch.bfloat16)
        if bias.numel() != 3 * D:
            raise ValueError("bias must have 3*heads*head_dim elements")
    if x.dim() != 3 or x.shape[2] != D or tuple(w_qkv.shape) != (3 * D, D):
        raise ValueError("x must be [B, S, heads*head_dim] and w_qkv [3*D, D]")
    B, S = x.shape[0], x.shape[1]
    out = torch.empty((B, S, 3 * D), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need_gpu("out", out, torch.bfloat16)
    if tuple(out.shape) != (B, S, 3 * D):
        raise ValueError("out must be [B, S, 3*D]")
    with torch.cuda.device(x.device):
        _check("wan_qkv_proj", lib().wan_qkv_proj(
            _ptr(x), _ptr(w_qkv), _ptr(bias), _ptr(out), B, S, heads, head_dim, _stream(x.device, stream)))
    return out


def qknorm_rope(qkv, gamma_q, gamma_k, grid, heads, head_dim=HEAD_DIM, eps=RMS_EPS,
                theta=ROPE_THETA, stream=None):
    """In-place Q/K RMSNorm + bf16 rounding + 3-D RoPE on a packed
    [B, S, 3*heads*head_dim] bf16 tensor (S = T*H*W). Returns qkv."""
    T, H, W = grid
    _need_gpu("qkv", qkv, torch.bfloat16)
    _need_gpu("gamma_q", gamma_q, torch.bfloat16)
    _need_gpu("gamma_k", gamma_k, torch.bfloat16)
    B = qkv.shape[0]
    D = heads * head_dim
    if qkv.dim() != 3 or qkv.shape[1] != T * H * W or qkv.shape[2] != 3 * D:
        raise ValueError(f"qkv must be [B, {T * H * W}, {3 * D}], got {tuple(qkv.shape)}")
    if gamma_q.numel() != D or gamma_k.numel() != D:
        raise ValueError("gammas must have heads*head_dim elements")
    with torch.cuda.device(qkv.device):
        _check("wan_qknorm_rope", lib().wan_qknorm_rope(
            _ptr(qkv), _ptr(gamma_q), _ptr(gamma_k), B, T, H, W, heads, head_dim, eps, theta,
            _stream(qkv.device, stream)))
    return qkv


def qkv_proj_norm_rope_workspace_bytes(B, S, heads, head_dim=HEAD_DIM):
    n = lib().wan_qkv_proj_norm_rope_workspace_bytes(B, S, heads, head_dim)
    if n < 0:
        raise ValueError("invalid sizes for the projection + norm + RoPE workspace")
    return n


def qkv_proj_norm_rope(x, w_qkv, gamma_q, gamma_k, grid, heads, bias=None, head_dim=HEAD_DIM, eps=RMS_EPS,
                       theta=ROPE_THETA, out=None, workspace=None, stream=None):
    """Packed [B, S, 3D] bf16 of the projection x w_qkv^T (+ bias) with the Q/K
    RMSNorm + 3-D RoPE applied in the epilogue (S = T*H*W). ``workspace`` is a
    uint8 device tensor of at least qkv_proj_norm_rope_workspace_bytes(B, S,
    heads) bytes (allocated when None). Returns (out, workspace); byte 4..7 of
    the workspace is the error word (nonzero after a wait hit its spin limit)."""
    T, H, W = grid
    D = heads * head_dim
    for name, t in (("x", x), ("w_qkv", w_qkv), ("gamma_q", gamma_q), ("gamma_k", gamma_k)):
        _need_gpu(name, t, torch.bfloat16)
    if bias is not None:
        _need_gpu("bias", bias, torch.bfloat16)
        if bias.numel() != 3 * D:
            raise ValueError("bias must have 3*heads*head_dim elements")
    if x.dim() != 3 or x.shape[1] != T * H * W or x.shape[2] != D or tuple(w_qkv.shape) != (3 * D, D):
        raise ValueError(f"x must be [B, {T * H * W}, {D}] and w_qkv [3*D, D]")
    if gamma_q.numel() != D or gamma_k.numel() != D:
        raise ValueError("gammas must have heads*head_dim elements")
    B, S = x.shape[0], x.shape[1]
    out = torch.empty((B, S, 3 * D), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need_gpu("out", out, torch.bfloat16)
    if tuple(out.shape) != (B, S, 3 * D):
        raise ValueError("out must be [B, S, 3*D]")
    if workspace is None:
        workspace = torch.empty(qkv_proj_norm_rope_workspace_bytes(B, S, heads, head_dim), dtype=torch.uint8,
                                device=x.device)
    _need_gpu("workspace", workspace, torch.uint8)
    with torch.cuda.device(x.device):
        _check("wan_qkv_proj_norm_rope", lib().wan_qkv_proj_norm_rope(
            _ptr(x), _ptr(w_qkv), _ptr(bias), _ptr(gamma_q), _ptr(gamma_k), _ptr(out), _ptr(workspace),
            workspace.numel(), B, T, H, W, heads, head_dim, eps, theta, _stream(x.device, stream)))
    return out, workspace


def proj_norm_rope_error_word(workspace):
    """The workspace's error word (synchronises with the device)."""
    return int(workspace[4:8].view(torch.int32).item())


def attn_fwd(qkv, heads, head_dim=HEAD_DIM, softmax_scale=None, out=None, lse=False, stream=None):
    """Bidirectional attention over a packed bf16 [B, S, 3*D] tensor.
    Returns out [B, S, D] bf16, or (out, lse [B, heads, S] fp32) when lse is
    True or a preallocated tensor."""
    _need_gpu("qkv", qkv, torch.bfloat16)
    B, S = qkv.shape[0], qkv.shape[1]
    D = heads * head_dim
    if qkv.dim() != 3 or qkv.shape[2] != 3 * D:
        raise ValueError(f"qkv must be [B, S, {3 * D}], got {tuple(qkv.shape)}")
    scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, S, D), dtype=torch.bfloat16, device=qkv.device)
    _need_gpu("out", out, torch.bfloat16)
    if tuple(out.shape) != (B, S, D):
        raise ValueError("out must be [B, S, D]")
    want_lse = lse is not False and lse is not None
    if lse is True:
        lse = torch.empty((B, heads, S), dtype=torch.float32, device=qkv.device)
    if want_lse:
        _need_gpu("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, heads, S):
            raise ValueError("lse must be [B, heads, S]")
    with torch.cuda.device(qkv.device):
        _check("wan_attn_fwd", lib().wan_attn_fwd(
            _ptr(qkv), _ptr(out), _ptr(lse) if want_lse else ctypes.c_void_p(0), B, S, heads,
            head_dim, scale, _stream(qkv.device, stream)))
    return (out, lse) if want_lse else out


SKIP_BLOCK_Q, SKIP_BLOCK_K = 48, 64  # WAN_SKIP_BLOCK_Q, WAN_SKIP_BLOCK_K of the header


def attn_fwd_skip(qkv, heads, threshold, head_dim=HEAD_DIM, softmax_scale=None, out=None, lse=False, kept=False,
                  stream=None):
    """Attention with Skip-Softmax in threshold mode over a packed bf16
    [B, S, 3*D] tensor. Returns out, followed by lse [B, heads, S] and/or the
    decision map kept [B, heads, ceil(S/48), ceil(S/64)] (uint8, 1 = kept)
    when those are requested (True or a preallocated tensor)."""
    _need_gpu("qkv", qkv, torch.bfloat16)
    B, S = qkv.shape[0], qkv.shape[1]
    D = heads * head_dim
    if qkv.dim() != 3 or qkv.shape[2] != 3 * D:
        raise ValueError(f"qkv must be [B, S, {3 * D}], got {tuple(qkv.shape)}")
    scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, S, D), dtype=torch.bfloat16, device=qkv.device)
    want_lse = lse is not False and lse is not None
    if lse is True:
        lse = torch.empty((B, heads, S), dtype=torch.float32, device=qkv.device)
    check_attn_outputs(out, lse if want_lse else None, B, S, heads, head_dim)
    _need_gpu("out", out, torch.bfloat16)
    if want_lse:
        _need_gpu("lse", lse, torch.float32)
    want_kept = kept is not False and kept is not None
    map_shape = (B, heads, -(-S // SKIP_BLOCK_Q), -(-S // SKIP_BLOCK_K))
    if kept is True:
        kept = torch.empty(map_shape, dtype=torch.uint8, device=qkv.device)
    if want_kept:
        _need_gpu("kept", kept, torch.uint8)
        if tuple(kept.shape) != map_shape:
            raise ValueError(f"kept must be {map_shape}")
    with torch.cuda.device(qkv.device):
        _check("wan_attn_fwd_skip", lib().wan_attn_fwd_skip(
            _ptr(qkv), _ptr(out), _ptr(lse) if want_lse else ctypes.c_void_p(0),
            _ptr(kept) if want_kept else ctypes.c_void_p(0), B, S, heads, head_dim, scale, float(threshold),
            _stream(qkv.device, stream)))
    res = (out,) + ((lse,) if want_lse else ()) + ((kept,) if want_kept else ())
    return res[0] if len(res) == 1 else res


def attn_fwd_chunk(q_src, kv_src, heads, head_dim=HEAD_DIM, softmax_scale=None, out=None, lse=None, stream=None):
    """Queries of q_src [B, Sq, 3D] against the keys/values of kv_src
    [B, Skv, 3D] (both packed bf16). Returns (out fp32 [B, Sq, D],
    lse fp32 [B, heads, Sq])."""
    _need_gpu("q_src", q_src, torch.bfloat16)
    _need_gpu("kv_src", kv_src, torch.bfloat16)
    B, Sq, Skv = q_src.shape[0], q_src.shape[1], kv_src.shape[1]
    D = heads * head_dim
    if q_src.dim() != 3 or kv_src.dim() != 3 or q_src.shape[2] != 3 * D or kv_src.shape[2] != 3 * D \
            or kv_src.shape[0] != B:
        raise ValueError("q_src and kv_src must be [B, S, 3*heads*head_dim] with the same B")
    scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else float(softmax_scale)
    dev = q_src.device
    out = torch.empty((B, Sq, D), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, heads, Sq), dtype=torch.float32, device=dev) if lse is None else lse
    _need_gpu("out", out, torch.float32)
    _need_gpu("lse", lse, torch.float32)
    if tuple(out.shape) != (B, Sq, D) or tuple(lse.shape) != (B, heads, Sq):
        raise ValueError("out must be [B, Sq, D] and lse [B, heads, Sq]")
    with torch.cuda.device(dev):
        _check("wan_attn_fwd_chunk", lib().wan_attn_fwd_chunk(
            _ptr(q_src), Sq, _ptr(kv_src), Skv, _ptr(out), _ptr(lse), B, heads, head_dim, scale,
            _stream(dev, stream)))
    return out, lse


def attn_merge(acc_out, acc_lse, chunk_out, chunk_lse, heads, head_dim=HEAD_DIM, out_bf16=None, stream=None):
    """Fold (chunk_out, chunk_lse) into (acc_out, acc_lse) in place; optionally
    also write the merged output as bf16 into out_bf16."""
    for name, t in (("acc_out", acc_out), ("acc_lse", acc_lse), ("chunk_out", chunk_out), ("chunk_lse", chunk_lse)):
        _need_gpu(name, t, torch.float32)
    B, Sq = acc_out.shape[0], acc_out.shape[1]
    D = heads * head_dim
    for t in (acc_out, chunk_out):
        if tuple(t.shape) != (B, Sq, D):
            raise ValueError("outputs must be [B, Sq, heads*head_dim]")
    for t in (acc_lse, chunk_lse):
        if tuple(t.shape) != (B, heads, Sq):
            raise ValueError("lse tensors must be [B, heads, Sq]")
    if out_bf16 is not None:
        _need_gpu("out_bf16", out_bf16, torch.bfloat16)
        if tuple(out_bf16.shape) != (B, Sq, D):
            raise ValueError("out_bf16 must be [B, Sq, D]")
    dev = acc_out.device
    with torch.cuda.device(dev):
        _check("wan_attn_merge", lib().wan_attn_merge(
            _ptr(acc_out), _ptr(acc_lse), _ptr(chunk_out), _ptr(chunk_lse), _ptr(out_bf16), B, Sq, heads,
            head_dim, _stream(dev, stream)))
    return acc_out, acc_lse


def attn_fwd_chunk_merge(q_src, kv_src, acc_out, acc_lse, heads, head_dim=HEAD_DIM, softmax_scale=None,
                         out_bf16=None, stream=None):
    """One ring round folded into (acc_out, acc_lse) in place: attention of
    the queries of q_src over the chunk kv_src, merged as attn_merge would.
    Returns (acc_out, acc_lse)."""
    _need_gpu("q_src", q_src, torch.bfloat16)
    _need_gpu("kv_src", kv_src, torch.bfloat16)
    _need_gpu("acc_out", acc_out, torch.float32)
    _need_gpu("acc_lse", acc_lse, torch.float32)
    B, Sq, Skv = q_src.shape[0], q_src.shape[1], kv_src.shape[1]
    D = heads * head_dim
    if q_src.dim() != 3 or kv_src.dim() != 3 or q_src.shape[2] != 3 * D or kv_src.shape[2] != 3 * D \
            or kv_src.shape[0] != B:
        raise ValueError("q_src and kv_src must be [B, S, 3*heads*head_dim] with the same B")
    if tuple(acc_out.shape) != (B, Sq, D) or tuple(acc_lse.shape) != (B, heads, Sq):
        raise ValueError("acc_out must be [B, Sq, D] and acc_lse [B, heads, Sq]")
    if out_bf16 is not None:
        _need_gpu("out_bf16", out_bf16, torch.bfloat16)
        if tuple(out_bf16.shape) != (B, Sq, D):
            raise ValueError("out_bf16 must be [B, Sq, D]")
    scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else float(softmax_scale)
    dev = q_src.device
    with torch.cuda.device(dev):
        _check("wan_attn_fwd_chunk_merge", lib().wan_attn_fwd_chunk_merge(
            _ptr(q_src), Sq, _ptr(kv_src), Skv, _ptr(acc_out), _ptr(acc_lse), _ptr(out_bf16), B, heads, head_dim,
            scale, _stream(dev, stream)))
    return acc_out, acc_lse


class Fp8QKV:
    """Outputs of qkv_quant_fp8: qk8 [B, S, 2D] and vt8 [B, heads, 128, S_pad]
    e4m3 bytes (uint8 tensors), per-tensor scales and amax (fp32 [3])."""

    def __init__(self, qk8, vt8, scales, amax, B, S, heads):
        self.qk8, self.vt8, self.scales, self.amax = qk8, vt8, scales, amax
        self.B, self.S, self.heads = B, S, heads

    @property
    def s_pad(self):
        return (self.S + 127) // 128 * 128


def check_fp8_buffers(f, B, S, heads, head_dim=HEAD_DIM):
    """Sizes of the buffers of an Fp8QKV against (B, S, heads): the C ABI cannot
    see buffer sizes, so a short or mismatched buffer is refused here. Checks
    shapes and dtypes only (works on tensors of any device)."""
    D = heads * head_dim
    if (f.B, f.S, f.heads) != (B, S, heads):
        raise ValueError(f"fp8 buffers are for (B, S, heads) = {(f.B, f.S, f.heads)}, not {(B, S, heads)}")
    for name, t, dt in (("qk8", f.qk8, torch.uint8), ("vt8", f.vt8, torch.uint8), ("scales", f.scales, torch.float32),
                        ("amax", f.amax, torch.float32)):
        if not isinstance(t, torch.Tensor) or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor")
    if f.qk8.numel() != B * S * 2 * D:
        raise ValueError(f"qk8 must hold B*S*2*D = {B * S * 2 * D} bytes, got {f.qk8.numel()}")
    vt_need = lib().wan_fp8_vt_bytes(B, S, heads, head_dim)
    if vt_need < 0 or f.vt8.numel() < vt_need:
        raise ValueError(f"vt8 must hold {vt_need} bytes, got {f.vt8.numel()}")
    if f.scales.numel() != 3 or f.amax.numel() != 3:
        raise ValueError("scales and amax must hold 3 floats each")


def check_attn_outputs(out, lse, B, S, heads, head_dim=HEAD_DIM):
    """out must be a contiguous bf16 [B, S, D] tensor and lse (if not None) a
    contiguous fp32 [B, heads, S] one; shapes and dtypes only."""
    D = heads * head_dim
    if not isinstance(out, torch.Tensor) or out.dtype != torch.bfloat16 or tuple(out.shape) != (B, S, D) \
            or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bf16 tensor of shape {(B, S, D)}")
    if lse is not None and (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32
                            or tuple(lse.shape) != (B, heads, S) or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous fp32 tensor of shape {(B, heads, S)}")


def fp8_buffers(B, S, heads, device, head_dim=HEAD_DIM):
    """Allocate the buffers qkv_quant_fp8 writes."""
    D = heads * head_dim
    n = lib().wan_fp8_vt_bytes(B, S, heads, head_dim)
    if n < 0:
        raise ValueError("invalid sizes")
    return Fp8QKV(torch.empty((B, S, 2 * D), dtype=torch.uint8, device=device),
                  torch.empty(n, dtype=torch.uint8, device=device),
                  torch.empty(3, dtype=torch.float32, device=device),
                  torch.empty(3, dtype=torch.float32, device=device), B, S, heads)


def qkv_quant_fp8(qkv, heads, head_dim=HEAD_DIM, out=None, stream=None):
    """Per-tensor e4m3 quantisation of the packed bf16 [B, S, 3D] buffer.
    Returns an Fp8QKV (allocated unless ``out`` is given)."""
    _need_gpu("qkv", qkv, torch.bfloat16)
    B, S = qkv.shape[0], qkv.shape[1]
    if qkv.dim() != 3 or qkv.shape[2] != 3 * heads * head_dim:
        raise ValueError("qkv must be [B, S, 3*heads*head_dim]")
    f = out if out is not None else fp8_buffers(B, S, heads, qkv.device, head_dim)
    check_fp8_buffers(f, B, S, heads, head_dim)
    for name in ("qk8", "vt8"):
        _need_gpu(name, getattr(f, name), torch.uint8)
    _need_gpu("scales", f.scales, torch.float32)
    _need_gpu("amax", f.amax, torch.float32)
    with torch.cuda.device(qkv.device):
        _check("wan_qkv_quant_fp8", lib().wan_qkv_quant_fp8(
            _ptr(qkv), _ptr(f.qk8), _ptr(f.vt8), _ptr(f.scales), _ptr(f.amax), B, S, heads, head_dim,
            _stream(qkv.device, stream)))
    return f


def qknorm_rope_quant_fp8(qkv, gamma_q, gamma_k, grid, heads, head_dim=HEAD_DIM, eps=RMS_EPS, theta=ROPE_THETA,
                          out=None, stream=None):
    """qknorm_rope (in place) and then qkv_quant_fp8 of the result, with the
    amax folded into the norm pass. Returns an Fp8QKV (allocated unless
    ``out`` is given)."""
    T, H, W = grid
    for name, t in (("qkv", qkv), ("gamma_q", gamma_q), ("gamma_k", gamma_k)):
        _need_gpu(name, t, torch.bfloat16)
    B, D = qkv.shape[0], heads * head_dim
    S = T * H * W
    if qkv.dim() != 3 or qkv.shape[1] != S or qkv.shape[2] != 3 * D:
        raise ValueError(f"qkv must be [B, {S}, {3 * D}], got {tuple(qkv.shape)}")
    if gamma_q.numel() != D or gamma_k.numel() != D:
        raise ValueError("gammas must have heads*head_dim elements")
    f = out if out is not None else fp8_buffers(B, S, heads, qkv.device, head_dim)
    check_fp8_buffers(f, B, S, heads, head_dim)
    for name in ("qk8", "vt8"):
        _need_gpu(name, getattr(f, name), torch.uint8)
    _need_gpu("scales", f.scales, torch.float32)
    _need_gpu("amax", f.amax, torch.float32)
    with torch.cuda.device(qkv.device):
        _check("wan_qknorm_rope_quant_fp8", lib().wan_qknorm_rope_quant_fp8(
            _ptr(qkv), _ptr(gamma_q), _ptr(gamma_k), B, T, H, W, heads, head_dim, eps, theta,
            _ptr(f.qk8), _ptr(f.vt8), _ptr(f.scales), _ptr(f.amax), _stream(qkv.device, stream)))
    return f


def qknorm_rope_quant_fp8_delayed(qkv, gamma_q, gamma_k, grid, heads, amax_prev, head_dim=HEAD_DIM, eps=RMS_EPS,
                                  theta=ROPE_THETA, out=None, stream=None):
    """Single-pass fp8 producer with delayed scales: norm + RoPE of qkv (read
    only) quantised to e4m3 at the scales 448 / amax_prev (a device fp32 [3]
    tensor, e.g. the ``amax`` of an earlier call's Fp8QKV). Returns an Fp8QKV
    whose ``scales`` are the scales used and ``amax`` this call's amax
    (allocated unless ``out`` is given; its amax must not be amax_prev)."""
    T, H, W = grid
    for name, t in (("qkv", qkv), ("gamma_q", gamma_q), ("gamma_k", gamma_k)):
        _need_gpu(name, t, torch.bfloat16)
    _need_gpu("amax_prev", amax_prev, torch.float32)
    B, D = qkv.shape[0], heads * head_dim
    S = T * H * W
    if qkv.dim() != 3 or qkv.shape[1] != S or qkv.shape[2] != 3 * D:
        raise ValueError(f"qkv must be [B, {S}, {3 * D}], got {tuple(qkv.shape)}")
    if gamma_q.numel() != D or gamma_k.numel() != D:
        raise ValueError("gammas must have heads*head_dim elements")
    if amax_prev.numel() != 3:
        raise ValueError("amax_prev must hold 3 floats")
    f = out if out is not None else fp8_buffers(B, S, heads, qkv.device, head_dim)
    check_fp8_buffers(f, B, S, heads, head_dim)
    for name in ("qk8", "vt8"):
        _need_gpu(name, getattr(f, name), torch.uint8)
    _need_gpu("scales", f.scales, torch.float32)
    _need_gpu("amax", f.amax, torch.float32)
    with torch.cuda.device(qkv.device):
        _check("wan_qknorm_rope_quant_fp8_delayed", lib().wan_qknorm_rope_quant_fp8_delayed(
            _ptr(qkv), _ptr(gamma_q), _ptr(gamma_k), B, T, H, W, heads, head_dim, eps, theta, _ptr(amax_prev),
            _ptr(f.qk8), _ptr(f.vt8), _ptr(f.scales), _ptr(f.amax), _stream(qkv.device, stream)))
    return f


def attn_fwd_fp8(f, head_dim=HEAD_DIM, softmax_scale=None, out=None, lse=False, stream=None):
    """Attention from an Fp8QKV. Returns out [B, S, D] bf16 (and lse)."""
    B, S, heads = f.B, f.S, f.heads
    D = heads * head_dim
    check_fp8_buffers(f, B, S, heads, head_dim)
    scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else float(softmax_scale)
    dev = f.qk8.device
    if out is None:
        out = torch.empty((B, S, D), dtype=torch.bfloat16, device=dev)
    want_lse = lse is not False and lse is not None
    if lse is True:
        lse = torch.empty((B, heads, S), dtype=torch.float32, device=dev)
    check_attn_outputs(out, lse if want_lse else None, B, S, heads, head_dim)
    for name in ("qk8", "vt8"):
        _need_gpu(name, getattr(f, name), torch.uint8)
    _need_gpu("scales", f.scales, torch.float32)
    _need_gpu("out", out, torch.bfloat16)
    if want_lse:
        _need_gpu("lse", lse, torch.float32)
    with torch.cuda.device(dev):
        _check("wan_attn_fwd_fp8", lib().wan_attn_fwd_fp8(
            _ptr(f.qk8), _ptr(f.vt8), _ptr(f.scales), _ptr(out), _ptr(lse) if want_lse else ctypes.c_void_p(0),
            B, S, heads, head_dim, scale, _stream(dev, stream)))
    return (out, lse) if want_lse else out
