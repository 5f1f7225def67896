"""GPU parity of wan_qknorm_rope_quant_fp8_delayed, the single-pass fp8
producer with delayed per-tensor scales, against the oracle
(oracle/wan_ref.py ``quant_fp8_delayed_ref``) and against the current-scale
two-call path (wan_qknorm_rope, then wan_qkv_quant_fp8): every e4m3 byte, the
scales used and the reported amax bit-exact; the packed input untouched."""

import numpy as np
import pytest
import torch

from oracle import wan_ref
from oracle.numerics import e4m3_encode, e4m3_rne_sat, f32
from video_diffusion_transformer_amd import synth, wan_attn
from video_diffusion_transformer_amd.configs import WORKLOADS

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _vt(f, heads):
    return f.vt8.view(f.B, heads, 128, f.s_pad)


def _setup(B, grid, heads, seed, device_gen=False):
    T, H, W = grid
    S = T * H * W
    qkv = synth.make_qkv(B, S, heads, seed=seed, device=DEV if device_gen else "cpu").to(DEV)
    gq, gk = synth.make_gammas(heads * 128, seed=seed, device=DEV)
    return qkv, gq, gk


@pytest.mark.parametrize("B,grid,heads,prev", [(1, (2, 8, 8), 2, (2.0, 3.5, 4.0)), (2, (3, 5, 7), 3, (0.5, 0.25, 1.0)),
                                               (1, (1, 1, 1), 1, (0.0, 0.0, 0.0)), (2, (2, 3, 5), 40, (6.0, 9.0, 5.0))])
def test_matches_oracle(B, grid, heads, prev):
    """Bytes, scales and amax against the oracle. amax_prev values below the
    data's amax saturate part of each tensor; 0 gives scale 1. Where the
    kernel's bf16 norm output sits on the other side of a rounding tie than the
    oracle's (the norm tests accept both), the byte is checked against the
    e4m3 rounding of the kernel's own value instead."""
    qkv, gq, gk = _setup(B, grid, heads, seed=sum(grid) + heads)
    D = heads * 128
    S = qkv.shape[1]
    before = qkv.clone()
    amax_prev = torch.tensor(prev, dtype=torch.float32, device=DEV)
    f = wan_attn.qknorm_rope_quant_fp8_delayed(qkv, gq, gk, grid, heads, amax_prev)
    normed = qkv.clone()
    wan_attn.qknorm_rope(normed, gq, gk, grid, heads)   # the kernel's own bf16 Q, K
    torch.cuda.synchronize()
    assert torch.equal(qkv, before), "the packed input must not be written"
    ref = wan_ref.quant_fp8_delayed_ref(_np(qkv), _np(gq), _np(gk), grid, heads, 128, list(prev))
    np.testing.assert_array_equal(f.scales.cpu().numpy().astype(np.float64), ref["scale"])
    g = _np(normed)
    own = [np.abs(g[..., i * D:(i + 1) * D]).max() for i in range(3)]
    np.testing.assert_array_equal(f.amax.cpu().numpy().astype(np.float64), own)
    np.testing.assert_allclose(own, ref["amax"], rtol=2.0 ** -8)
    qk = f.qk8.cpu().numpy()
    r16 = wan_ref.qknorm_rope_ref(_np(qkv), _np(gq), _np(gk), grid, heads, 128)
    oracle16 = np.concatenate([r16["out16_q"], r16["out16_k"]], axis=1).reshape(B, S, 2 * D)
    same = g[..., :2 * D] == oracle16
    assert same.mean() >= 0.9999
    np.testing.assert_array_equal(qk[same], ref["codes"][..., :2 * D][same])
    scales = np.repeat(ref["scale"][:2], D)
    own_codes = e4m3_encode(e4m3_rne_sat(f32(g[..., :2 * D] * scales)))
    np.testing.assert_array_equal(qk, own_codes)
    vt = _vt(f, heads).cpu().numpy()
    np.testing.assert_array_equal(vt[..., :S], ref["codes"][..., 2 * D:].reshape(B, S, heads, 128).transpose(0, 2, 3, 1))
    assert not vt[..., S:].any(), "padding past S must be zero"


def _two_call(qkv, gq, gk, grid, heads):
    a = qkv.clone()
    wan_attn.qknorm_rope(a, gq, gk, grid, heads)
    return wan_attn.qkv_quant_fp8(a, heads)


@pytest.mark.parametrize("B,grid,heads", [(1, (2, 8, 8), 2), (2, (1, 5, 21), 3), (2, (3, 7, 11), 40)])
def test_true_amax_equals_two_call_path(B, grid, heads):
    """With amax_prev = the data's own amax (as the two-call path reports it),
    every output equals the current-scale two-call path's."""
    qkv, gq, gk = _setup(B, grid, heads, seed=5 * heads + B)
    ref = _two_call(qkv, gq, gk, grid, heads)
    f = wan_attn.qknorm_rope_quant_fp8_delayed(qkv, gq, gk, grid, heads, ref.amax.clone())
    torch.cuda.synchronize()
    for name in ("amax", "scales", "qk8"):
        assert torch.equal(getattr(f, name), getattr(ref, name)), name
    assert torch.equal(_vt(f, heads), _vt(ref, heads))


def test_delayed_loop_reaches_current_scaling_in_one_call():
    """A first call with a guessed amax reports the data's amax; the next call
    on the same data with that amax equals the current-scale path (delayed
    scaling on static data converges after one call)."""
    grid, heads = (3, 6, 10), 4
    qkv, gq, gk = _setup(2, grid, heads, seed=77)
    guess = torch.ones(3, dtype=torch.float32, device=DEV)
    f1 = wan_attn.qknorm_rope_quant_fp8_delayed(qkv, gq, gk, grid, heads, guess)
    f2 = wan_attn.qknorm_rope_quant_fp8_delayed(qkv, gq, gk, grid, heads, f1.amax)
    ref = _two_call(qkv, gq, gk, grid, heads)
    torch.cuda.synchronize()
    assert torch.equal(f1.amax, ref.amax)
    for name in ("amax", "scales", "qk8"):
        assert torch.equal(getattr(f2, name), getattr(ref, name)), name
    assert torch.equal(_vt(f2, heads), _vt(ref, heads))


def test_720p_equals_two_call_path():
    """The 720p fp8 workload, in the launch configuration the benchmark
    times: bytes, scales and amax equal to the two-call path's, and the fp8
    attention of both buffer sets gives the same bits."""
    w = WORKLOADS["720p_fp8"]
    grid = (w.T, w.H, w.W)
    qkv, gq, gk = _setup(w.B, grid, w.heads, seed=w.seed, device_gen=True)
    ref = _two_call(qkv, gq, gk, grid, w.heads)
    f = wan_attn.qknorm_rope_quant_fp8_delayed(qkv, gq, gk, grid, w.heads, ref.amax.clone())
    torch.cuda.synchronize()
    for name in ("amax", "scales", "qk8"):
        assert torch.equal(getattr(f, name), getattr(ref, name)), name
    assert torch.equal(_vt(f, w.heads), _vt(ref, w.heads))


def test_errors():
    grid, heads = (1, 2, 4), 1
    qkv, gq, gk = _setup(1, grid, heads, seed=3)
    f = wan_attn.fp8_buffers(1, 8, heads, DEV)
    with pytest.raises(wan_attn.WanError) as e:  # amax_prev is the buffer this call clears and writes
        wan_attn.qknorm_rope_quant_fp8_delayed(qkv, gq, gk, grid, heads, f.amax, out=f)
    assert e.value.status == -5
    with pytest.raises(wan_attn.WanError) as e:  # ... or the scales it writes
        wan_attn.qknorm_rope_quant_fp8_delayed(qkv, gq, gk, grid, heads, f.scales, out=f)
    assert e.value.status == -5
    with pytest.raises(wan_attn.WanError) as e:
        wan_attn.qknorm_rope_quant_fp8_delayed(qkv, gq, gk, grid, heads, torch.ones(3, device=DEV), eps=-1.0)
    assert e.value.status == -9
