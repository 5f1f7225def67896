"""GPU parity of the fp8 path (wan_qkv_quant_fp8, wan_attn_fwd_fp8) against
the oracle: amax and scales exact, every e4m3 byte bit-exact (the code decision
is taken in fp32 on both sides), V transposed per head with zero padding, and
the fp8 attention within the fp8 gates of the dequantised fp64 reference."""

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import wan_ref
from oracle.numerics import e4m3_encode, e4m3_rne_sat, f32
from tests.parity import FP8_GATES, LSE_ABS, assert_gates, attn_error_stats, sample_rows, worker_threads
from video_diffusion_transformer_amd import synth, wan_attn
from video_diffusion_transformer_amd.configs import WORKLOADS

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 1.0 / math.sqrt(128.0)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _vt_view(f, heads):
    return f.vt8.view(f.B, heads, 128, f.s_pad)


def _check_quant(qkv, heads):
    B, S = qkv.shape[0], qkv.shape[1]
    D = heads * 128
    f = wan_attn.qkv_quant_fp8(qkv.to(DEV), heads)
    torch.cuda.synchronize()
    r = wan_ref.quant_fp8_ref(_np(qkv), heads, 128)
    np.testing.assert_array_equal(f.amax.cpu().numpy().astype(np.float64), r["amax"])
    np.testing.assert_array_equal(f.scales.cpu().numpy().astype(np.float64), r["scale"])
    codes = r["codes"]
    np.testing.assert_array_equal(f.qk8.cpu().numpy(), codes[..., :2 * D])
    vt = _vt_view(f, heads).cpu().numpy()
    ref_vt = codes[..., 2 * D:].reshape(B, S, heads, 128).transpose(0, 2, 3, 1)
    np.testing.assert_array_equal(vt[..., :S], ref_vt)
    assert not vt[..., S:].any(), "padding past S must be zero"
    return f, r


@pytest.mark.parametrize("B,S,heads", [(1, 128, 2), (2, 200, 3), (1, 1, 1), (1, 300, 40)])
def test_quant_bit_exact(B, S, heads):
    _check_quant(synth.make_qkv(B, S, heads, seed=S + 7 * heads), heads)


def test_quant_all_zero_and_outlier():
    qkv = torch.zeros((1, 64, 768), dtype=torch.bfloat16)
    qkv[0, 5, 300] = 1000.0   # one K outlier; Q and V all zero
    f, r = _check_quant(qkv, 2)
    assert list(f.scales.cpu().numpy()) == [1.0, float(np.float32(448.0) / np.float32(1000.0)), 1.0]


def _check_attn(qkv, heads, what, rows=None, scale=SCALE):
    f, r = _check_quant(qkv, heads) if rows is None else (wan_attn.qkv_quant_fp8(qkv.to(DEV), heads), None)
    out, lse = wan_attn.attn_fwd_fp8(f, lse=True, softmax_scale=scale)
    torch.cuda.synchronize()
    deq = r["deq"]
    o_ref, l_ref = wan_ref.attn_packed_ref(deq, heads, 128, scale)
    st = attn_error_stats(_np(out), o_ref)
    assert_gates(st, FP8_GATES, what)
    assert np.abs(_np(lse) - l_ref).max() <= LSE_ABS, what
    return st


def test_tiny_fp8_attention():
    w = WORKLOADS["tiny"]
    _check_attn(synth.make_qkv(w.B, w.S, w.heads, seed=w.seed), w.heads, "tiny fp8")


@pytest.mark.parametrize("B,S,heads", [(1, 1, 1), (1, 129, 2), (2, 333, 3), (1, 1000, 2), (2, 256, 40)])
def test_ragged_fp8_attention(B, S, heads):
    _check_attn(synth.make_qkv(B, S, heads, seed=3 * S + heads), heads, f"fp8 B{B} S{S} h{heads}")


def test_fp8_largest_head_count():
    """256 heads (the largest the library accepts) through quantisation and fp8 attention."""
    _check_attn(synth.make_qkv(1, 130, 256, seed=257), 256, "fp8 256 heads")


@pytest.mark.parametrize("scale", [0.03, 0.25])
def test_fp8_non_default_softmax_scale(scale):
    """The softmax scale reaches the fp8 kernel (the oracle runs at the same scale)."""
    _check_attn(synth.make_qkv(1, 200, 2, seed=17), 2, f"fp8 scale {scale}", scale=scale)


def test_peaky_fp8_attention():
    qkv = synth.make_qkv(1, 700, 2, seed=5).float()
    qkv[..., :256] *= 6
    _check_attn(qkv.to(torch.bfloat16), 2, "fp8 peaky")


def test_fp8_720p_sampled_rows():
    """The fp8 workload: 720p shape. amax and scales exact; every e4m3 byte of
    Q, K and V^T bit-exact against the oracle's quantisation; attention on
    sampled query rows (with the forced edges of the 256-row workgroups) of
    EVERY (b, h), against all keys."""
    w = WORKLOADS["720p_fp8"]
    D = w.D
    qkv = synth.make_qkv(w.B, w.S, w.heads, seed=w.seed, device=DEV)
    f = wan_attn.qkv_quant_fp8(qkv, w.heads)
    out, lse = wan_attn.attn_fwd_fp8(f, lse=True)
    torch.cuda.synchronize()
    # exact amax / scales from the whole tensor (computed here with torch, a library reduction)
    amax = [qkv[..., i * D:(i + 1) * D].abs().max().item() for i in range(3)]
    np.testing.assert_array_equal(f.amax.cpu().numpy(), np.array(amax, np.float32))
    scales = [wan_ref.fp8_scale(a) for a in amax]
    np.testing.assert_array_equal(f.scales.cpu().numpy().astype(np.float64), scales)
    rows = sample_rows(w.S, 48, seed=w.seed, hw=w.H * w.W)
    assert rows.min() >= 0 and rows.max() < w.S
    rows_t = torch.from_numpy(rows).to(DEV)
    got = _np(out.index_select(1, rows_t))
    got_lse = _np(lse.index_select(2, rows_t))
    host = qkv.cpu()
    qk8 = f.qk8.cpu().view(w.B * w.S, 2 * D)
    vt = _vt_view(f, w.heads).cpu()
    del qkv, out, lse, f
    # every Q and K byte, in chunks of tokens on the host threads
    flat = host.view(w.B * w.S, 3 * D)

    def qk_chunk(r0):
        r1 = min(r0 + 4096, w.B * w.S)
        x = flat[r0:r1, :2 * D].double().numpy()
        ref = np.concatenate([e4m3_encode(e4m3_rne_sat(f32(x[:, :D] * scales[0]))),
                              e4m3_encode(e4m3_rne_sat(f32(x[:, D:] * scales[1])))], axis=1)
        return int((ref != qk8[r0:r1].numpy()).sum())

    with ThreadPoolExecutor(worker_threads()) as ex:
        assert sum(ex.map(qk_chunk, range(0, w.B * w.S, 4096))) == 0, "Q/K e4m3 bytes differ"
    worst = {"max": 0.0, "lse": 0.0}
    for b in range(w.B):
        for h in range(w.heads):
            q = host[b, rows, h * 128:(h + 1) * 128].double().numpy()
            k = host[b, :, D + h * 128:D + (h + 1) * 128].double().numpy()
            v = host[b, :, 2 * D + h * 128:2 * D + (h + 1) * 128].double().numpy()
            # oracle quantisation of this head's slices with the tensor-wide scales
            q8 = e4m3_rne_sat(f32(q * scales[0])) / scales[0]
            k8 = e4m3_rne_sat(f32(k * scales[1])) / scales[1]
            v8c = e4m3_rne_sat(f32(v * scales[2]))
            np.testing.assert_array_equal(vt[b, h, :, :w.S].numpy().T, e4m3_encode(v8c))
            assert not vt[b, h, :, w.S:].any(), "padding past S must be zero"
            o_ref, l_ref = wan_ref.attention_ref(q8, k8, v8c / scales[2], SCALE)
            st = attn_error_stats(got[b, :, h * 128:(h + 1) * 128], o_ref)
            assert_gates(st, FP8_GATES, f"720p fp8 b{b} h{h}")
            le = float(np.abs(got_lse[b, h] - l_ref).max())
            assert le <= LSE_ABS, (b, h, le)
            worst = {"max": max(worst["max"], st["max"]), "lse": max(worst["lse"], le)}
    print(f"720p fp8: {len(rows)} rows x {w.B * w.heads} (b, h): worst {worst}")


def _fused_vs_two_calls(B, grid, heads, seed, device_gen=False, **norm_args):
    """wan_qknorm_rope_quant_fp8 against wan_qknorm_rope then wan_qkv_quant_fp8
    on copies of the same buffer: every output bit-identical."""
    T, H, W = grid
    S = T * H * W
    qkv = synth.make_qkv(B, S, heads, seed=seed, device=DEV if device_gen else "cpu").to(DEV)
    gq, gk = synth.make_gammas(heads * 128, seed=seed, device=DEV)
    a = qkv.clone()
    wan_attn.qknorm_rope(a, gq, gk, grid, heads, **norm_args)
    fa = wan_attn.qkv_quant_fp8(a, heads)
    b = qkv
    fb = wan_attn.qknorm_rope_quant_fp8(b, gq, gk, grid, heads, **norm_args)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "in-place bf16 Q/K differ"
    for name in ("amax", "scales", "qk8"):
        assert torch.equal(getattr(fa, name), getattr(fb, name)), name
    assert torch.equal(_vt_view(fa, heads), _vt_view(fb, heads)), "vt8"
    return b, fb


@pytest.mark.parametrize("B,grid,heads", [(1, (2, 8, 8), 2), (2, (1, 5, 21), 3), (1, (1, 1, 1), 1),
                                          (2, (3, 7, 11), 40), (1, (5, 9, 13), 8)])
def test_fused_norm_quant_equals_two_calls(B, grid, heads):
    _fused_vs_two_calls(B, grid, heads, seed=sum(grid) + heads)


def test_fused_norm_quant_passes_eps_and_theta():
    """Non-default eps and theta reach the fused norm pass the same way as the
    plain norm call (whose parity with these values the norm tests check)."""
    _fused_vs_two_calls(2, (3, 4, 5), 2, seed=31, eps=1e-2, theta=500.0)


def test_fused_norm_quant_matches_oracle():
    """The fused outputs against the oracle's quantisation of the buffer the
    same call left in place (amax, scales and every e4m3 byte bit-exact; the
    bf16 norm output itself is pinned by the norm parity tests and by the
    equality with the two-call path above)."""
    heads, grid = 2, (2, 8, 8)
    qkv = synth.make_qkv(1, 128, heads, seed=40).to(DEV)
    gq, gk = synth.make_gammas(heads * 128, seed=40, device=DEV)
    f = wan_attn.qknorm_rope_quant_fp8(qkv, gq, gk, grid, heads)
    torch.cuda.synchronize()
    r = wan_ref.quant_fp8_ref(_np(qkv), heads, 128)
    np.testing.assert_array_equal(f.amax.cpu().numpy().astype(np.float64), r["amax"])
    np.testing.assert_array_equal(f.scales.cpu().numpy().astype(np.float64), r["scale"])
    np.testing.assert_array_equal(f.qk8.cpu().numpy(), r["codes"][..., :2 * heads * 128])
    vt = _vt_view(f, heads).cpu().numpy()
    np.testing.assert_array_equal(vt[..., :128], r["codes"][..., 2 * heads * 128:].reshape(1, 128, heads, 128)
                                  .transpose(0, 2, 3, 1))


def test_fused_norm_quant_720p():
    w = WORKLOADS["720p_fp8"]
    _fused_vs_two_calls(w.B, (w.T, w.H, w.W), w.heads, seed=w.seed, device_gen=True)


def test_fused_norm_quant_beyond_one_launch():
    """More than 2^21 token rows (several norm launches feed one amax)."""
    _fused_vs_two_calls(1, (33, 256, 256), 1, seed=22, device_gen=True)
