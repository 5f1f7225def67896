"""GPU parity of wan_qkv_proj (through the C ABI) against the fp64 oracle.

The GPU accumulates bf16 products in fp32 (MFMA) and rounds once to bf16, so
each output must equal the bf16 rounding of some value within the fp32
accumulation error of the exact result: |err| <= 2^-16 * sum_k |x_k w_k| (a
generous bound on 5120-term fp32 sums), i.e. a value between
bf16(exact - E) and bf16(exact + E); at least 99% must equal bf16(exact).
Small shapes are compared in full (ragged token and feature tiles included),
the full 480p and 720p shapes on sampled tokens against every feature.
"""

import math

import numpy as np
import pytest
import torch

from oracle import wan_ref
from oracle.numerics import bf16_rne
from tests.parity import BF16_GATES, LSE_ABS, assert_gates, attn_error_stats
from video_diffusion_transformer_amd import synth, wan_attn
from video_diffusion_transformer_amd.configs import WORKLOADS

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check(gpu, x, w, b, what):
    y, y16 = wan_ref.qkv_proj_ref(x, w, b)
    E = 2.0 ** -16 * (np.abs(x) @ np.abs(w).T) + (0.0 if b is None else 2.0 ** -24 * np.abs(b))
    lo, hi = bf16_rne(y - E), bf16_rne(y + E)
    ok = (gpu >= lo) & (gpu <= hi)
    assert ok.all(), f"{what}: {(~ok).sum()} outputs outside the accumulation window"
    exact = np.mean(gpu == y16)
    assert exact >= 0.99, f"{what}: only {exact:.4f} equal bf16(exact)"
    return exact


@pytest.mark.parametrize("B,S,heads,with_bias", [(1, 1, 1, True), (1, 77, 2, False), (2, 300, 2, True),
                                                 (1, 513, 3, True), (1, 256, 1, False),
                                                 (1, 700, 40, True), (2, 1100, 40, False)])
def test_small_full(B, S, heads, with_bias):
    """Every output. With 40 heads (60 feature tiles in 8 bands) the tiles come
    from the per-XCD queues, here with block rows of 3 and of 9 token tiles
    (ragged: a block row holds 4)."""
    D = heads * 128
    x = synth.make_tokens(B, S, D, seed=S + heads)
    w, b = synth.make_qkv_weights(D, seed=S + heads)
    b = b if with_bias else None
    out = wan_attn.qkv_proj(x.to(DEV), w.to(DEV), heads, bias=None if b is None else b.to(DEV))
    torch.cuda.synchronize()
    _check(_np(out).reshape(B * S, 3 * D), _np(x).reshape(B * S, D), _np(w), None if b is None else _np(b),
           f"B{B} S{S} h{heads}")


@pytest.mark.parametrize("name", ["480p", "720p"])
def test_full_size_sampled_tokens(name):
    """Full workload shape (480p: 65,520 tokens, 720p: 151,200 tokens, x 5120
    -> 15360) in the configuration the benchmark times; 96 seeded tokens plus
    the first and last token and the edges of the last token tile, against
    every output feature."""
    wl = WORKLOADS[name]
    B, S, heads, D = wl.B, wl.S, wl.heads, wl.D
    x = synth.make_tokens(B, S, D, seed=wl.seed, device=DEV)
    w, b = synth.make_qkv_weights(D, seed=wl.seed, device=DEV)
    out = wan_attn.qkv_proj(x, w, heads, bias=b)
    torch.cuda.synchronize()
    M = B * S
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.integers(0, M, 96), [0, M - 1, (M // 256) * 256, (M // 256) * 256 - 1]]))
    assert rows.min() >= 0 and rows.max() < M
    rt = torch.from_numpy(rows).to(DEV)
    g = _np(out.view(M, 3 * D).index_select(0, rt))
    xs = _np(x.view(M, D).index_select(0, rt))
    _check(g, xs, _np(w), _np(b), name)


def test_projection_feeds_the_step():
    """qkv_proj output is the packed buffer the norm + RoPE and attention read:
    the GPU chain (projection, norm + RoPE in place, attention) against the
    oracle chain from the same x, W, b (the oracle's own bf16 projection feeds
    its norm and attention), to the bf16 attention gates."""
    heads, grid = 2, (2, 8, 8)
    S, D = 128, 256
    x = synth.make_tokens(1, S, D, seed=3)
    w, b = synth.make_qkv_weights(D, seed=3)
    gq, gk = synth.make_gammas(D, seed=3)
    qkv = wan_attn.qkv_proj(x.to(DEV), w.to(DEV), heads, bias=b.to(DEV))
    torch.cuda.synchronize()
    _, y16 = wan_ref.qkv_proj_ref(_np(x).reshape(S, D), _np(w), _np(b))
    assert np.mean(_np(qkv).reshape(S, 3 * D) == y16) >= 0.99
    wan_attn.qknorm_rope(qkv, gq.to(DEV), gk.to(DEV), grid, heads)
    out, lse = wan_attn.attn_fwd(qkv, heads, lse=True)
    torch.cuda.synchronize()
    host = y16.reshape(1, S, 3 * D)
    r = wan_ref.qknorm_rope_ref(host, _np(gq), _np(gk), grid, heads, 128)
    normed = host.copy().reshape(S, 3 * D)
    normed[:, :D] = r["out16_q"]
    normed[:, D:2 * D] = r["out16_k"]
    o_ref, l_ref = wan_ref.attn_packed_ref(normed.reshape(1, S, 3 * D), heads, 128, 1.0 / math.sqrt(128.0))
    assert_gates(attn_error_stats(_np(out), o_ref), BF16_GATES, "projection chain")
    assert np.abs(_np(lse) - l_ref).max() <= LSE_ABS


def test_wide_model():
    """64 heads (D = 8192: 128 K steps, 96 feature tiles) on a few tokens,
    every output against the oracle."""
    heads, S = 64, 5
    D = heads * 128
    x = synth.make_tokens(1, S, D, seed=64)
    w, b = synth.make_qkv_weights(D, seed=64)
    out = wan_attn.qkv_proj(x.to(DEV), w.to(DEV), heads, bias=b.to(DEV))
    torch.cuda.synchronize()
    _check(_np(out).reshape(S, 3 * D), _np(x).reshape(S, D), _np(w), _np(b), "64 heads")


def test_degenerate_inputs():
    """Zero tokens give the bias exactly; zero weights give the bias exactly;
    without a bias, zero tokens give zeros (the oracle's closed forms)."""
    heads, S = 2, 300
    D = heads * 128
    x = synth.make_tokens(1, S, D, seed=9).to(DEV)
    w, b = (t.to(DEV) for t in synth.make_qkv_weights(D, seed=9))
    zx, zw = torch.zeros_like(x), torch.zeros_like(w)
    for xx, ww, bb, want in ((zx, w, b, b), (x, zw, b, b), (zx, w, None, torch.zeros_like(b))):
        out = wan_attn.qkv_proj(xx, ww, heads, bias=bb)
        torch.cuda.synchronize()
        assert torch.equal(out.view(S, 3 * D), want.view(1, 3 * D).expand(S, 3 * D))


def test_errors():
    x = torch.zeros((1, 8, 256), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((768, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        wan_attn.qkv_proj(x, w[:512], 2)
    out = torch.empty((1, 8, 768), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(wan_attn.WanError) as e:  # output on top of the weights
        wan_attn.qkv_proj(x, w, 2, out=w.view(-1)[:8 * 768].view(1, 8, 768))
    assert e.value.status == -5
    assert wan_attn.qkv_proj(x[:, :0], w, 2).shape == (1, 0, 768)
    del out
