"""GPU parity of wan_qkv_proj_norm_rope, the projection with the Q/K RMSNorm
and 3-D RoPE in its epilogue, through the C ABI.

The fused kernel computes y = bf16(x W^T + b) with the same tiles and the same
fp32 accumulation order as wan_qkv_proj, so
  * its V part must equal wan_qkv_proj's V bit for bit (the projection itself
    is pinned to the oracle by the projection tests);
  * its Q and K must be the oracle's norm + RoPE (oracle/wan_ref.py
    ``qknorm_rope_tokens_ref``) of wan_qkv_proj's Q and K, over EVERY token,
    under the candidate-set rule of the norm tests (a bit may differ from the
    oracle's nearest bf16 value only at a rounding tie; the fused mean square
    is summed from per-head partial sums, in another fp32 order than the
    in-place norm's).
Shapes: one token, ragged token blocks, odd head counts (a tile straddling K
and V), several token blocks at the full 40-head width, and the full 480p
workload in the launch configuration the benchmark times.
"""

import numpy as np
import pytest
import torch

from tests.parity import norm_rope_full_parity
from video_diffusion_transformer_amd import synth, wan_attn
from video_diffusion_transformer_amd.configs import WORKLOADS

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(B, grid, heads, seed, device="cpu"):
    T, H, W = grid
    D = heads * 128
    x = synth.make_tokens(B, T * H * W, D, seed=seed, device=device).to(DEV)
    w, b = (t.to(DEV) for t in synth.make_qkv_weights(D, seed=seed))
    gq, gk = synth.make_gammas(D, seed=seed, device=DEV)
    return x, w, b, gq, gk


def _check(x, w, b, gq, gk, grid, heads, what, bias=True):
    D = heads * 128
    out, ws = wan_attn.qkv_proj_norm_rope(x, w, gq, gk, grid, heads, bias=b if bias else None)
    y = wan_attn.qkv_proj(x, w, heads, bias=b if bias else None)
    torch.cuda.synchronize()
    assert wan_attn.proj_norm_rope_error_word(ws) == 0, what
    M = x.shape[0] * x.shape[1]
    o, yy = out.view(M, 3 * D), y.view(M, 3 * D)
    assert torch.equal(o[:, 2 * D:], yy[:, 2 * D:]), f"{what}: V differs from the projection's"
    res = norm_rope_full_parity(yy.cpu(), o.cpu(), gq.double().cpu().numpy(), gk.double().cpu().numpy(), grid,
                                heads)
    assert res["bad"] == 0, f"{what}: {res['bad']} Q/K outputs outside the candidate sets"
    assert res["exact"] >= 0.999, f"{what}: only {res['exact']:.5f} equal to the oracle's nearest value"
    return out, y, res


@pytest.mark.parametrize("B,grid,heads", [(1, (1, 1, 1), 1), (1, (2, 8, 8), 2), (2, (3, 5, 7), 3),
                                          (1, (2, 9, 15), 5), (2, (3, 10, 20), 40), (1, (1, 2, 190), 2)])
def test_small_every_token(B, grid, heads):
    """Every token against the oracle; the last grid is one long row (a
    rotary table of 4,054 entries, most on the column axis)."""
    x, w, b, gq, gk = _inputs(B, grid, heads, seed=sum(grid) + heads)
    _check(x, w, b, gq, gk, grid, heads, f"B{B} {grid} h{heads}")


def test_random_shapes_against_the_two_calls():
    """24 seeded shapes (1-12 heads, odd and even; grids of 1 to ~2,500
    tokens; with and without bias): V bit-equal to the projection's, Q and K
    in the candidate sets of the oracle's norm + RoPE of the projection's
    output, the error word clear."""
    rng = np.random.default_rng(2024)
    for case in range(24):
        heads = int(rng.integers(1, 13))
        grid = tuple(int(v) for v in rng.integers(1, [5, 24, 24]))
        B = int(rng.integers(1, 3))
        x, w, b, gq, gk = _inputs(B, grid, heads, seed=100 + case)
        _check(x, w, b, gq, gk, grid, heads, f"case {case}: B{B} {grid} h{heads}", bias=bool(case % 3))


def test_wide_model():
    """64 heads (D = 8192: a Q unit of 32 tiles, 128 K steps) on a few tokens:
    every output against the oracle."""
    grid, heads = (1, 1, 5), 64
    x, w, b, gq, gk = _inputs(1, grid, heads, seed=64)
    _check(x, w, b, gq, gk, grid, heads, "64 heads")


def test_without_bias_and_repeat_calls():
    """No bias; two calls in a row on one workspace (its counters are cleared
    by each call) give the same bits; a call on a smaller input after a larger
    one is still correct."""
    grid, heads = (2, 12, 13), 4
    x, w, b, gq, gk = _inputs(1, grid, heads, seed=11)
    out1, ws = wan_attn.qkv_proj_norm_rope(x, w, gq, gk, grid, heads)
    out2, _ = wan_attn.qkv_proj_norm_rope(x, w, gq, gk, grid, heads, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    _check(x, w, None, gq, gk, grid, heads, "no bias", bias=False)
    small = (1, 3, 5)
    xs = x[:, :15].contiguous()
    out3, _ = wan_attn.qkv_proj_norm_rope(xs, w, gq, gk, small, heads, workspace=ws)
    y3 = wan_attn.qkv_proj(xs, w, heads)
    torch.cuda.synchronize()
    assert wan_attn.proj_norm_rope_error_word(ws) == 0
    D = heads * 128
    res = norm_rope_full_parity(y3.view(15, 3 * D).cpu(), out3.view(15, 3 * D).cpu(), gq.double().cpu().numpy(),
                                gk.double().cpu().numpy(), small, heads)
    assert res["bad"] == 0


def test_matches_two_call_path_bits_mostly():
    """Against the two-call GPU path (projection, then norm + RoPE in place):
    V equal everywhere, Q and K equal except at rounding ties of the norm."""
    grid, heads = (2, 16, 16), 40
    x, w, b, gq, gk = _inputs(1, grid, heads, seed=21)
    out, _ = wan_attn.qkv_proj_norm_rope(x, w, gq, gk, grid, heads, bias=b)
    two = wan_attn.qkv_proj(x, w, heads, bias=b)
    wan_attn.qknorm_rope(two, gq, gk, grid, heads)
    torch.cuda.synchronize()
    eq = (out == two).float().mean().item()
    assert eq >= 0.999, eq
    D = heads * 128
    assert torch.equal(out[..., 2 * D:], two[..., 2 * D:])


def test_full_480p_every_token():
    """The 480p workload (B = 2, 32,760 tokens, 40 heads: 256 token blocks x 60
    feature tiles on a persistent grid) in the benchmark's launch
    configuration: V bit-equal to the projection's, every Q and K output
    against the oracle's norm + RoPE of the projection's Q and K."""
    wl = WORKLOADS["480p"]
    grid = (wl.T, wl.H, wl.W)
    x = synth.make_tokens(wl.B, wl.S, wl.D, seed=wl.seed, device=DEV)
    w, b = synth.make_qkv_weights(wl.D, seed=wl.seed, device=DEV)
    gq, gk = synth.make_gammas(wl.D, seed=wl.seed, device=DEV)
    _, _, res = _check(x, w, b, gq, gk, grid, wl.heads, "480p")
    print(f"480p fused projection + norm + RoPE: exact {res['exact']:.6f}, max err {res['max']:.3g}")


def test_forced_wait_timeouts(monkeypatch):
    """The bounded waits' time-out path, forced from the host: with
    WAN_PROJ_NORM_SPIN_LIMIT=0 a wave whose (token block, part) unit is not
    complete at its first poll gives up (every wait still ends). V stays
    exact; every Q/K output is either the normal result's bits or NaN; NaNs
    appear exactly when the workspace's error word is set. 16 token blocks x
    60 tiles on a 256-workgroup grid: the tiles of later units are taken over
    time, so some wave finds its unit incomplete."""
    grid, heads = (4, 16, 32), 40
    x, w, b, gq, gk = _inputs(2, grid, heads, seed=31)
    ref, ws = wan_attn.qkv_proj_norm_rope(x, w, gq, gk, grid, heads, bias=b)
    torch.cuda.synchronize()
    assert wan_attn.proj_norm_rope_error_word(ws) == 0
    monkeypatch.setenv("WAN_PROJ_NORM_SPIN_LIMIT", "0")
    out, ws2 = wan_attn.qkv_proj_norm_rope(x, w, gq, gk, grid, heads, bias=b)
    torch.cuda.synchronize()
    monkeypatch.delenv("WAN_PROJ_NORM_SPIN_LIMIT")
    D = heads * 128
    assert torch.equal(out[..., 2 * D:], ref[..., 2 * D:])
    qk, rq = out[..., :2 * D], ref[..., :2 * D]
    nan = torch.isnan(qk.float())
    assert torch.equal(qk[~nan], rq[~nan])
    err = wan_attn.proj_norm_rope_error_word(ws2)
    assert (err != 0) == bool(nan.any())
    assert bool(nan.any()), "no wave timed out"
    print(f"forced time-outs: {nan.float().mean().item():.3f} of the Q/K outputs are NaN")
    # and the normal bounds again: no time-out
    out3, ws3 = wan_attn.qkv_proj_norm_rope(x, w, gq, gk, grid, heads, bias=b)
    torch.cuda.synchronize()
    assert wan_attn.proj_norm_rope_error_word(ws3) == 0 and torch.equal(out3, ref)


def test_errors_and_empty():
    grid, heads = (1, 2, 4), 2
    x, w, b, gq, gk = _inputs(1, grid, heads, seed=3)
    need = wan_attn.qkv_proj_norm_rope_workspace_bytes(1, 8, heads)
    small = torch.empty(need - 4, dtype=torch.uint8, device=DEV)
    with pytest.raises(wan_attn.WanError) as e:
        wan_attn.qkv_proj_norm_rope(x, w, gq, gk, grid, heads, workspace=small)
    assert e.value.status == -2
    out = torch.empty((1, 8, 3 * heads * 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(wan_attn.WanError) as e:  # workspace inside the output
        wan_attn.qkv_proj_norm_rope(x, w, gq, gk, grid, heads, out=out,
                                    workspace=out.view(torch.uint8).view(-1)[:need])
    assert e.value.status == -5
    with pytest.raises(wan_attn.WanError) as e:
        wan_attn.qkv_proj_norm_rope(x, w, gq, gk, grid, heads, eps=float("nan"))
    assert e.value.status == -9
    empty = torch.empty((0, 8, heads * 128), dtype=torch.bfloat16, device=DEV)
    o, _ = wan_attn.qkv_proj_norm_rope(empty, w, gq, gk, grid, heads,
                                       workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert o.shape == (0, 8, 3 * heads * 128)
