"""CPU checks of the GPU-parity comparator (tests/parity.py): the oracle's own
bf16 output passes, a planted one-ulp error away from any rounding tie is
caught, and a planted error in attention output trips the relative gates."""

import numpy as np

from oracle import wan_ref
from oracle.numerics import bf16_rne, bf16_neighbors
from tests.parity import BF16_GATES, attn_error_stats, norm_rope_candidates_match


def _setup():
    rng = np.random.default_rng(0)
    heads, d, grid = 2, 128, (2, 3, 4)
    S = 24
    x = bf16_rne(rng.standard_normal((1, S, 3 * heads * d)))
    g = bf16_rne(1 + 0.1 * rng.standard_normal(heads * d))
    r = wan_ref.qknorm_rope_ref(x, g, g, grid, heads, d)
    tok = np.arange(S)
    f, y, w = tok // 12, (tok // 4) % 3, tok % 4
    return r, heads, d, f, y, w


def test_oracle_output_passes():
    r, heads, d, f, y, w = _setup()
    ok, exact, _ = norm_rope_candidates_match(r["out16_q"], r, "q", heads, d, f, y, w)
    assert ok.all() and exact == 1.0


def test_planted_one_ulp_error_is_caught():
    r, heads, d, f, y, w = _setup()
    g = r["out16_q"].copy()
    # pick an element of moderate size (no cancellation) and move it one bf16 step
    i, j = np.argwhere(np.abs(g) > 0.5)[3]
    lo, hi = bf16_neighbors(np.nextafter(g[i, j], np.inf))
    g[i, j] = hi if hi != g[i, j] else lo
    ok, exact, _ = norm_rope_candidates_match(g, r, "q", heads, d, f, y, w)
    assert not ok[i, j] and ok.sum() == ok.size - 1


def test_attention_gates_catch_a_scaled_output():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((100, 128)) * 0.01
    assert attn_error_stats(o, o)["rel_l2"] == 0
    st = attn_error_stats(o * 1.03, o)       # 3% gain error: max abs tiny, relative gate trips
    assert st["max"] < BF16_GATES["max"] and st["rel_l2"] > BF16_GATES["rel_l2"]


def test_full_parity_helper_passes_oracle_and_catches_a_planted_ulp():
    """norm_rope_full_parity (the every-token check of the full-size GPU tests),
    run over several chunks: the oracle's own bf16 output has no bad element,
    and one element moved by one bf16 step is counted as bad."""
    import torch

    from tests.parity import norm_rope_full_parity
    from video_diffusion_transformer_amd import synth

    B, grid, heads = 2, (3, 5, 7), 3
    S, D = 105, 384
    qkv = synth.make_qkv(B, S, heads, seed=5)
    gq, gk = synth.make_gammas(D, seed=5)
    g64q, g64k = gq.double().numpy(), gk.double().numpy()
    ref = wan_ref.qknorm_rope_ref(qkv.double().numpy(), g64q, g64k, grid, heads, 128)
    out = qkv.clone().view(-1, 3 * D)
    out[:, :D] = torch.from_numpy(ref["out16_q"]).to(torch.bfloat16)
    out[:, D:2 * D] = torch.from_numpy(ref["out16_k"]).to(torch.bfloat16)
    r = norm_rope_full_parity(qkv.view(-1, 3 * D), out, g64q, g64k, grid, heads, chunk=64)
    assert r["bad"] == 0 and r["exact"] == 1.0
    i, j = np.argwhere(np.abs(ref["out16_k"]) > 0.5)[7]
    v = float(out[i, D + j])
    out[i, D + j] = torch.tensor(v * (1 + 2.0 ** -7)).to(torch.bfloat16)
    assert float(out[i, D + j]) != v
    r = norm_rope_full_parity(qkv.view(-1, 3 * D), out, g64q, g64k, grid, heads, chunk=64)
    assert r["bad"] == 1 and r["exact"] < 1.0
