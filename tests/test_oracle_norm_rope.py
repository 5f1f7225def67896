"""Pins of the norm + RoPE oracle (oracle/wan_ref.py) against closed forms,
invariants, textbook special cases, the pages' worked example of the token
grid, and a scalar brute-force loop on tiny inputs.

Each test is chosen so that a plausible mistake fails it: a per-head instead of
full-width reduction, a wrong gamma index, a wrong rotary band order or size,
a wrong frequency base, a sign error in the rotation, a transposed token order.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import wan_ref
from oracle.brute import rms_scale_brute, rope_head_brute
from oracle.numerics import bf16_rne

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "output_spec.json")


def _bf16_normal(rng, shape, scale=1.0):
    return bf16_rne(rng.standard_normal(shape) * scale)


def _packed(rng, B, S, heads, d=128):
    return _bf16_normal(rng, (B, S, 3 * heads * d))


# ---------------------------------------------------------------- token grid
def test_token_grid_matches_worked_examples():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        T, H, W = wan_ref.token_grid(c["width"], c["height"], c["frames"])
        assert (T, H, W) == (c["T"], c["H"], c["W"]), c
        assert T * H * W == c["S"]


def test_token_order_is_frame_row_column():
    f, y, x = wan_ref.token_positions(2, 3, 4)
    assert (f[0], y[0], x[0]) == (0, 0, 0)
    assert (f[1], y[1], x[1]) == (0, 0, 1)      # column varies fastest
    assert (f[4], y[4], x[4]) == (0, 1, 0)
    assert (f[12], y[12], x[12]) == (1, 0, 0)   # frame slowest
    assert (f[23], y[23], x[23]) == (1, 2, 3)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_form_mean_square():
    """With gamma = 1: mean(pre^2) = ms / (ms + eps) exactly."""
    rng = np.random.default_rng(0)
    heads, d = 4, 128
    qkv = _packed(rng, 1, 12, heads) * 1e-3  # small ms so eps matters
    g = np.ones(heads * d)
    r = wan_ref.qknorm_rope_ref(qkv, g, g, (1, 3, 4), heads, d)
    for name, off in (("q", 0), ("k", heads * d)):
        x = qkv[0, :, off:off + heads * d]
        ms = np.mean(x * x, axis=1)
        np.testing.assert_allclose(np.mean(r["pre_" + name] ** 2, axis=1), ms / (ms + 1e-6), rtol=1e-12)


def test_rmsnorm_scale_invariance():
    rng = np.random.default_rng(1)
    heads, d = 2, 128
    qkv = _packed(rng, 1, 8, heads)
    g = bf16_rne(1 + 0.1 * rng.standard_normal(heads * d))
    a = wan_ref.qknorm_rope_ref(qkv, g, g, (1, 2, 4), heads, d)
    b = wan_ref.qknorm_rope_ref(qkv * 4.0, g, g, (1, 2, 4), heads, d)
    np.testing.assert_allclose(a["pre_q"], b["pre_q"], rtol=1e-5)
    np.testing.assert_allclose(a["pre_k"], b["pre_k"], rtol=1e-5)


def test_rmsnorm_reduces_over_all_heads():
    """Head 0 x100, other heads x1: the full-width mean square is
    (1e4*128 + 39*128)/5120 ~ 251, so every other head shrinks ~15.8x; a
    per-head reduction would leave them at unit RMS."""
    rng = np.random.default_rng(2)
    heads, d = 40, 128
    D = heads * d
    x = rng.standard_normal((1, 4, 3 * D))
    x[..., 0:d] *= 100.0
    x[..., D:D + d] *= 100.0
    x = bf16_rne(x)
    g = np.ones(D)
    r = wan_ref.qknorm_rope_ref(x, g, g, (1, 2, 2), heads, d)
    for name, off in (("q", 0), ("k", D)):
        xr = x[0, :, off:off + D]
        full_rms = np.sqrt(np.mean(xr ** 2, axis=1))
        head1_in = np.sqrt(np.mean(xr[:, d:2 * d] ** 2, axis=1))
        head1_out = np.sqrt(np.mean(r["pre_" + name][:, d:2 * d] ** 2, axis=1))
        np.testing.assert_allclose(head1_out, head1_in / full_rms, rtol=1e-6)
        assert np.all(head1_out < 0.1)           # per-head RMSNorm would give ~1
        assert np.all(full_rms > 14) and np.all(full_rms < 18)


def test_rmsnorm_gamma_uses_global_channel():
    """Identical content in every head, gamma_h = (h+1): the output of head h is
    (h+1) times head 0's. Reusing the first head's weights would make them equal."""
    rng = np.random.default_rng(3)
    heads, d = 3, 128
    D = heads * d
    one = rng.standard_normal((1, 2, d))
    x = bf16_rne(np.concatenate([np.tile(one, (1, 1, heads))] * 3, axis=-1))
    g = np.repeat(np.arange(1, heads + 1, dtype=np.float64), d)
    gk = g[::-1].copy()  # K weights run the other way: heads, ..., 1
    r = wan_ref.qknorm_rope_ref(x, g, gk, (1, 1, 2), heads, d)
    for h in range(heads):
        np.testing.assert_allclose(r["pre_q"][:, h * d:(h + 1) * d], (h + 1) * r["pre_q"][:, :d], rtol=1e-14)
        np.testing.assert_allclose(r["pre_k"][:, h * d:(h + 1) * d] * heads, (heads - h) * r["pre_k"][:, :d], rtol=1e-14)


def test_rmsnorm_single_head_equals_brute():
    rng = np.random.default_rng(4)
    d = 128
    x = _packed(rng, 1, 3, 1, d)
    g = bf16_rne(1 + 0.1 * rng.standard_normal(d))
    r = wan_ref.qknorm_rope_ref(x, g, g, (1, 1, 3), 1, d)
    for t in range(3):
        ref = rms_scale_brute(list(x[0, t, :d]), list(g), 1e-6)
        np.testing.assert_allclose(r["pre_q"][t], ref, rtol=1e-13)


# ---------------------------------------------------------------- RoPE
def test_rope_identity_at_origin_and_single_frame():
    rng = np.random.default_rng(5)
    heads, d = 2, 128
    x = _packed(rng, 1, 6, heads)
    g = bf16_rne(1 + 0.1 * rng.standard_normal(heads * d))
    r = wan_ref.qknorm_rope_ref(x, g, g, (1, 2, 3), heads, d)
    np.testing.assert_array_equal(r["out64_q"][0], r["n_q"][0])  # token (0,0,0)
    # T = 1: frame band (channels 0..43 of each head) is never rotated
    for h in range(heads):
        np.testing.assert_array_equal(r["out64_k"][:, h * d:h * d + 44], r["n_k"][:, h * d:h * d + 44])


def test_rope_textbook_angles():
    """Pair 0 of every band has frequency 1 (angle = position); pair 11 of the
    44-channel frame band has frequency 10000**(-1/2) = 0.01."""
    e0 = np.zeros(128)
    e = e0.copy(); e[0] = 1.0                       # pair 0 (frame band, j=0)
    np.testing.assert_allclose(wan_ref.rope_apply(e, 1, 0, 0)[:2], [0.5403023058681398, 0.8414709848078965], rtol=1e-15)
    e = e0.copy(); e[22] = 1.0                      # pair 11 of the frame band
    np.testing.assert_allclose(wan_ref.rope_apply(e, 100, 0, 0)[22:24], [0.5403023058681398, 0.8414709848078965], rtol=1e-12)
    e = e0.copy(); e[44] = 1.0                      # pair 22: first pair of the row band
    np.testing.assert_allclose(wan_ref.rope_apply(e, 7, 1, 5)[44:46], [0.5403023058681398, 0.8414709848078965], rtol=1e-15)
    e = e0.copy(); e[86] = 1.0                      # pair 43: first pair of the column band
    np.testing.assert_allclose(wan_ref.rope_apply(e, 7, 9, 2)[86:88], [-0.4161468365471424, 0.9092974268256817], rtol=1e-15)
    e = e0.copy(); e[87] = 1.0                      # second component rotates the other way
    np.testing.assert_allclose(wan_ref.rope_apply(e, 0, 0, 2)[86:88], [-0.9092974268256817, -0.4161468365471424], rtol=1e-15)


@pytest.mark.parametrize("band,first_pair,pairs,theta,pos_index", [
    ("frame", 0, 22, 2.0 ** 22, 0), ("row", 22, 21, 2.0 ** 21, 1), ("column", 43, 21, 2.0 ** 21, 2)])
def test_rope_every_pair_of_each_band(band, first_pair, pairs, theta, pos_index):
    """Every pair of a band, not only its first: with theta = 2^22 for the
    44-channel frame band (or 2^21 for a 42-channel band), pair j' of the band
    has frequency 2^-j', so at position p its angle is p / 2^j' -- a closed
    form that does not go through the theta ** (-2 j / d) expression. A wrong
    band width, band offset or pair index within the band fails it."""
    p = 5.0
    pos = [1.0, 2.0, 3.0]
    pos[pos_index] = p
    for j in range(pairs):
        e = np.zeros(128)
        c = 2 * (first_pair + j)
        e[c] = 1.0
        out = wan_ref.rope_apply(e, pos[0], pos[1], pos[2], theta=theta)
        ang = p / 2.0 ** j
        np.testing.assert_allclose(out[c:c + 2], [math.cos(ang), math.sin(ang)], rtol=0, atol=1e-14,
                                   err_msg=f"{band} band pair {j}")


def test_rope_axis_separability():
    rng = np.random.default_rng(6)
    v = rng.standard_normal(128)
    base = wan_ref.rope_apply(v, 3, 4, 5)
    for pos, band in (((9, 4, 5), slice(0, 44)), ((3, 11, 5), slice(44, 86)), ((3, 4, 13), slice(86, 128))):
        out = wan_ref.rope_apply(v, *pos)
        changed = np.abs(out - base) > 0
        mask = np.zeros(128, bool); mask[band] = True
        assert not changed[~mask].any()
        assert changed[mask].sum() >= mask.sum() - 2


def test_rope_preserves_pair_norms():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((50, 128))
    f, y, x = rng.integers(0, 30, 50), rng.integers(0, 45, 50), rng.integers(0, 80, 50)
    out = wan_ref.rope_apply(v, f, y, x)
    np.testing.assert_allclose(out[:, 0::2] ** 2 + out[:, 1::2] ** 2, v[:, 0::2] ** 2 + v[:, 1::2] ** 2, rtol=1e-12)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_rope_relative_position_invariance(axis):
    """<R(p) q, R(p') k> depends only on p - p' along each axis."""
    rng = np.random.default_rng(8 + axis)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    p, pp = np.array([3, 7, 11]), np.array([5, 2, 29])
    delta = np.zeros(3, int); delta[axis] = 17
    a = wan_ref.rope_apply(q, *p) @ wan_ref.rope_apply(k, *pp)
    b = wan_ref.rope_apply(q, *(p + delta)) @ wan_ref.rope_apply(k, *(pp + delta))
    np.testing.assert_allclose(a, b, rtol=1e-11)
    c = wan_ref.rope_apply(q, *(p + delta)) @ wan_ref.rope_apply(k, *pp)  # a shift of one side only changes it
    assert abs(c - a) > 1e-6


def test_norm_rope_matches_brute_on_tiny_grid():
    rng = np.random.default_rng(9)
    heads, d, T, H, W = 2, 128, 2, 3, 4
    S = T * H * W
    x = _packed(rng, 2, S, heads)
    gq = bf16_rne(1 + 0.1 * rng.standard_normal(heads * d))
    gk = bf16_rne(1 + 0.1 * rng.standard_normal(heads * d))
    r = wan_ref.qknorm_rope_ref(x, gq, gk, (T, H, W), heads, d)
    D = heads * d
    for b in range(2):
        for s in range(S):
            f, y, w = s // (H * W), (s // W) % H, s % W
            row = b * S + s
            for name, off, g in (("q", 0, gq), ("k", D, gk)):
                pre = rms_scale_brute(list(x[b, s, off:off + D]), list(g), 1e-6)
                n = bf16_rne(np.array(pre))
                out = []
                for h in range(heads):
                    out += rope_head_brute(list(n[h * d:(h + 1) * d]), f, y, w)
                np.testing.assert_allclose(r["pre_" + name][row], pre, rtol=1e-13)
                np.testing.assert_allclose(r["out64_" + name][row], out, rtol=1e-12, atol=1e-14)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(10)
    heads, d = 2, 128
    x = _packed(rng, 2, 12, heads)
    g = bf16_rne(1 + 0.1 * rng.standard_normal(heads * d))
    full = wan_ref.qknorm_rope_ref(x, g, g, (1, 3, 4), heads, d)
    rows = np.array([0, 5, 11, 12, 23])
    sub = wan_ref.qknorm_rope_ref(x, g, g, (1, 3, 4), heads, d, rows=rows)
    np.testing.assert_array_equal(sub["out16_q"], full["out16_q"][rows])
    np.testing.assert_array_equal(sub["out16_k"], full["out16_k"][rows])
