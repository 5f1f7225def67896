"""Pins of the attention oracle (oracle/wan_ref.py): brute-force loops on tiny
grids (including odd sizes that leave ragged tiles), closed forms (zero query,
one key, equal keys, constant values), invariants (joint key/value
permutation), and the two-chunk log-sum-exp merge."""

import numpy as np
import pytest

from oracle import wan_ref
from oracle.brute import attention_brute
from oracle.numerics import bf16_rne

SCALE = 1.0 / np.sqrt(128.0)


def _rand(rng, *shape, scale=1.0):
    return bf16_rne(rng.standard_normal(shape) * scale)


@pytest.mark.parametrize("S,d,qscale", [(1, 128, 1.0), (17, 128, 1.0), (64, 128, 1.0),
                                        (105, 32, 1.0), (129, 32, 1.0), (40, 128, 8.0)])
def test_attention_matches_brute(S, d, qscale):
    rng = np.random.default_rng(S * 7 + d)
    q, k, v = _rand(rng, S, d, scale=qscale), _rand(rng, S, d), _rand(rng, S, d)
    scale = 1.0 / np.sqrt(d)
    o, lse = wan_ref.attention_ref(q, k, v, scale)
    ob, lb = attention_brute(q.tolist(), k.tolist(), v.tolist(), scale)
    np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-12)


def test_zero_query_gives_mean_of_values_and_log_n():
    rng = np.random.default_rng(1)
    S = 50
    k, v = _rand(rng, S, 128), _rand(rng, S, 128)
    o, lse = wan_ref.attention_ref(np.zeros((3, 128)), k, v, SCALE)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (3, 1)), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, np.log(S), rtol=1e-14)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 4, 128), _rand(rng, 1, 128), _rand(rng, 1, 128)
    o, lse = wan_ref.attention_ref(q, k, v, SCALE)
    np.testing.assert_array_equal(o, np.tile(v, (4, 1)))
    np.testing.assert_allclose(lse, (q @ k[0]) * SCALE, rtol=1e-13)


def test_equal_keys_and_constant_values():
    rng = np.random.default_rng(3)
    q = _rand(rng, 5, 128, scale=4.0)
    k = np.tile(_rand(rng, 1, 128), (30, 1))
    v = _rand(rng, 30, 128)
    o, _ = wan_ref.attention_ref(q, k, v, SCALE)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (5, 1)), rtol=1e-12, atol=1e-15)
    o2, _ = wan_ref.attention_ref(q, _rand(rng, 30, 128), np.full((30, 128), -1.75), SCALE)
    np.testing.assert_allclose(o2, -1.75, rtol=1e-14)


def test_joint_key_value_permutation_invariance():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 7, 128), _rand(rng, 33, 128), _rand(rng, 33, 128)
    perm = rng.permutation(33)
    o1, l1 = wan_ref.attention_ref(q, k, v, SCALE)
    o2, l2 = wan_ref.attention_ref(q, k[perm], v[perm], SCALE)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)
    o3, _ = wan_ref.attention_ref(q, k[perm], v, SCALE)  # permuting keys alone changes the answer
    assert np.abs(o3 - o1).max() > 1e-3


@pytest.mark.parametrize("split", [1, 16, 64, 99])
def test_two_chunk_lse_merge_equals_full(split):
    rng = np.random.default_rng(5 + split)
    q, k, v = _rand(rng, 9, 128, scale=3.0), _rand(rng, 100, 128), _rand(rng, 100, 128)
    o, l = wan_ref.attention_ref(q, k, v, SCALE)
    oa, la = wan_ref.attn_chunk_ref(q, k[:split], v[:split], SCALE)
    ob, lb = wan_ref.attn_chunk_ref(q, k[split:], v[split:], SCALE)
    om, lm = wan_ref.lse_merge_ref(oa, la, ob, lb)
    np.testing.assert_allclose(om, o, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(lm, l, rtol=1e-13)


def test_packed_layout_heads_and_rows():
    """Q of head h lives at channels h*d.., K at D + h*d.., V at 2D + h*d..; a
    change in K of head 1 only moves head 1's output; the row subset equals the
    full result's rows."""
    rng = np.random.default_rng(6)
    B, S, heads, d = 2, 24, 3, 128
    D = heads * d
    x = _rand(rng, B, S, 3 * D)
    o, lse = wan_ref.attn_packed_ref(x, heads, d, SCALE)
    for b in range(B):
        for h in range(heads):
            c = slice(h * d, (h + 1) * d)
            ref, lref = wan_ref.attention_ref(x[b, :, c], x[b, :, D + h * d:D + (h + 1) * d],
                                              x[b, :, 2 * D + h * d:2 * D + (h + 1) * d], SCALE)
            np.testing.assert_array_equal(o[b, :, c], ref)
            np.testing.assert_array_equal(lse[b, h], lref)
    y = x.copy()
    y[1, 5, D + d:D + 2 * d] *= 3.0
    o2, _ = wan_ref.attn_packed_ref(y, heads, d, SCALE)
    np.testing.assert_array_equal(o2[0], o[0])
    np.testing.assert_array_equal(o2[1, :, :d], o[1, :, :d])
    np.testing.assert_array_equal(o2[1, :, 2 * d:], o[1, :, 2 * d:])
    assert np.abs(o2[1, :, d:2 * d] - o[1, :, d:2 * d]).max() > 1e-4
    rows = np.array([0, 7, 23])
    o3, l3 = wan_ref.attn_packed_ref(x, heads, d, SCALE, rows=rows)
    np.testing.assert_array_equal(o3, o[:, rows])
    np.testing.assert_array_equal(l3, lse[:, :, rows])
