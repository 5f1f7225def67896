"""Pins of the QKV projection oracle (oracle/wan_ref.qkv_proj_ref): a
scalar brute force with exact summation on non-square shapes (a transposed
operand or a dropped bias fails it), identity weights return the input, the
bias alone is returned for a zero input, the bf16 value is the round-to-
nearest-even of the exact one, and Q, K, V occupy consecutive feature blocks."""

import numpy as np
import pytest

from oracle import wan_ref
from oracle.brute import linear_brute
from oracle.numerics import bf16_rne


def _rand(rng, *shape, scale=1.0):
    return bf16_rne(rng.standard_normal(shape) * scale)


@pytest.mark.parametrize("M,K,N,with_bias", [(3, 8, 5, True), (7, 16, 24, False), (1, 33, 9, True)])
def test_matches_brute(M, K, N, with_bias):
    rng = np.random.default_rng(M * 100 + K + N)
    x, w = _rand(rng, M, K), _rand(rng, N, K, scale=K ** -0.5)
    b = _rand(rng, N, scale=0.1) if with_bias else None
    y, y16 = wan_ref.qkv_proj_ref(x, w, b)
    yb = np.array(linear_brute(x.tolist(), w.tolist(), None if b is None else b.tolist()))
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-14)
    assert y.shape == (M, N)
    np.testing.assert_array_equal(y16, bf16_rne(yb))


def test_identity_and_bias_only():
    rng = np.random.default_rng(5)
    x = _rand(rng, 6, 16)
    y, y16 = wan_ref.qkv_proj_ref(x, np.eye(16))
    np.testing.assert_array_equal(y, x)
    np.testing.assert_array_equal(y16, x)
    b = _rand(rng, 48, scale=0.3)
    y, _ = wan_ref.qkv_proj_ref(np.zeros((4, 16)), _rand(rng, 48, 16), b)
    np.testing.assert_array_equal(y, np.broadcast_to(b, (4, 48)))


def test_feature_blocks_are_q_k_v():
    """Feature n of the output comes from row n of w: with w = [Wq; Wk; Wv]
    stacked, the three column blocks are the three separate projections."""
    rng = np.random.default_rng(6)
    D, dim = 8, 12
    x = _rand(rng, 5, dim)
    wq, wk, wv = (_rand(rng, D, dim) for _ in range(3))
    y, _ = wan_ref.qkv_proj_ref(x, np.concatenate([wq, wk, wv]))
    for i, wi in enumerate((wq, wk, wv)):
        np.testing.assert_allclose(y[:, i * D:(i + 1) * D], x @ wi.T, rtol=1e-13)
