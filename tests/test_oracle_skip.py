"""Pins of the Skip-Softmax (threshold mode) oracle, oracle/wan_ref.py
``skip_blocks_ref`` and ``attention_skip_ref``: threshold 0 is dense
attention, a hand-built score matrix whose skipped set is worked out by hand,
the all-rows rule of a query block, agreement with a scalar brute force, the
kept keys' attention computed independently by gathering them, and the
monotonicity of the skipped set in the threshold."""

import math

import numpy as np
import pytest

from oracle import wan_ref
from oracle.brute import attention_skip_brute
from oracle.numerics import bf16_rne

SCALE = 1.0 / np.sqrt(128.0)


def _rand(rng, *shape, scale=1.0):
    return bf16_rne(rng.standard_normal(shape) * scale)


def test_threshold_zero_is_dense_attention():
    rng = np.random.default_rng(0)
    q, k, v = _rand(rng, 70, 128, scale=3.0), _rand(rng, 200, 128), _rand(rng, 200, 128)
    o, lse, kept, margin = wan_ref.attention_skip_ref(q, k, v, SCALE, 0.0, 48, 64)
    od, ld = wan_ref.attention_ref(q, k, v, SCALE)
    assert kept.all() and np.isinf(margin).all()
    np.testing.assert_allclose(o, od, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, ld, rtol=1e-13)


def _scores_case():
    """Two queries, eight keys with block_k = 2: scores are set through the
    first channel only (q = a e0, k_t = s_t / (a scale) e0)."""
    rows = [[5.0, 4.0, 0.0, 1.0, 6.0, -10.0, 5.5, 5.9],
            [0.0, 0.0, 3.0, 0.5, 1.0, 1.0, 2.0, 0.0]]
    a = 2.0
    q = np.zeros((2, 4))
    q[0, 0], q[1, 1] = a, a
    k = np.zeros((8, 4))
    k[:, 0] = np.array(rows[0]) / (a * SCALE)
    k[:, 1] = np.array(rows[1]) / (a * SCALE)
    v = np.arange(32, dtype=np.float64).reshape(8, 4) / 7.0
    return q, k, v, np.array(rows)


def test_hand_built_skipped_sets():
    """Row 0 has block maxima 5, 1, 6, 5.9 against running maxima -inf, 5, 5,
    6: d = inf, -4, 1, -0.1. Row 1: maxima 0, 3, 1, 2 against -inf, 0, 3, 3:
    d = inf, 3, -2, -1. With one query per block, threshold 0.02 skips only
    (row 0, block 1) (exp(-4) = 0.0183); threshold 0.5 also skips (row 1,
    block 2) (exp(-2) = 0.135) and (row 1, block 3) (exp(-1) = 0.368); and
    threshold 1 adds (row 0, block 3) (exp(-0.1) = 0.905). With both rows in
    one query block a block is skipped only if skipped for both rows (here
    every kept block moves the running max only where the rows agree, so the
    joint decision is the OR of the two rows')."""
    q, k, v, s = _scores_case()
    exp = {0.02: [[1, 0, 1, 1], [1, 1, 1, 1]],
           0.5: [[1, 0, 1, 1], [1, 1, 0, 0]],
           1.0: [[1, 0, 1, 0], [1, 1, 0, 0]]}
    for tau, want in exp.items():
        kept, _ = wan_ref.skip_blocks_ref(s, tau, 1, 2)
        np.testing.assert_array_equal(kept, np.array(want, bool), err_msg=f"tau {tau}")
        kept2, _ = wan_ref.skip_blocks_ref(s, tau, 2, 2)
        np.testing.assert_array_equal(kept2[0], np.array(want, bool).any(axis=0), err_msg=f"tau {tau} joint")
    # the output is the softmax over the kept keys, written out for row 0 at tau = 1
    o, lse, kept, _ = wan_ref.attention_skip_ref(q, k, v, SCALE, 1.0, 1, 2)
    keys = [0, 1, 4, 5]
    w = np.array([math.exp(s[0, t]) for t in keys])
    np.testing.assert_allclose(o[0], (w[:, None] * v[keys]).sum(axis=0) / w.sum(), rtol=1e-12)
    np.testing.assert_allclose(lse[0], math.log(w.sum()), rtol=1e-13)


def test_margin_is_distance_from_the_threshold():
    _, _, _, s = _scores_case()
    _, margin = wan_ref.skip_blocks_ref(s, 0.02, 1, 2)
    np.testing.assert_allclose(margin[0, 1:], np.abs(np.array([-4.0, 1.0, -0.1]) - math.log(0.02)), rtol=1e-12)
    assert np.isinf(margin[:, 0]).all()


@pytest.mark.parametrize("M,N,bq,bk,tau", [(7, 23, 3, 4, 0.05), (5, 16, 5, 3, 0.3), (9, 30, 2, 7, 1.5)])
def test_matches_brute_force(M, N, bq, bk, tau):
    rng = np.random.default_rng(M * 100 + N)
    q, k, v = _rand(rng, M, 16, scale=4.0), _rand(rng, N, 16), _rand(rng, N, 16)
    k[:bk] *= 3.0     # a strong first block, so that later blocks can fall below it
    k[N // 2] *= 3.0  # and a late dominant key
    o, lse, kept, _ = wan_ref.attention_skip_ref(q, k, v, 0.25, tau, bq, bk)
    ob, lb, kb = attention_skip_brute(q.tolist(), k.tolist(), v.tolist(), 0.25, tau, bq, bk)
    np.testing.assert_array_equal(kept, np.array(kb, bool))
    assert not kept.all(), "the case must skip something"
    np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-12)


def test_equals_attention_over_the_gathered_kept_keys():
    """Skipped blocks contribute nothing: each query block's result is plain
    attention over the keys of its kept blocks, gathered explicitly."""
    rng = np.random.default_rng(9)
    M, N, bq, bk = 100, 300, 48, 64
    q, k, v = _rand(rng, M, 128, scale=4.0), _rand(rng, N, 128), _rand(rng, N, 128)
    k[:bk] *= 3.0  # a strong first block
    o, lse, kept, _ = wan_ref.attention_skip_ref(q, k, v, SCALE, 0.1, bq, bk)
    assert not kept.all()
    for b in range(kept.shape[0]):
        keys = np.concatenate([np.arange(j * bk, min(N, (j + 1) * bk)) for j in range(kept.shape[1]) if kept[b, j]])
        rows = slice(b * bq, min(M, (b + 1) * bq))
        ob, lb = wan_ref.attention_ref(q[rows], k[keys], v[keys], SCALE)
        np.testing.assert_allclose(o[rows], ob, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[rows], lb, rtol=1e-13)


def test_skipped_set_grows_with_the_threshold():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((96, 640)) * 3.0
    prev = None
    for tau in (0.0, 0.001, 0.01, 0.1, 0.5, 1.0, 3.0):
        kept, _ = wan_ref.skip_blocks_ref(s, tau, 48, 64)
        assert kept[:, 0].all()
        if prev is not None:
            assert np.all(kept <= prev), tau
        prev = kept
    assert not prev.all()


def test_running_max_is_that_of_the_kept_blocks():
    """A threshold above 1 can skip a block that holds a new maximum; the
    running max then stays at the kept blocks' maximum, so a later block is
    judged against that. Scores (one query, block_k = 1): 0, 0.5, 0.9. With
    threshold 2 (ln 2 = 0.693): block 1 has d = 0.5 < 0.693 -> skipped, the
    running max stays 0; block 2 has d = 0.9 -> kept. (Judged against the max
    of all earlier blocks, 0.5, block 2 would have d = 0.4 and be skipped.)"""
    s = np.array([[0.0, 0.5, 0.9]])
    kept, _ = wan_ref.skip_blocks_ref(s, 2.0, 1, 1)
    np.testing.assert_array_equal(kept, [[True, False, True]])


def test_imposed_decisions_are_used():
    """attention_skip_ref with decisions given (as the GPU tests do where a
    decision lies within rounding of the threshold) uses them as given."""
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 10, 128), _rand(rng, 130, 128), _rand(rng, 130, 128)
    forced = np.array([[True, False, True]])
    o, _, kept, _ = wan_ref.attention_skip_ref(q, k, v, SCALE, 0.0, 48, 64, kept=forced)
    keys = np.r_[0:64, 128:130]
    ob, _ = wan_ref.attention_ref(q, k[keys], v[keys], SCALE)
    np.testing.assert_array_equal(kept, forced)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-14)


def test_history_judges_later_blocks_after_an_imposed_decision():
    """With a history, each block is judged by the rule given the imposed
    earlier decisions: in the three-block case above (threshold 2), imposing
    'kept' on block 1 raises the running max to 0.5, so block 2 (d = 0.4 <
    ln 2) is then skipped by the rule."""
    s = np.array([[0.0, 0.5, 0.9]])
    kept, margin = wan_ref.skip_blocks_ref(s, 2.0, 1, 1, history=np.array([[True, True, True]]))
    np.testing.assert_array_equal(kept, [[True, False, False]])
    np.testing.assert_allclose(margin[0, 2], abs(0.4 - math.log(2.0)), rtol=1e-12)
    same, _ = wan_ref.skip_blocks_ref(s, 2.0, 1, 1, history=np.array([[True, False, True]]))
    np.testing.assert_array_equal(same, wan_ref.skip_blocks_ref(s, 2.0, 1, 1)[0])
