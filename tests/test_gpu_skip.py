"""GPU parity of wan_attn_fwd_skip (Skip-Softmax, threshold mode) against the
oracle (oracle/wan_ref.py ``skip_blocks_ref``, ``attention_skip_ref``).

For every (b, h) the kernel's decision map must equal the rule's decisions,
block by block, except where the deciding quantity lies within rounding of
the threshold (there either outcome is correct; the later blocks are then
judged against the running max the kernel's outcome leaves). The output and
LSE are then compared with the oracle's attention over the kernel's kept
blocks, to the bf16 gates.

Inputs: the seeded local-score buffer (scores falling off with 3-D grid
distance, so that blocks do get skipped) and plain N(0, 1) buffers.
"""

import math

import numpy as np
import pytest
import torch

from oracle import wan_ref
from tests.parity import BF16_GATES, LSE_ABS, assert_gates, attn_error_stats
from video_diffusion_transformer_amd import synth, wan_attn
from video_diffusion_transformer_amd.configs import WORKLOADS

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 1.0 / math.sqrt(128.0)
BQ, BK = wan_attn.SKIP_BLOCK_Q, wan_attn.SKIP_BLOCK_K
# |deciding quantity - ln threshold| below this (natural-log units) is a tie:
# the kernel's fp32 scores of bf16 inputs differ from the exact ones by far less
AMBIGUOUS = 5e-4


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check_head(q, k, v, tau, gpu_kept, got_o, got_lse, what, rows=None):
    """One (b, h): decisions, then output and LSE. q may hold only the rows of
    some query blocks (``rows`` maps them; gpu_kept/got_* are for those)."""
    s = (q @ k.T) * SCALE
    rule, margin = wan_ref.skip_blocks_ref(s, tau, BQ, BK, history=gpu_kept)
    firm = margin >= AMBIGUOUS
    bad = np.argwhere(firm & (rule != gpu_kept))
    assert len(bad) == 0, f"{what}: decisions differ at (query block, key block) {bad[:5].tolist()}"
    o_ref, l_ref, _, _ = wan_ref.attention_skip_ref(q, k, v, SCALE, tau, BQ, BK, kept=gpu_kept)
    st = attn_error_stats(got_o, o_ref)
    assert_gates(st, BF16_GATES, what)
    assert np.abs(got_lse - l_ref).max() <= LSE_ABS, what
    return int((~firm).sum())


def _run(qkv, heads, tau, what):
    B, S = qkv.shape[0], qkv.shape[1]
    D = heads * 128
    out, lse, kept = wan_attn.attn_fwd_skip(qkv.to(DEV), heads, tau, lse=True, kept=True)
    torch.cuda.synchronize()
    host, o, l, km = _np(qkv), _np(out), _np(lse), kept.cpu().numpy().astype(bool)
    assert km.shape == (B, heads, -(-S // BQ), -(-S // BK))
    for b in range(B):
        for h in range(heads):
            c = slice(h * 128, (h + 1) * 128)
            q, k, v = host[b, :, c], host[b, :, D + h * 128:D + (h + 1) * 128], host[b, :, 2 * D + h * 128:2 * D + (h + 1) * 128]
            _check_head(q, k, v, tau, km[b, h], o[b, :, c], l[b, h], f"{what} b{b} h{h}")
    return 1.0 - km.mean()


@pytest.mark.parametrize("tau", [0.02, 0.1, 1.0, 3.0])
def test_local_scores_skip_blocks(tau):
    """Scores that fall off with grid distance: a large part of the blocks is
    skipped, and every decision and output matches the oracle."""
    T, H, W, heads = 5, 12, 16, 2
    qkv = synth.make_qkv_local(1, T, H, W, heads, seed=3)
    frac = _run(qkv, heads, tau, f"local tau {tau}")
    assert frac > 0.3, frac


def test_threshold_zero_is_dense():
    qkv = synth.make_qkv_local(2, 3, 10, 17, 3, seed=4)
    out, kept = wan_attn.attn_fwd_skip(qkv.to(DEV), 3, 0.0, kept=True)
    torch.cuda.synchronize()
    assert bool(kept.all())
    o_ref, _ = wan_ref.attn_packed_ref(_np(qkv), 3, 128, SCALE)
    assert_gates(attn_error_stats(_np(out), o_ref), BF16_GATES, "threshold 0")


@pytest.mark.parametrize("B,grid,heads,tau", [(2, (3, 7, 11), 3, 0.05), (1, (1, 1, 1), 1, 0.5),
                                              (1, (2, 9, 13), 40, 0.02), (1, (7, 4, 5), 2, 2.0)])
def test_ragged_shapes(B, grid, heads, tau):
    """S not a multiple of the 48-row or 64-key blocks (a ragged last block of
    each), one token, 40 heads."""
    qkv = synth.make_qkv_local(B, *grid, heads, seed=sum(grid) + heads)
    _run(qkv, heads, tau, f"ragged {grid} h{heads} tau {tau}")


def test_unstructured_scores_with_a_peaky_row():
    """N(0, 1) inputs (little to skip at a small threshold) with Q scaled up:
    peaky rows whose running max moves late; a threshold above 1 skips
    blocks that would raise it."""
    qkv = synth.make_qkv(1, 700, 2, seed=19).float()
    qkv[..., :256] *= 4
    _run(qkv.to(torch.bfloat16), 2, 1.5, "peaky")
    _run(qkv.to(torch.bfloat16), 2, 0.01, "peaky small threshold")


def test_lse_free_instance_and_no_map():
    """Without lse and without the map the same output (the LSE-free instance
    normalises by the bf16 weights, within the gates of the oracle)."""
    qkv = synth.make_qkv_local(1, 4, 8, 16, 2, seed=8)
    out_a, kept = wan_attn.attn_fwd_skip(qkv.to(DEV), 2, 0.05, kept=True)
    out_b = wan_attn.attn_fwd_skip(qkv.to(DEV), 2, 0.05)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    host = _np(qkv)
    for h in range(2):
        q, k, v = host[0, :, h * 128:(h + 1) * 128], host[0, :, 256 + h * 128:256 + (h + 1) * 128], \
            host[0, :, 512 + h * 128:512 + (h + 1) * 128]
        o_ref, _, _, _ = wan_ref.attention_skip_ref(q, k, v, SCALE, 0.05, BQ, BK, kept=kept[0, h].cpu().numpy() > 0)
        assert_gates(attn_error_stats(_np(out_a[0, :, h * 128:(h + 1) * 128]), o_ref), BF16_GATES, f"h{h}")


def test_full_480p_sampled_query_blocks():
    """The 480p shape (B = 2, 40 heads, S = 32,760) on the local-score input:
    for every (b, h), four query blocks (first, last -- ragged --, and two
    seeded) against all keys: decisions and outputs."""
    w = WORKLOADS["480p"]
    qkv = synth.make_qkv_local(w.B, w.T, w.H, w.W, w.heads, seed=w.seed)
    out, lse, kept = wan_attn.attn_fwd_skip(qkv.to(DEV), w.heads, 0.02, lse=True, kept=True)
    torch.cuda.synchronize()
    nqb = -(-w.S // BQ)
    rng = np.random.default_rng(w.seed)
    blocks = sorted({0, nqb - 1, *rng.integers(1, nqb - 1, 2).tolist()})
    rows = np.concatenate([np.arange(b * BQ, min(w.S, (b + 1) * BQ)) for b in blocks])
    assert rows.max() < w.S
    rows_t = torch.from_numpy(rows).to(DEV)
    got = _np(out.index_select(1, rows_t))
    got_lse = _np(lse.index_select(2, rows_t))
    km = kept.cpu().numpy().astype(bool)
    frac = 1.0 - km.mean()
    del out, lse, kept
    host = qkv
    D = w.D
    for b in range(w.B):
        for h in range(w.heads):
            k = host[b, :, D + h * 128:D + (h + 1) * 128].double().numpy()
            v = host[b, :, 2 * D + h * 128:2 * D + (h + 1) * 128].double().numpy()
            start = 0
            for qb in blocks:
                n = min(w.S, (qb + 1) * BQ) - qb * BQ
                q = host[b, qb * BQ:qb * BQ + n, h * 128:(h + 1) * 128].double().numpy()
                sl = slice(start, start + n)
                _check_head(q, k, v, 0.02, km[b, h, qb:qb + 1], got[b, sl, h * 128:(h + 1) * 128],
                            got_lse[b, h, sl], f"480p b{b} h{h} block {qb}")
                start += n
    print(f"480p local scores, threshold 0.02: {frac:.3f} of the blocks skipped")
    assert frac > 0.3


def test_errors():
    qkv = torch.zeros((1, 16, 768), dtype=torch.bfloat16, device=DEV)
    for tau in (-0.1, float("nan"), float("inf")):
        with pytest.raises(wan_attn.WanError) as e:
            wan_attn.attn_fwd_skip(qkv, 2, tau)
        assert e.value.status == -9
    with pytest.raises(wan_attn.WanError) as e:  # map inside the input
        wan_attn.attn_fwd_skip(qkv, 2, 0.1, kept=qkv.view(torch.uint8).view(-1)[:2].view(1, 2, 1, 1))
    assert e.value.status == -5
    out = wan_attn.attn_fwd_skip(torch.empty((0, 16, 768), dtype=torch.bfloat16, device=DEV), 2, 0.1)
    assert out.shape == (0, 16, 256)
