"""GPU parity of the ring-attention building blocks (wan_attn_fwd_chunk,
wan_attn_merge): queries attend K/V chunks one at a time and the partial
results are merged by their log-sum-exp; the merged result must match the
oracle's full attention, and each chunk the oracle's chunk attention."""

import math

import numpy as np
import pytest
import torch

from oracle import wan_ref
from tests.parity import BF16_GATES, LSE_ABS, assert_gates, attn_error_stats, sample_rows
from video_diffusion_transformer_amd import synth, wan_attn
from video_diffusion_transformer_amd.configs import WORKLOADS

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 1.0 / math.sqrt(128.0)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _ring(q_src, kv_full, heads, bounds, order=None):
    """Attend q_src to the K/V chunks kv_full[:, a:b] and merge them."""
    B, Sq = q_src.shape[0], q_src.shape[1]
    D = heads * 128
    acc = torch.zeros((B, Sq, D), dtype=torch.float32, device=DEV)
    acc_lse = torch.full((B, heads, Sq), -math.inf, dtype=torch.float32, device=DEV)
    out16 = torch.empty((B, Sq, D), dtype=torch.bfloat16, device=DEV)
    chunks = list(zip(bounds[:-1], bounds[1:]))
    for i in (order or range(len(chunks))):
        a, b = chunks[i]
        kv = kv_full[:, a:b].contiguous()
        o, l = wan_attn.attn_fwd_chunk(q_src, kv, heads)
        wan_attn.attn_merge(acc, acc_lse, o, l, heads, out_bf16=out16)
    torch.cuda.synchronize()
    return acc, acc_lse, out16


@pytest.mark.parametrize("B,S,heads,bounds", [(1, 500, 2, [0, 130, 333, 500]), (2, 777, 3, [0, 1, 400, 777]),
                                              (1, 300, 40, [0, 150, 300]), (1, 1000, 2, [0, 64, 128, 640, 1000]),
                                              (1, 70, 256, [0, 30, 70])])
def test_ring_merge_equals_full_attention(B, S, heads, bounds):
    qkv = synth.make_qkv(B, S, heads, seed=S + heads).to(DEV)
    acc, acc_lse, out16 = _ring(qkv, qkv, heads, bounds)
    o_ref, l_ref = wan_ref.attn_packed_ref(_np(qkv), heads, 128, SCALE)
    assert_gates(attn_error_stats(_np(out16), o_ref), BF16_GATES, "merged bf16")
    st = attn_error_stats(_np(acc), o_ref)
    assert st["rel_l2"] <= 5e-3 and st["max"] <= 1e-2, st
    assert np.abs(_np(acc_lse) - l_ref).max() <= LSE_ABS


def test_query_shard_against_chunks_and_order():
    """A contiguous query shard (as one ring rank holds) against chunks merged
    in two different orders."""
    B, S, heads = 1, 900, 2
    D = heads * 128
    qkv = synth.make_qkv(B, S, heads, seed=31).to(DEV)
    shard = qkv[:, 300:600].contiguous()
    bounds = [0, 300, 600, 900]
    a, la, oa = _ring(shard, qkv, heads, bounds, order=[1, 0, 2])
    b, lb, ob = _ring(shard, qkv, heads, bounds, order=[2, 1, 0])
    o_ref, l_ref = wan_ref.attn_packed_ref(_np(qkv), heads, 128, SCALE, rows=np.arange(300, 600))
    for acc, lse, o16 in ((a, la, oa), (b, lb, ob)):
        assert_gates(attn_error_stats(_np(o16), o_ref), BF16_GATES, "shard")
        assert np.abs(_np(lse) - l_ref).max() <= LSE_ABS
    assert (a - b).abs().max().item() <= 1e-5


def test_chunk_matches_oracle_chunk_and_full_kernel():
    B, S, heads = 2, 333, 2
    D = heads * 128
    qkv = synth.make_qkv(B, S, heads, seed=32).to(DEV)
    kv = qkv[:, 100:250].contiguous()
    o, l = wan_attn.attn_fwd_chunk(qkv, kv, heads)
    torch.cuda.synchronize()
    host = _np(qkv)
    for b in range(B):
        for h in range(heads):
            c = slice(h * 128, (h + 1) * 128)
            ref, lref = wan_ref.attn_chunk_ref(host[b, :, c], host[b, 100:250, D + h * 128:D + (h + 1) * 128],
                                               host[b, 100:250, 2 * D + h * 128:2 * D + (h + 1) * 128], SCALE)
            assert_gates(attn_error_stats(_np(o[b, :, c]), ref), BF16_GATES, f"chunk b{b} h{h}")
            assert np.abs(_np(l[b, h]) - lref).max() <= LSE_ABS
    # the whole sequence as one chunk is the full kernel's LSE-returning
    # instance (both sum the fp32 probabilities), before its bf16 rounding
    full_f32, full_l = wan_attn.attn_fwd_chunk(qkv, qkv, heads)
    full_bf16, l16 = wan_attn.attn_fwd(qkv, heads, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(full_f32.to(torch.bfloat16), full_bf16)
    assert torch.equal(full_l, l16)


def test_merge_into_empty_accumulator_ignores_its_contents():
    """An accumulator row with LSE = -inf is empty: the merge returns the chunk
    exactly, whatever the accumulator's output rows hold (here NaN)."""
    B, Sq, heads = 1, 70, 2
    D = heads * 128
    qkv = synth.make_qkv(B, Sq, heads, seed=33).to(DEV)
    o, l = wan_attn.attn_fwd_chunk(qkv, qkv, heads)
    acc = torch.full((B, Sq, D), math.nan, dtype=torch.float32, device=DEV)
    acc_lse = torch.full((B, heads, Sq), -math.inf, dtype=torch.float32, device=DEV)
    out16 = torch.empty((B, Sq, D), dtype=torch.bfloat16, device=DEV)
    wan_attn.attn_merge(acc, acc_lse, o, l, heads, out_bf16=out16)
    torch.cuda.synchronize()
    assert torch.equal(acc, o) and torch.equal(acc_lse, l)
    assert torch.equal(out16, o.to(torch.bfloat16))


@pytest.mark.parametrize("B,S,heads,bounds", [(1, 500, 2, [0, 130, 333, 500]), (2, 777, 3, [0, 1, 400, 777]),
                                              (1, 300, 40, [0, 150, 300])])
def test_chunk_merge_equals_chunk_then_merge(B, S, heads, bounds):
    """The merge in the attention epilogue gives the same bits as the chunk
    output merged by the separate kernel, round after round (the first round
    into a NaN-filled empty accumulator)."""
    D = heads * 128
    qkv = synth.make_qkv(B, S, heads, seed=S + 2 * heads).to(DEV)
    a_acc = torch.full((B, S, D), math.nan, dtype=torch.float32, device=DEV)
    b_acc = a_acc.clone()
    a_lse = torch.full((B, heads, S), -math.inf, dtype=torch.float32, device=DEV)
    b_lse = a_lse.clone()
    a16 = torch.empty((B, S, D), dtype=torch.bfloat16, device=DEV)
    b16 = torch.empty_like(a16)
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        kv = qkv[:, lo:hi].contiguous()
        o, l = wan_attn.attn_fwd_chunk(qkv, kv, heads)
        wan_attn.attn_merge(a_acc, a_lse, o, l, heads, out_bf16=a16)
        wan_attn.attn_fwd_chunk_merge(qkv, kv, b_acc, b_lse, heads, out_bf16=b16)
        torch.cuda.synchronize()
        assert torch.equal(a_acc, b_acc) and torch.equal(a_lse, b_lse) and torch.equal(a16, b16), (lo, hi)
    o_ref, l_ref = wan_ref.attn_packed_ref(_np(qkv), heads, 128, SCALE)
    assert_gates(attn_error_stats(_np(b16), o_ref), BF16_GATES, "folded bf16")
    assert np.abs(_np(b_lse) - l_ref).max() <= LSE_ABS


def test_ring_non_default_softmax_scale():
    """The softmax scale reaches both chunk kernels: chunks at scale 0.03
    merged (separately and in the epilogue) equal full attention at 0.03."""
    B, S, heads, scale = 1, 500, 2, 0.03
    D = heads * 128
    qkv = synth.make_qkv(B, S, heads, seed=23).to(DEV)
    acc = torch.zeros((B, S, D), dtype=torch.float32, device=DEV)
    lse = torch.full((B, heads, S), -math.inf, dtype=torch.float32, device=DEV)
    f_acc, f_lse = acc.clone(), lse.clone()
    a16, f16 = (torch.empty((B, S, D), dtype=torch.bfloat16, device=DEV) for _ in range(2))
    for lo, hi in ((0, 130), (130, 333), (333, 500)):
        kv = qkv[:, lo:hi].contiguous()
        o, l = wan_attn.attn_fwd_chunk(qkv, kv, heads, softmax_scale=scale)
        wan_attn.attn_merge(acc, lse, o, l, heads, out_bf16=a16)
        wan_attn.attn_fwd_chunk_merge(qkv, kv, f_acc, f_lse, heads, softmax_scale=scale, out_bf16=f16)
    torch.cuda.synchronize()
    o_ref, l_ref = wan_ref.attn_packed_ref(_np(qkv), heads, 128, scale)
    for out, l, what in ((a16, lse, "chunk + merge"), (f16, f_lse, "chunk with merge")):
        assert_gates(attn_error_stats(_np(out), o_ref), BF16_GATES, what)
        assert np.abs(_np(l) - l_ref).max() <= LSE_ABS, what


def test_chunk_merge_errors():
    buf = torch.zeros(2 * 8 * 768, dtype=torch.bfloat16, device=DEV)
    q = buf[:8 * 768].view(1, 8, 768)
    acc = torch.zeros((1, 8, 256), dtype=torch.float32, device=DEV)
    lse = torch.full((1, 2, 8), -math.inf, dtype=torch.float32, device=DEV)
    with pytest.raises(wan_attn.WanError) as e:  # the bf16 copy inside the queries' buffer
        wan_attn.attn_fwd_chunk_merge(q, q, acc, lse, 2, out_bf16=buf[3008:3008 + 2048].view(1, 8, 256))
    assert e.value.status == -5
    with pytest.raises(wan_attn.WanError) as e:  # no keys
        wan_attn.attn_fwd_chunk_merge(q, torch.zeros((1, 0, 768), dtype=torch.bfloat16, device=DEV), acc, lse, 2)
    assert e.value.status == -2
    with pytest.raises(wan_attn.WanError) as e:  # accumulator and its LSE overlap
        wan_attn.attn_fwd_chunk_merge(q, q, acc, acc.view(-1)[:16].view(1, 2, 8), 2)
    assert e.value.status == -5


def test_chunk_errors():
    q = torch.zeros((1, 8, 768), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(wan_attn.WanError) as e:
        wan_attn.attn_fwd_chunk(q, torch.zeros((1, 0, 768), dtype=torch.bfloat16, device=DEV), 2)
    assert e.value.status == -2
    o, l = wan_attn.attn_fwd_chunk(q, q, 2)
    with pytest.raises(wan_attn.WanError) as e:  # merging a buffer into itself
        wan_attn.attn_merge(o, l, o, l, 2)
    assert e.value.status == -5


def test_full_480p_share_cp8_sampled_rows():
    """One rank's share of ring attention at the 480p shape with CP = 8, as the
    benchmark runs it: the first 4,095 queries of each (b, h) attend the 8 K/V
    chunks of 4,095 keys, each folded into the accumulator in the attention
    epilogue (wan_attn_fwd_chunk_merge; at this size with 256 queries per
    workgroup). For every (b, h), seeded rows plus the edges of both workgroup
    sizes, against the oracle's attention over all 32,760 keys."""
    w = WORKLOADS["480p"]
    cp = 8
    sq = w.S // cp
    assert sq * cp == w.S
    qkv = synth.make_qkv(w.B, w.S, w.heads, seed=w.seed, device=DEV)
    shard = qkv[:, :sq].contiguous()
    acc = torch.empty((w.B, sq, w.D), dtype=torch.float32, device=DEV)
    acc_lse = torch.full((w.B, w.heads, sq), -math.inf, dtype=torch.float32, device=DEV)
    out16 = torch.empty((w.B, sq, w.D), dtype=torch.bfloat16, device=DEV)
    for c in range(cp):
        chunk = qkv[:, c * sq:(c + 1) * sq].contiguous()
        wan_attn.attn_fwd_chunk_merge(shard, chunk, acc, acc_lse, w.heads, out_bf16=out16 if c == cp - 1 else None)
        del chunk
    torch.cuda.synchronize()
    rows = sample_rows(sq, 48, seed=11, bms=(256, 384))
    assert rows.min() >= 0 and rows.max() < sq  # host-side bounds check before the GPU gather
    rows_t = torch.from_numpy(rows).to(DEV)
    got = _np(out16.index_select(1, rows_t))
    got_lse = _np(acc_lse.index_select(2, rows_t))
    host = qkv.cpu()
    del qkv, shard, acc, acc_lse, out16
    worst = {"max": 0.0, "lse": 0.0}
    for b in range(w.B):
        for h in range(w.heads):
            q = host[b, rows, h * 128:(h + 1) * 128].double().numpy()
            k = host[b, :, w.D + h * 128:w.D + (h + 1) * 128].double().numpy()
            v = host[b, :, 2 * w.D + h * 128:2 * w.D + (h + 1) * 128].double().numpy()
            o_ref, l_ref = wan_ref.attention_ref(q, k, v, SCALE)
            st = attn_error_stats(got[b, :, h * 128:(h + 1) * 128], o_ref)
            assert_gates(st, BF16_GATES, f"ring share b{b} h{h}")
            le = float(np.abs(got_lse[b, h] - l_ref).max())
            assert le <= LSE_ABS, (b, h, le)
            worst = {"max": max(worst["max"], st["max"]), "lse": max(worst["lse"], le)}
    print(f"480p ring share, cp = {cp}: {len(rows)} rows x {w.B * w.heads} (b, h): worst {worst}")
