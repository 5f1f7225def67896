"""GPU test of wan_qknorm_rope_noalloc, the allocation-free variant of
wan_qknorm_rope, called through the C ABI: its in-place output must equal the
allocating entry point's bit for bit (the norm parity bar: that entry point is
checked element by element against the oracle elsewhere), on two calls in a
row with the second on a smaller input (the shared scratch keeps the first
call's tables, which the second must not use), and sizes beyond its fixed
table capacity are refused without a launch."""

import ctypes

import pytest
import torch

from video_diffusion_transformer_amd import synth, wan_attn

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _noalloc(qkv, gq, gk, grid, heads, theta=1e4):
    T, H, W = grid
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return wan_attn.lib().wan_qknorm_rope_noalloc(
        ctypes.c_void_p(qkv.data_ptr()), ctypes.c_void_p(gq.data_ptr()), ctypes.c_void_p(gk.data_ptr()),
        qkv.shape[0], T, H, W, heads, 128, 1e-6, theta, stream)


@pytest.mark.parametrize("calls", [[(2, (21, 30, 52), 40, 1e4), (1, (3, 5, 7), 3, 500.0)],
                                   [(1, (5, 9, 13), 8, 1e4), (2, (1, 2, 3), 1, 1e4)]])
def test_noalloc_equals_allocating_entry_point(calls):
    for B, grid, heads, theta in calls:
        S = grid[0] * grid[1] * grid[2]
        qkv = synth.make_qkv(B, S, heads, seed=S + heads, device=DEV)
        gq, gk = synth.make_gammas(heads * 128, seed=S, device=DEV)
        a = qkv.clone()
        wan_attn.qknorm_rope(a, gq, gk, grid, heads, theta=theta)
        assert _noalloc(qkv, gq, gk, grid, heads, theta) == 0
        torch.cuda.synchronize()
        assert torch.equal(qkv, a), (B, grid, heads)


def test_noalloc_refuses_grids_beyond_its_table():
    heads = 1
    qkv = torch.zeros((1, 8, 384), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(128, dtype=torch.bfloat16, device=DEV)
    before = qkv.clone()
    # T*22 + H*21 + W*21 > 65536: W = 3200 columns (one row, one frame) -> 67,243 entries
    big = torch.zeros((1, 3200, 384), dtype=torch.bfloat16, device=DEV)
    assert _noalloc(big, g, g, (1, 1, 3200), heads) == -10
    assert wan_attn.lib().wan_status_str(-10).decode().startswith("beyond the fixed capacity")
    torch.cuda.synchronize()
    assert not big.any()
    assert torch.equal(qkv, before)
