"""The persistent projection kernels inside a captured HIP graph.

Both take their output tiles from a device counter that each launch clears
with a fill kernel (no memset node), so a graph replays them correctly: every
replay, with eager work and synchronisations between the replays, must give
the eager result bit for bit (wan_qkv_proj, whose captured call keeps the
counter slot it took at capture time, and wan_qkv_proj_norm_rope with its
caller-owned workspace). The rotary tables and the counter ring are made by a
first call before the capture starts.
"""

import pytest
import torch

from video_diffusion_transformer_amd import synth, wan_attn

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(grid, heads, seed):
    T, H, W = grid
    D = heads * 128
    x = synth.make_tokens(2, T * H * W, D, seed=seed, device=DEV)
    w, b = synth.make_qkv_weights(D, seed=seed, device=DEV)
    gq, gk = synth.make_gammas(D, seed=seed, device=DEV)
    return x, w, b, gq, gk


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replays_equal_eager(fused):
    grid, heads = (3, 9, 13), 6
    x, w, b, gq, gk = _inputs(grid, heads, seed=7 + fused)
    D = heads * 128
    out = torch.empty((2, x.shape[1], 3 * D), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(wan_attn.qkv_proj_norm_rope_workspace_bytes(2, x.shape[1], heads), dtype=torch.uint8,
                     device=DEV)
    s = torch.cuda.Stream(DEV)

    def call():
        if fused:
            wan_attn.qkv_proj_norm_rope(x, w, gq, gk, grid, heads, bias=b, out=out, workspace=ws, stream=s)
        else:
            wan_attn.qkv_proj(x, w, heads, bias=b, out=out, stream=s)

    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        call()                       # the tables and the counter ring exist before the capture
    s.synchronize()
    eager = out.clone()
    if fused:
        assert wan_attn.proj_norm_rope_error_word(ws) == 0

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        if fused:
            assert wan_attn.proj_norm_rope_error_word(ws) == 0
        # eager work between the replays, on the default stream
        wan_attn.qkv_proj(x, w, heads, bias=b)
        torch.cuda.synchronize()
