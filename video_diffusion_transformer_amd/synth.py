"""Seeded synthetic inputs for the self-attention step.

This module holds no arithmetic of the method: it only draws the packed QKV
activations (independent N(0, 1) values rounded to bfloat16), the two RMSNorm
weight vectors (1 + 0.1 * N(0, 1), rounded to bfloat16), for the QKV
projection token activations (N(0, 1)) and a weight matrix and bias
(N(0, 1/dim) and 0.02 N(0, 1)), and, for block-skipping attention, a packed
buffer whose scores fall off with grid distance (random Fourier features of
the token positions), from torch generators seeded per workload. Both the HIP
path and the CPU oracle receive exactly these tensors.

The pages measure on the MLPerf Wan2.2 720p workload, whose activations are not
available; these draws stand in for it with the same shapes. Dense attention
timing does not depend on the values.
"""

import torch


def make_qkv(B, S, heads, head_dim=128, seed=0, device="cpu", chunk_tokens=8192):
    """Packed [B, S, 3 * heads * head_dim] bfloat16 tensor of N(0, 1) draws.

    Drawn in chunks of ``chunk_tokens`` rows (float32, then rounded to bf16) so
    that the float32 temporary stays small. The same (seed, device, chunking)
    always gives the same tensor."""
    D = heads * head_dim
    out = torch.empty((B, S, 3 * D), dtype=torch.bfloat16, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    flat = out.view(B * S, 3 * D)
    for i in range(0, B * S, chunk_tokens):
        n = min(chunk_tokens, B * S - i)
        flat[i:i + n] = torch.randn((n, 3 * D), generator=gen, device=device,
                                    dtype=torch.float32).to(torch.bfloat16)
    return out


def make_qkv_local(B, T, H, W, heads, head_dim=128, seed=0, length=2.0, amplitude=1.46, noise=0.3, device="cpu"):
    """Packed [B, S, 3 * heads * head_dim] bfloat16 tensor (S = T*H*W, token
    s at frame s // (H*W), row (s // W) % H, column s % W) whose scores fall off
    with the distance of two tokens on the 3-D grid: per (batch entry, head)
    the Q and K rows of a token are amplitude * cos(w_c . p + b_c) over the
    channels c (random frequencies w_c ~ N(0, I / length^2) in grid units,
    random phases b_c ~ U[0, 2 pi), p the token's (frame, row, column)), plus
    ``noise`` * N(0, 1); V is N(0, 1). q . k of two tokens is then close to
    amplitude^2 * head_dim / 2 * exp(-|p - p'|^2 / (2 length^2)): about 12
    after the 1/sqrt(128) scale at distance 0, near 0 a few lengths away
    (random features of a Gaussian kernel). The rows have about unit RMS, as
    normalised activations do. This is the attention input (Q and K already
    normalised and rotated), for block-skipping attention."""
    D = heads * head_dim
    S = T * H * W
    gen = torch.Generator()
    gen.manual_seed(50_000 + seed)
    s = torch.arange(S)
    pos = torch.stack([s // (H * W), (s // W) % H, s % W], dim=1).to(torch.float32)  # [S, 3]
    out = torch.empty((B, S, 3 * D), dtype=torch.bfloat16)
    for b in range(B):
        for h in range(heads):
            w = torch.randn((head_dim, 3), generator=gen, dtype=torch.float32) / length
            ph = torch.rand((head_dim,), generator=gen, dtype=torch.float32) * 2 * torch.pi
            feat = amplitude * torch.cos(pos @ w.T + ph)  # [S, head_dim]
            for part in (0, 1):
                n = torch.randn((S, head_dim), generator=gen, dtype=torch.float32)
                out[b, :, part * D + h * head_dim:part * D + (h + 1) * head_dim] = (feat + noise * n).to(torch.bfloat16)
            out[b, :, 2 * D + h * head_dim:2 * D + (h + 1) * head_dim] = torch.randn(
                (S, head_dim), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    return out.to(device)


def make_gammas(D, seed=0, device="cpu"):
    """RMSNorm weights for Q and K, each [D] bfloat16 = bf16(1 + 0.1 * N(0, 1)),
    drawn on the CPU from their own generator so they do not depend on the
    device."""
    gen = torch.Generator()
    gen.manual_seed(10_000 + seed)
    g = 1.0 + 0.1 * torch.randn((2, D), generator=gen, dtype=torch.float32)
    g = g.to(torch.bfloat16).to(device)
    return g[0].contiguous(), g[1].contiguous()


def make_tokens(B, S, dim, seed=0, device="cpu", chunk_tokens=8192):
    """Token activations [B, S, dim] bfloat16 of N(0, 1) draws (chunked like make_qkv)."""
    out = torch.empty((B, S, dim), dtype=torch.bfloat16, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(20_000 + seed)
    flat = out.view(B * S, dim)
    for i in range(0, B * S, chunk_tokens):
        n = min(chunk_tokens, B * S - i)
        flat[i:i + n] = torch.randn((n, dim), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def make_qkv_weights(dim, seed=0, device="cpu"):
    """Stacked QKV projection weights [3 * dim, dim] bfloat16 = bf16(N(0, 1/dim))
    (unit-variance outputs for unit-variance inputs) and the bias [3 * dim] =
    bf16(0.02 N(0, 1)), drawn on the CPU so they do not depend on the device."""
    gen = torch.Generator()
    gen.manual_seed(30_000 + seed)
    w = (torch.randn((3 * dim, dim), generator=gen, dtype=torch.float32) * dim ** -0.5).to(torch.bfloat16)
    b = (0.02 * torch.randn((3 * dim,), generator=gen, dtype=torch.float32)).to(torch.bfloat16)
    return w.to(device), b.to(device)

