"""fp64 definitions of one Wan2.2 DiT self-attention step.

Test infrastructure only (see the package docstring). Everything here is the
plain definition, written with numpy in float64, in the order the pages give:

  packed [Q|K|V] buffer  ->  full-width RMSNorm of Q and of K  ->  x gamma
  ->  bf16 rounding point  ->  3-D RoPE over (frame, row, column)  ->  bf16
  ->  bidirectional softmax attention per head.

Sources (web pages on Wan2.2; cited by title and section):
  [P1] "Optimizing High-Quality Offline Video Generation" (AWS Neuron docs):
       section "Grounding in an output spec" (latent shape, patchify, S);
       "Overview" (the DiT denoiser is bidirectional); "Tensor parallelism"
       (40 heads x 128 channels, hidden 5120).
  [P4] "Wan2.2-A14B" (TT-DiT model notes), section "Details": each block has
       self-attention with RoPE positional embeddings.
  [P2] "Wan2.2 Text-to-Video" (vLLM-Omni recipe), section "Accelerating
       with TRTLLM_ATTN + Skip-Softmax": the Skip-Softmax threshold mode.
  [P5] "[visual_gen] Optimize Wan2.2 Dataflow" (TensorRT-LLM pull request):
       change 1 (Q and K read as strided views of one fused QKV allocation,
       [Q | K | V] layout kept, updated in place); "Numerical Behavior ->
       Fused Q/K Norm and RoPE" (fp32 RMSNorm, bf16 rounding, fp32 RoPE, bf16
       output); the review comments (norm_q / norm_k normalise over the full
       hidden width num_heads * head_dim, and the weight index is
       headIdx * head_dim + dim); change 2 (amax -> E4M3 inverse scale ->
       quantise) for the fp8 configuration.

Readings where the pages are silent (each is listed in the design notes):
  * RMSNorm is x * (mean(x^2) + eps)^-1/2 * gamma with eps inside the root.
  * gamma multiplies before the single bf16 rounding of the norm output.
  * RoPE rotates interleaved channel pairs (2i, 2i+1) of every head; the 128
    channels split 44 / 42 / 42 over (frame, row, column) and each axis is an
    independent 1-D rotary embedding with angular frequency
    theta ** (-2 j / d_axis) for pair j of that axis (theta = 10000). The split
    and theta are parameters of the Wan2.2 workload, not printed on the pages.
  * Token s of the grid T x H x W sits at frame f, row y, column x with
    s = (f * H + y) * W + x; positions are the integer indices.
  * Attention scale is 1/sqrt(head_dim); no mask; the log-sum-exp is natural.
  * fp8: one scale per tensor (Q, K, V), scale = fl32(448 / amax), computed
    after norm and RoPE; an all-zero tensor gets scale 1.
  * Skip-Softmax threshold mode: a key block is skipped for a query block when
    no row of it has exp(block max - running max of the kept blocks) >=
    threshold (``skip_blocks_ref``); keys in increasing order, fixed block
    sizes.
"""

import numpy as np

from .numerics import bf16_rne, e4m3_rne_sat, e4m3_encode, f32

ROPE_SPLIT = (44, 42, 42)  # channels of a 128-channel head per axis (frame, row, column)
ROPE_THETA = 10000.0
RMS_EPS = 1e-6


# --------------------------------------------------------------------------
# Output spec -> token grid   ([P1] "Grounding in an output spec")
# --------------------------------------------------------------------------
def token_grid(width, height, num_frames):
    """(T, H, W) DiT token grid of a clip. Height and width are first rounded
    down to a multiple of 16; the VAE compresses space 8x and time 4x
    (T_lat = (frames - 1) / 4 + 1); the DiT patchifies 2x2 in space."""
    if (num_frames - 1) % 4:
        raise ValueError("num_frames must be 4k+1 for the 4x temporal compression")
    w_lat = (width // 16) * 16 // 8
    h_lat = (height // 16) * 16 // 8
    t_lat = (num_frames - 1) // 4 + 1
    return t_lat, h_lat // 2, w_lat // 2


def token_positions(T, H, W):
    """Integer (frame, row, column) of every token, in sequence order."""
    s = np.arange(T * H * W)
    return s // (H * W), (s // W) % H, s % W


# --------------------------------------------------------------------------
# RoPE   ([P4] "Details"; [P5] "Fused Q/K Norm and RoPE")
# --------------------------------------------------------------------------
def rope_pairs(head_dim=128, split=ROPE_SPLIT, theta=ROPE_THETA):
    """Per channel pair of a head: which axis it rotates with (0 frame, 1 row,
    2 column) and its angular frequency theta ** (-2 j / d_axis)."""
    if sum(split) != head_dim or any(n % 2 for n in split):
        raise ValueError("rotary split must cover the head with even bands")
    axis, omega = [], []
    for a, n in enumerate(split):
        for j in range(n // 2):
            axis.append(a)
            omega.append(theta ** (-2.0 * j / n))
    return np.array(axis), np.array(omega, dtype=np.float64)


def rope_apply(x, f, y, w, theta=ROPE_THETA, split=ROPE_SPLIT):
    """Rotate interleaved pairs of the last axis of x (length head_dim) by the
    angle position * omega of each pair. f, y, w broadcast against x[..., 0]."""
    x = np.asarray(x, dtype=np.float64)
    axis, omega = rope_pairs(x.shape[-1], split, theta)
    pos = np.stack(np.broadcast_arrays(np.asarray(f, np.float64),
                                       np.asarray(y, np.float64),
                                       np.asarray(w, np.float64)), axis=-1)
    phi = pos[..., axis] * omega  # [..., head_dim/2]
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


# --------------------------------------------------------------------------
# Q/K RMSNorm + bf16 rounding point + RoPE on the packed buffer
# ([P5] change 1, "Fused Q/K Norm and RoPE", review comments)
# --------------------------------------------------------------------------
def split_packed(qkv, heads, head_dim):
    """Views of Q, K, V in a packed [B, S, 3D] buffer: per token the row holds
    all heads of Q, then all heads of K, then all heads of V."""
    D = heads * head_dim
    if qkv.shape[-1] != 3 * D:
        raise ValueError("packed row must hold 3 * heads * head_dim channels")
    return qkv[..., :D], qkv[..., D:2 * D], qkv[..., 2 * D:]


def qknorm_rope_ref(qkv, gamma_q, gamma_k, grid, heads, head_dim,
                    eps=RMS_EPS, theta=ROPE_THETA, rows=None):
    """Reference of the in-place norm + RoPE step.

    qkv     : [B, S, 3D] float64 array (bf16 values).
    gamma_* : [D] float64 arrays (bf16 values), indexed by the global channel
              head * head_dim + i.
    grid    : (T, H, W) with S = T * H * W.
    rows    : optional 1-D array of flat token indices b * S + s; when given only
              those tokens are computed and the outputs are [len(rows), D].

    Returns a dict with, for X in (q, k): ``pre_X`` the fp64 normalised and
    scaled value before the rounding point, ``n_X`` = bf16(pre_X), ``out64_X``
    the exact rotation of n_X, and ``out16_X`` = bf16(out64_X), the value the
    step stores in place.
    """
    T, H, W = grid
    S = T * H * W
    B = qkv.shape[0]
    if qkv.shape[1] != S:
        raise ValueError("S must equal T*H*W")
    D = heads * head_dim
    flat = qkv.reshape(B * S, 3 * D)
    rows = np.arange(B * S) if rows is None else np.asarray(rows)
    out = qknorm_rope_tokens_ref(flat[rows], rows % S, gamma_q, gamma_k, grid, heads, head_dim, eps, theta)
    out["rows"] = rows
    return out


def qknorm_rope_tokens_ref(x_rows, tokens, gamma_q, gamma_k, grid, heads, head_dim,
                           eps=RMS_EPS, theta=ROPE_THETA):
    """The same step for a set of packed rows given directly: x_rows [N, 3D]
    (bf16 values) are the rows of tokens ``tokens`` (sequence index s of the
    T x H x W grid). Returns the dict described in ``qknorm_rope_ref``."""
    T, H, W = grid
    D = heads * head_dim
    tok = np.asarray(tokens)
    f, y, w = tok // (H * W), (tok // W) % H, tok % W
    out = {}
    for name, off, gamma in (("q", 0, gamma_q), ("k", D, gamma_k)):
        x = np.asarray(x_rows[:, off:off + D], dtype=np.float64)
        ms = np.mean(x * x, axis=-1, keepdims=True)  # over all heads of the token
        pre = x / np.sqrt(ms + eps) * np.asarray(gamma, np.float64)[None, :]
        n = bf16_rne(pre)
        rot = rope_apply(n.reshape(-1, heads, head_dim),
                         f[:, None], y[:, None], w[:, None], theta).reshape(-1, D)
        out["pre_" + name] = pre
        out["n_" + name] = n
        out["out64_" + name] = rot
        out["out16_" + name] = bf16_rne(rot)
    return out


# --------------------------------------------------------------------------
# Attention   ([P1] "Overview": bidirectional; "Tensor parallelism": 40 x 128)
# --------------------------------------------------------------------------
def attention_ref(q, k, v, scale):
    """softmax(q k^T * scale) v for one head, every query against every key,
    with the natural log-sum-exp of each query row. q [M, d], k [N, d], v [N, dv]."""
    s = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ np.asarray(v, np.float64)) / l
    return o, m[:, 0] + np.log(l[:, 0])


def attn_packed_ref(qkv, heads, head_dim, scale, rows=None):
    """Attention of every head over a packed [B, S, 3D] buffer.

    rows: optional 1-D array of query token indices (shared by every batch and
    head); keys and values are always all S tokens.
    Returns O [B, M, D] (head h at channels h*head_dim...) and LSE [B, heads, M].
    """
    q, k, v = split_packed(qkv, heads, head_dim)
    B, S = qkv.shape[0], qkv.shape[1]
    rows = np.arange(S) if rows is None else np.asarray(rows)
    D = heads * head_dim
    o = np.empty((B, len(rows), D))
    lse = np.empty((B, heads, len(rows)))
    for b in range(B):
        for h in range(heads):
            c = slice(h * head_dim, (h + 1) * head_dim)
            o[b, :, c], lse[b, h] = attention_ref(q[b, rows, c], k[b, :, c], v[b, :, c], scale)
    return o, lse


def attn_chunk_ref(q, k_chunk, v_chunk, scale):
    """One ring-attention round on one device: local queries against one K/V
    chunk, returning the chunk-normalised output and its log-sum-exp ([P1]
    "Context parallelism": K/V chunks rotate so local Q attends the whole
    sequence)."""
    return attention_ref(q, k_chunk, v_chunk, scale)


def lse_merge_ref(o_a, lse_a, o_b, lse_b):
    """Combine two partial attentions over disjoint key sets into the
    attention over their union: weights exp(lse_i - lse) with
    lse = log(exp(lse_a) + exp(lse_b))."""
    lse = np.logaddexp(lse_a, lse_b)
    wa = np.exp(lse_a - lse)[..., None]
    wb = np.exp(lse_b - lse)[..., None]
    return wa * o_a + wb * o_b, lse


# --------------------------------------------------------------------------
# Skip-Softmax, threshold mode   ([P2] "Accelerating with TRTLLM_ATTN +
# Skip-Softmax", table "Skip-Softmax controls": ``threshold`` is a direct skip
# threshold, finite and >= 0, needing no calibration)
# --------------------------------------------------------------------------
def skip_blocks_ref(s, threshold, block_q, block_k, history=None):
    """Which (query block, key block) pairs the threshold rule keeps.

    The page names the knob, not the rule; the reading taken here: keys are
    processed in blocks of ``block_k`` consecutive keys in increasing order,
    queries in blocks of ``block_q`` consecutive rows. For query row i and key
    block j, let m_j(i) be the largest score of the block and M_j(i) the
    running maximum of the softmax before it: the largest score of the
    earlier blocks KEPT for i's query block (-inf for j = 0). The block's
    softmax (and its product with V) is skipped for a query block when
    exp(m_j(i) - M_j(i)) < threshold for EVERY row i of the query block, i.e.
    no row can gain from it more than ``threshold`` relative to the best key
    it has used so far. threshold = 0 keeps everything; block 0 is always kept.
    (For threshold <= 1 a skipped block never holds a new maximum, so M_j is
    also the largest score of all earlier blocks.)

    s: [M, N] fp64 scores (already scaled). Returns (kept [nqb, nkb] bool,
    margin [nqb, nkb]): margin = |max_i (m_j(i) - M_j(i)) - ln threshold|, the
    distance of the deciding quantity from the threshold (inf where nothing
    is decided: threshold 0, block 0).

    history: optional [nqb, nkb] decisions to carry the running max with
    instead of the rule's own (each block is still judged by the rule, given
    that history): where a decision lies within rounding of the threshold
    either outcome is correct, and the later blocks are then judged against
    the running max the other outcome leaves."""
    M, N = s.shape
    nqb, nkb = -(-M // block_q), -(-N // block_k)
    blockmax = np.stack([s[:, j * block_k:(j + 1) * block_k].max(axis=1) for j in range(nkb)])  # [nkb, M]
    run = np.full(M, -np.inf)  # running max of the kept blocks, per row
    kept = np.ones((nqb, nkb), bool)
    margin = np.full((nqb, nkb), np.inf)
    for j in range(nkb):
        d = blockmax[j] - run  # +inf for block 0
        for b in range(nqb):
            rows = slice(b * block_q, (b + 1) * block_q)
            dmax = d[rows].max()
            with np.errstate(over="ignore"):
                kept[b, j] = not (np.exp(dmax) < threshold)
            if threshold > 0 and np.isfinite(dmax):
                margin[b, j] = abs(dmax - np.log(threshold))
            if (kept[b, j] if history is None else history[b, j]):
                run[rows] = np.maximum(run[rows], blockmax[j][rows])
    return kept, margin


def attention_skip_ref(q, k, v, scale, threshold, block_q, block_k, kept=None):
    """Attention of one head with Skip-Softmax in threshold mode: softmax over
    the keys of the kept blocks only (a skipped block adds nothing to the
    numerator or the denominator), the rule of ``skip_blocks_ref``.

    ``kept`` may be given to impose the block decisions (used where a decision
    lies within rounding of the threshold and both outcomes are correct).
    Returns (o, lse, kept, margin); lse is over the kept keys."""
    s = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) * scale
    k_kept, margin = skip_blocks_ref(s, threshold, block_q, block_k)
    kept = k_kept if kept is None else np.asarray(kept, bool)
    M, N = s.shape
    mask = np.repeat(np.repeat(kept, block_q, axis=0)[:M], block_k, axis=1)[:, :N]
    sm = np.where(mask, s, -np.inf)
    m = sm.max(axis=1, keepdims=True)
    p = np.exp(sm - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ np.asarray(v, np.float64)) / l
    return o, m[:, 0] + np.log(l[:, 0]), kept, margin


# --------------------------------------------------------------------------
# fp8 configuration   ([P5] change 2: amax, E4M3 inverse scale, quantise)
# --------------------------------------------------------------------------
def fp8_scale(amax):
    """Per-tensor quantisation scale 448 / amax, computed in fp32 (an all-zero
    tensor keeps scale 1)."""
    a = np.float32(amax)
    if a == 0:
        return 1.0
    return float(np.float32(448.0) / a)


def quant_fp8_ref(qkv, heads, head_dim):
    """Per-tensor e4m3 quantisation of Q, K and V in a packed buffer.

    The product x * scale is formed in fp32 and then rounded to e4m3 (ties to
    even, saturating), so the code decision is taken in the same precision as
    a GPU that multiplies in fp32. Returns a dict with ``amax`` [3],
    ``scale`` [3], ``codes`` (uint8, same shape as qkv) and ``deq`` (fp64
    dequantised values code / scale)."""
    parts = split_packed(np.asarray(qkv, np.float64), heads, head_dim)
    amax, scale, codes, deq = [], [], [], []
    for x in parts:
        a = float(np.max(np.abs(x))) if x.size else 0.0
        sc = fp8_scale(a)
        v8 = e4m3_rne_sat(f32(x * sc))
        amax.append(a)
        scale.append(sc)
        codes.append(e4m3_encode(v8))
        deq.append(v8 / sc)
    return {"amax": np.array(amax), "scale": np.array(scale),
            "codes": np.concatenate(codes, axis=-1), "deq": np.concatenate(deq, axis=-1)}


def quant_fp8_delayed_ref(qkv, gamma_q, gamma_k, grid, heads, head_dim, amax_prev,
                          eps=RMS_EPS, theta=ROPE_THETA):
    """The norm + RoPE step followed by the per-tensor e4m3 quantisation with
    a DELAYED scale: the producer does not know the amax of the tensor it is
    writing, so each tensor's scale comes from the amax the previous call
    reported (scale = 448 / amax_prev in fp32, 1 when that amax is 0), and the
    call reports the amax of what it quantised for the next one ([P5] change
    2 fuses amax, E4M3 scale and quantisation into the producing kernel; with a
    per-tensor scale a single pass can only use an earlier amax -- the reading
    taken here). A value with |x * scale| > 448 saturates to +-448.

    qkv: [B, S, 3D] fp64 (bf16 values) before the norm; amax_prev: three
    floats (Q, K, V). Q and K are quantised as the norm + RoPE step would
    store them (out16 of ``qknorm_rope_ref``), V as it is. Returns a dict with
    ``scale`` [3] (the scales used), ``amax`` [3] (of the values quantised),
    ``codes`` ([B, S, 3D] uint8) and ``deq`` (fp64 code / scale)."""
    T, H, W = grid
    B, S = qkv.shape[0], qkv.shape[1]
    D = heads * head_dim
    r = qknorm_rope_ref(qkv, gamma_q, gamma_k, grid, heads, head_dim, eps, theta)
    parts = [r["out16_q"].reshape(B, S, D), r["out16_k"].reshape(B, S, D),
             np.asarray(qkv, np.float64)[..., 2 * D:]]
    scale, amax, codes, deq = [], [], [], []
    for x, ap in zip(parts, amax_prev):
        sc = fp8_scale(ap)
        v8 = e4m3_rne_sat(f32(x * sc))
        scale.append(sc)
        amax.append(float(np.max(np.abs(x))) if x.size else 0.0)
        codes.append(e4m3_encode(v8))
        deq.append(v8 / sc)
    return {"scale": np.array(scale), "amax": np.array(amax),
            "codes": np.concatenate(codes, axis=-1), "deq": np.concatenate(deq, axis=-1)}


def qkv_proj_ref(x, w, bias=None):
    """The QKV projection whose output is the packed [Q|K|V] buffer.

    [P5] change 1: the fused QKV projection produces Q, K and V in one shared
    allocation; [P1] "NKI kernels": the qkv_cte kernel is this projection.
    x    : [M, dim] float64 array (bf16 values), one token per row.
    w    : [3 * D, dim] float64 array (bf16 values), one output feature per row
           (features 0..D-1 are Q, D..2D-1 K, 2D..3D-1 V).
    bias : [3 * D] float64 array (bf16 values) or None.
    Returns (y, y16): y = x w^T + bias in fp64, and y16 = bf16(y), the value
    stored in the packed buffer."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    y = x @ w.T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)
    return y, bf16_rne(y)

