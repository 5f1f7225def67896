"""Comparison helpers for the GPU parity tests (test infrastructure).

The norm + RoPE step has two rounding points. Where the exact (fp64) value of a
rounding input lies so close to a bf16 midpoint that the kernel's fp32
arithmetic may legitimately land on either side, both neighbours are accepted;
everywhere else the kernel must produce the oracle's bf16 value bit for bit.

Windows (derived from the fp32 arithmetic of the kernel):
  * first rounding (x * r * gamma): the fp32 sum of squares over D <= 65536
    channels by a butterfly/LDS tree has relative error <= ~17 * 2^-24, the
    reciprocal square root <= 2 ulp, the two products 1 ulp each: below
    2^-19 relative. The window used is 2^-17 relative (4x margin).
  * second rounding (a*cos - b*sin): fp32 cos/sin carry 2^-24 relative error,
    the two products and the sum one rounding each, so the absolute error is
    below 4 * 2^-24 * (|a| + |b|); the window used is E = 2^-21 * (|a| + |b|).
    Under cancellation (|a cos - b sin| << |a| + |b|) E can span several bf16
    quanta of the small result, so the accepted set is every bf16 value that
    rounding can reach from [out - E, out + E]: bf16(out - E) .. bf16(out + E).
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import wan_ref
from oracle.numerics import bf16_rne, bf16_neighbors

REL_WINDOW_1 = 2.0 ** -17
ABS_WINDOW_2 = 2.0 ** -21


def _flag_near_mid(x, window):
    lo, hi = bf16_neighbors(x)
    return (np.abs(x - (lo + hi) / 2) <= window) & (lo != hi), lo, hi


def norm_rope_candidates_match(gpu, ref, name, heads, head_dim, tok_f, tok_y, tok_x, theta=1e4):
    """gpu: [N, D] fp64 values read back from the kernel's output (bf16).
    ref: the oracle dict for the same rows. Returns (ok_mask [N, D],
    exact_fraction, err) where exact means equal to the oracle's nearest value
    and err is the distance from the exact fp64 rotation of the nearest
    admissible norm output (the error metric at rounding ties)."""
    pre, n, out64 = ref["pre_" + name], ref["n_" + name], ref["out64_" + name]
    flag1, lo, hi = _flag_near_mid(pre, REL_WINDOW_1 * np.abs(pre))
    n_lo = np.where(flag1, lo, n)
    n_hi = np.where(flag1, hi, n)
    N, D = n.shape
    ok = np.zeros((N, D), bool)
    err = np.full((N, D), np.inf)
    for a_src in (n_lo, n_hi):
        for b_src in (n_lo, n_hi):
            mix = np.empty_like(n)
            mix[:, 0::2] = a_src[:, 0::2]
            mix[:, 1::2] = b_src[:, 1::2]
            rot = wan_ref.rope_apply(mix.reshape(N, heads, head_dim), tok_f[:, None], tok_y[:, None],
                                     tok_x[:, None], theta).reshape(N, D)
            mag = np.abs(mix[:, 0::2]) + np.abs(mix[:, 1::2])
            e = ABS_WINDOW_2 * np.repeat(mag, 2, axis=1)
            ok |= (gpu >= bf16_rne(rot - e)) & (gpu <= bf16_rne(rot + e))
            err = np.minimum(err, np.abs(gpu - rot))
    exact = np.mean(gpu == ref["out16_" + name])
    return ok, exact, err


def worker_threads():
    """Threads for the chunked oracle runs: numpy releases the GIL inside its
    array operations, so chunks of tokens run in parallel on the host cores."""
    return max(1, min(8, len(os.sched_getaffinity(0))))


def norm_rope_full_parity(host_in, host_out, gamma_q, gamma_k, grid, heads, head_dim=128, eps=1e-6, theta=1e4,
                          chunk=4096):
    """Parity of the norm + RoPE step over EVERY token of a buffer.

    host_in, host_out: CPU bf16 tensors [B*S, >= 2D] whose first 2D columns are
    Q and K before and after the kernel. gamma_q, gamma_k: fp64 arrays [D].
    The oracle runs over all tokens in chunks; the kernel's bits are compared
    with the oracle's bf16 value everywhere, and only rows holding a mismatch
    get the candidate-set check (a mismatch is allowed only at a rounding tie).
    Returns {"bad": elements outside the candidate sets, "exact": fraction
    equal to the oracle's nearest value, "max"/"mean": error against the exact
    rotation of the nearest admissible norm output}."""
    T, H, W = grid
    S = T * H * W
    N = host_in.shape[0]
    D = heads * head_dim

    def work(r0):
        r1 = min(r0 + chunk, N)
        x = host_in[r0:r1, :2 * D].double().numpy()
        g = host_out[r0:r1, :2 * D].double().numpy()
        tok = np.arange(r0, r1) % S
        ref = wan_ref.qknorm_rope_tokens_ref(x, tok, gamma_q, gamma_k, grid, heads, head_dim, eps, theta)
        res = {"bad": 0, "eq": 0, "max": 0.0, "sum": 0.0}
        for name, off in (("q", 0), ("k", D)):
            gg = g[:, off:off + D]
            eq = gg == ref["out16_" + name]
            err = np.abs(gg - ref["out64_" + name])
            res["eq"] += int(eq.sum())
            rows = np.nonzero(~eq.all(axis=1))[0]
            if len(rows):
                sub = {k: v[rows] for k, v in ref.items()}
                t = tok[rows]
                ok, _, e2 = norm_rope_candidates_match(gg[rows], sub, name, heads, head_dim, t // (H * W),
                                                       (t // W) % H, t % W, theta=theta)
                res["bad"] += int((~ok).sum())
                err[rows] = e2
            res["max"] = max(res["max"], float(err.max()))
            res["sum"] += float(err.sum())
        return res

    with ThreadPoolExecutor(worker_threads()) as ex:
        parts = list(ex.map(work, range(0, N, chunk)))
    n = 2 * N * D
    return {"bad": sum(p["bad"] for p in parts), "exact": sum(p["eq"] for p in parts) / n,
            "max": max(p["max"] for p in parts), "mean": sum(p["sum"] for p in parts) / n}


def attn_error_stats(gpu, ref):
    """max / mean absolute error, relative L2 error and cosine similarity."""
    g = np.asarray(gpu, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    err = np.abs(g - r)
    rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    cos = float(g @ r / max(np.linalg.norm(g) * np.linalg.norm(r), 1e-300))
    return {"max": float(err.max()) if err.size else 0.0, "mean": float(err.mean()) if err.size else 0.0,
            "rel_l2": float(rel), "cos": cos}


# Gates: absolute bounds of the workload definition plus relative gates that
# stay meaningful when the output magnitude shrinks as 1/sqrt(S).
BF16_GATES = {"max": 2e-2, "mean": 2e-3, "rel_l2": 1e-2, "cos": 0.9999}
FP8_GATES = {"max": 6e-2, "rel_l2": 5e-2, "cos": 0.999}
# The LSE is ln sum_j exp(s_j) by definition; the kernel instances that return
# it add up the fp32 probabilities (not the rounded weights PV multiplies), so
# what remains is fp32 rounding of the scores, exponentials and sums.
LSE_ABS = 1e-3

# Query rows per workgroup of the attention kernels (bf16: 8 waves x 48 rows;
# fp8: 8 waves x 32 rows) and the 128-row tiling of earlier kernels: the
# sampled rows force the edges of each of these partitions.
ROW_BLOCKS = (128, 256, 384)


def assert_gates(stats, gates, what=""):
    for k, v in gates.items():
        if k == "cos":
            assert stats[k] >= v, f"{what}: cosine {stats[k]} < {v} ({stats})"
        else:
            assert stats[k] <= v, f"{what}: {k} {stats[k]} > {v} ({stats})"


def sample_rows(S, n, seed, bms=ROW_BLOCKS, hw=None):
    """Seeded query rows plus forced edge rows: the first and last row, and
    for each row-block size in ``bms`` the first row of the second block, the
    first row of the last (possibly ragged) block and the row before it, and
    frame boundaries (multiples of ``hw`` = H*W) when given."""
    rng = np.random.default_rng(seed)
    rows = set(rng.integers(0, S, size=min(n, S)).tolist())
    rows |= {0, S - 1}
    for bm in bms:
        last_block = ((S - 1) // bm) * bm
        rows |= {last_block, max(last_block - 1, 0), min(bm, S - 1), min(bm - 1, S - 1)}
    if hw:
        rows |= {min(k * hw, S - 1) for k in (1, 2)} | {max(k * hw - 1, 0) for k in (1, 2)}
    return np.array(sorted(rows))
