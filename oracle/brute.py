"""Pure-Python loop versions of the definitions, for tiny inputs.

Test infrastructure only (see the package docstring). These are written as
explicit scalar loops with ``math`` so that they share no vectorisation,
broadcasting or library path with ``wan_ref``; they serve as one of the pins
of the vectorised oracle on tiny grids.
"""

import math


def attention_brute(q, k, v, scale):
    """Row-by-row softmax attention with exact summation (math.fsum).
    q, k, v: lists of lists of floats. Returns (o, lse) as lists."""
    o, lse = [], []
    for qi in q:
        s = [scale * math.fsum(qi[c] * kj[c] for c in range(len(qi))) for kj in k]
        m = max(s)
        p = [math.exp(x - m) for x in s]
        den = math.fsum(p)
        row = [math.fsum(p[j] * v[j][c] for j in range(len(k))) / den for c in range(len(v[0]))]
        o.append(row)
        lse.append(m + math.log(den))
    return o, lse


def rms_scale_brute(row, gamma, eps):
    """x_c / sqrt(mean over all channels of x^2 + eps) * gamma_c, one token."""
    ms = math.fsum(x * x for x in row) / len(row)
    r = 1.0 / math.sqrt(ms + eps)
    return [row[c] * r * gamma[c] for c in range(len(row))]


def rope_angle_brute(pair, f, y, w, head_dim=128, split=(44, 42, 42), theta=10000.0):
    """Rotation angle of channel pair ``pair`` of a head at grid position (f, y, w)."""
    start = 0
    for pos, n in zip((f, y, w), split):
        if pair < start + n // 2:
            j = pair - start
            return pos * theta ** (-2.0 * j / n)
        start += n // 2
    raise IndexError(pair)


def rope_head_brute(vec, f, y, w, theta=10000.0, split=(44, 42, 42)):
    """Rotate the interleaved pairs of one head vector."""
    out = list(vec)
    for p in range(len(vec) // 2):
        phi = rope_angle_brute(p, f, y, w, len(vec), split, theta)
        a, b = vec[2 * p], vec[2 * p + 1]
        out[2 * p] = a * math.cos(phi) - b * math.sin(phi)
        out[2 * p + 1] = a * math.sin(phi) + b * math.cos(phi)
    return out


def linear_brute(x, w, bias=None):
    """y[m][n] = sum_k x[m][k] w[n][k] (+ bias[n]) with exact summation; lists."""
    out = []
    for xm in x:
        row = []
        for n, wn in enumerate(w):
            terms = [xm[k] * wn[k] for k in range(len(xm))]
            if bias is not None:
                terms.append(bias[n])
            row.append(math.fsum(terms))
        out.append(row)
    return out


def attention_skip_brute(q, k, v, scale, threshold, block_q, block_k):
    """Skip-Softmax threshold mode with scalar loops: running maximum of the
    kept key blocks in order, the per-query-block decision with math.exp, then the
    softmax over the kept keys with exact summation. Returns (o, lse, kept)."""
    M, N = len(q), len(k)
    s = [[scale * math.fsum(qi[c] * kj[c] for c in range(len(qi))) for kj in k] for qi in q]
    nqb, nkb = (M + block_q - 1) // block_q, (N + block_k - 1) // block_k
    kept = [[True] * nkb for _ in range(nqb)]
    run = [-math.inf] * M  # running max of the kept blocks
    for j in range(nkb):
        keys = range(j * block_k, min(N, (j + 1) * block_k))
        bmax = [max(s[i][t] for t in keys) for i in range(M)]
        for b in range(nqb):
            rows = range(b * block_q, min(M, (b + 1) * block_q))
            if j > 0 and all(math.exp(bmax[i] - run[i]) < threshold for i in rows):
                kept[b][j] = False
            else:
                for i in rows:
                    run[i] = max(run[i], bmax[i])
    o, lse = [], []
    for i in range(M):
        use = [t for t in range(N) if kept[i // block_q][t // block_k]]
        m = max(s[i][t] for t in use)
        p = {t: math.exp(s[i][t] - m) for t in use}
        den = math.fsum(p.values())
        o.append([math.fsum(p[t] * v[t][c] for t in use) / den for c in range(len(v[0]))])
        lse.append(m + math.log(den))
    return o, lse, kept
