"""Benchmark of one Wan2.2 DiT self-attention step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 480p|720p|720p_fp8|long]

A step is the whole hot path over one batch of synthetic input already resident
in HBM: in-place Q/K RMSNorm + bf16 rounding + 3-D RoPE on the packed [Q|K|V]
buffer, then bidirectional attention over every token (the fp8 workload adds
the per-tensor e4m3 quantisation, its amax taken in the norm pass, and runs
attention on fp8 MFMA). Before every step Q and K are restored from a pristine
device copy (the norm works in place, so each step sees the same input, normalised
once); the restore is outside the timed events. W untimed warm-up steps, then K
timed steps. One JSON line is printed.

  value       attention FLOP of one step (4 * B * heads * S^2 * 128) divided by
              the measured time of the whole step (HIP events on the stream the
              kernels run on, from the first kernel of the step to the end of
              attention), in TFLOP/s.
  roofline    the dominant kernel (attention): algorithmic FLOP per launch over
              its average launch time from HIP events recorded on its stream,
              against the dense MFMA peak of its dtype; ``traffic`` is the HBM
              bytes per launch from the committed rocprofv3 counter summary when
              it was taken on the current kernel source, else null.
  720p, 720p_fp8, long
              (with the default --workload 480p) the same step on the other
              workloads, a few steps each: step time, attention and norm (or
              fused fp8 prep) against their rooflines.
  cpu_baseline the fp64 numpy oracle on the host cores: attention on a bounded
              sample (query rows of one head against all keys) and the norm +
              RoPE over the full 480p tensor.
  skip_softmax (bf16 workloads) Skip-Softmax attention (threshold mode)
              against dense attention on a local-score input of the same
              shape: skipped fraction of the (query block, key block) pairs,
              both times and the speedup; not part of the step or of value.
  ring_share  (bf16 workloads) one GPU's share of ring attention with the
              sequence split over --ring-cp ranks: S/cp queries against cp
              K/V chunks, each round folded into the accumulator by the
              log-sum-exp merge; not part of the step or of value.
  qkv_proj    (bf16 workloads) the QKV projection x W^T + b that produces the
              packed [Q|K|V] buffer the step reads: FLOP per launch over the
              launch time from HIP events on its stream, against the bf16
              MFMA peak; with_norm_rope: the projection with the norm + RoPE
              fused into its epilogue against the two calls; not part of the
              step or of value.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0                           # MI355X HBM3E
# The files each measured kernel is built from (its launch source first).
KERNEL_SOURCES = {"attn_fwd": ("attn_fwd.hip", "attn_fwd_impl.hpp", "common.hpp"),
                  "attn_fwd_fp8": ("attn_fwd_fp8.hip", "common.hpp"),
                  "qknorm_rope": ("qknorm_rope.hip", "common.hpp"),
                  "qkv_proj": ("qkv_proj.hip", "common.hpp"),
                  "qkv_proj_norm_rope": ("qkv_proj.hip", "common.hpp")}
EXTRA_WORKLOADS = ("720p", "720p_fp8", "long")


def kernel_source_hash(name):
    """Hash of a kernel's source files and of the compiler flags its launch
    source is built with (a change of either invalidates its committed
    counters)."""
    from video_diffusion_transformer_amd import build

    files = KERNEL_SOURCES[name]
    h = hashlib.sha256()
    for src in files:
        with open(os.path.join(ROOT, "video_diffusion_transformer_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    h.update(" ".join(build.kernel_flags(files[0])).encode())
    return h.hexdigest()[:16]


def committed_traffic(kernel, workload):
    """HBM bytes per launch from profiles/traffic_<kernel>_<workload>.json, if
    those counters were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s=12.0):
    """The oracle on the host cores: its attention on query rows of (b=0,
    h=0) against all S keys until about ``budget_s`` seconds of CPU work are
    done, and its norm + RoPE over the full 480p tensor (chunks of 4096
    tokens, one chunk per host thread at a time)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    from oracle import wan_ref
    from video_diffusion_transformer_amd import synth
    from video_diffusion_transformer_amd.configs import WORKLOADS

    cores = len(os.sched_getaffinity(0))
    gen = torch.Generator().manual_seed(w.seed)
    k = torch.randn((w.S, 128), generator=gen).to(torch.bfloat16).double().numpy()
    v = torch.randn((w.S, 128), generator=gen).to(torch.bfloat16).double().numpy()
    rows, t0, batch = 0, time.perf_counter(), 64
    while time.perf_counter() - t0 < budget_s:
        q = torch.randn((batch, 128), generator=gen).to(torch.bfloat16).double().numpy()
        wan_ref.attention_ref(q, k, v, 1.0 / math.sqrt(128))
        rows += batch
    dt = time.perf_counter() - t0
    flop = 4.0 * rows * w.S * 128
    del k, v

    n = WORKLOADS["480p"]
    qkv = synth.make_qkv(n.B, n.S, n.heads, seed=n.seed).view(n.B * n.S, 3 * n.D)
    gq, gk = (g.double().numpy() for g in synth.make_gammas(n.D, seed=n.seed))
    chunk = 4096

    def norm_chunk(r0):
        r1 = min(r0 + chunk, n.B * n.S)
        x = qkv[r0:r1, :2 * n.D].double().numpy()
        wan_ref.qknorm_rope_tokens_ref(x, np.arange(r0, r1) % n.S, gq, gk, (n.T, n.H, n.W), n.heads, 128)
        return r1 - r0

    t1 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        tokens = sum(ex.map(norm_chunk, range(0, n.B * n.S, chunk)))
    dn = time.perf_counter() - t1
    del qkv
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"attention: {rows} query rows of head 0 x all {w.S} keys, fp64 numpy (BLAS threads = "
                      f"{cores}), {dt:.1f} s; full-step attention time extrapolated: "
                      f"{w.attn_flop() / (flop / dt):.0f} s",
            "qknorm_rope_480p": {"seconds": round(dn, 2), "tokens": tokens, "threads": cores,
                                 "GB/s": round(n.norm_bytes() / dn / 1e9, 3),
                                 "note": "exact time of the oracle's norm + RoPE over the whole 480p tensor "
                                         "(B=2, S=32760, 40 heads), chunks of 4096 tokens on a pool of host "
                                         "threads"}}


def ring_share(w, qkv, cp, reps=3):
    """One GPU's share of a ring-attention call with the sequence split over cp
    ranks: its S/cp queries attend each of the cp K/V chunks, each round folded
    into the accumulator in the attention epilogue (wan_attn_fwd_chunk_merge).
    Also times the same share with the chunk output written out and merged by
    the separate kernel (wan_attn_fwd_chunk + wan_attn_merge). HIP events on
    the stream, reps shares after one warm-up each."""
    import torch

    from video_diffusion_transformer_amd import wan_attn

    if cp < 2 or w.S % cp or w.dtype != "bf16":
        return None
    sq = w.S // cp
    dev = qkv.device
    shard = qkv[:, :sq].contiguous()
    chunks = [qkv[:, c * sq:(c + 1) * sq].contiguous() for c in range(cp)]
    o = torch.empty((w.B, sq, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.heads, sq), dtype=torch.float32, device=dev)
    acc = torch.empty_like(o)
    acc_lse = torch.empty_like(lse)
    out16 = torch.empty((w.B, sq, w.D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def fused():
        acc_lse.fill_(-math.inf)  # empty accumulator
        for c in range(cp):
            wan_attn.attn_fwd_chunk_merge(shard, chunks[c], acc, acc_lse, w.heads,
                                          out_bf16=out16 if c == cp - 1 else None)

    def separate():
        acc_lse.fill_(-math.inf)
        for c in range(cp):
            wan_attn.attn_fwd_chunk(shard, chunks[c], w.heads, out=o, lse=lse)
            wan_attn.attn_merge(acc, acc_lse, o, lse, w.heads, out_bf16=out16 if c == cp - 1 else None)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0, t1 = E(), E()
        t0.record(stream)
        for _ in range(reps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    ms = timed(fused)
    ms_sep = timed(separate)
    flop = 4.0 * w.B * w.heads * sq * w.S * 128
    return {"cp": cp, "queries": sq, "ms_per_share": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
            "ms_per_share_separate_merge": round(ms_sep, 4),
            "note": "S/cp local queries against cp K/V chunks of S/cp keys, each round merged in the attention "
                    "epilogue; TFLOP/s counts the attention FLOP of the share over the whole share time"}


def qkv_proj(w, dev, reps=3):
    """The QKV projection on the workload's token matrix: x [B, S, D] times the
    fused weight [3D, D] plus bias into the packed [B, S, 3D] buffer. Two
    warm-up calls, then reps calls timed with HIP events on the stream (the
    same for the projection + norm + RoPE, fused and as two calls)."""
    import torch

    from video_diffusion_transformer_amd import synth, wan_attn

    if reps < 1 or w.dtype != "bf16":
        return None
    x = synth.make_tokens(w.B, w.S, w.D, seed=w.seed, device=dev)
    wq, bq = synth.make_qkv_weights(w.D, seed=w.seed, device=dev)
    gq, gk = synth.make_gammas(w.D, seed=w.seed, device=dev)
    grid = (w.T, w.H, w.W)
    out = torch.empty((w.B, w.S, 3 * w.D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(wan_attn.qkv_proj_norm_rope_workspace_bytes(w.B, w.S, w.heads), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def proj():
        wan_attn.qkv_proj(x, wq, w.heads, bias=bq, out=out)

    def two_call():
        wan_attn.qkv_proj(x, wq, w.heads, bias=bq, out=out)
        wan_attn.qknorm_rope(out, gq, gk, grid, w.heads)

    def fused():
        wan_attn.qkv_proj_norm_rope(x, wq, gq, gk, grid, w.heads, bias=bq, out=out, workspace=ws)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(reps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    ms = timed(proj)
    ms_two, ms_fused = timed(two_call), timed(fused)
    if wan_attn.proj_norm_rope_error_word(ws) != 0:
        raise RuntimeError("wan_qkv_proj_norm_rope: a token block's wait hit its spin limit")
    flop = 2.0 * w.B * w.S * 3 * w.D * w.D
    tf = flop / (ms * 1e-3) / 1e12
    del x, wq, bq, out, ws
    return {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
            "frac": round(tf / PEAK_TFLOPS["bf16"], 4), "ms_per_launch": round(ms, 4), "flop_per_launch": flop,
            "traffic": committed_traffic("qkv_proj", w.name),
            "with_norm_rope": {"ms_fused": round(ms_fused, 4), "ms_two_call": round(ms_two, 4),
                               "traffic_fused": committed_traffic("qkv_proj_norm_rope", w.name),
                               "note": "projection followed by the Q/K norm + RoPE: one fused kernel "
                                       "(wan_qkv_proj_norm_rope) against wan_qkv_proj then wan_qknorm_rope"}}


def skip_softmax(w, dev, threshold, reps=3):
    """Skip-Softmax (threshold mode) against dense attention on the same
    input: the seeded local-score buffer of the workload's shape (scores fall
    off with 3-D grid distance; Q and K already at unit RMS, i.e. the attention
    input). HIP events on the stream, reps calls each after one warm-up; the
    skipped fraction comes from one more call that writes the decision map."""
    import torch

    from video_diffusion_transformer_amd import synth, wan_attn

    if threshold <= 0 or w.dtype != "bf16":
        return None
    qkv = synth.make_qkv_local(w.B, w.T, w.H, w.W, w.heads, seed=w.seed).to(dev)
    out = torch.empty((w.B, w.S, w.D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(reps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    dense = timed(lambda: wan_attn.attn_fwd(qkv, w.heads, out=out))
    skip = timed(lambda: wan_attn.attn_fwd_skip(qkv, w.heads, threshold, out=out))
    _, kept = wan_attn.attn_fwd_skip(qkv, w.heads, threshold, out=out, kept=True)
    frac = 1.0 - kept.float().mean().item()
    del qkv, out, kept
    flop = w.attn_flop()
    return {"threshold": threshold, "skipped_fraction": round(frac, 4), "ms_dense": round(dense, 4),
            "ms_skip": round(skip, 4), "speedup": round(dense / skip, 3),
            "dense_equivalent_tflops": round(flop / (skip * 1e-3) / 1e12, 2),
            "input": "local scores: per (b, h) random Fourier features of the token's 3-D grid position "
                     "(length 2 tokens) plus 0.3 N(0, 1) noise, q.k/sqrt(128) about 12 at distance 0; "
                     f"{w.name} shape"}


def run_steps(w, dev, steps, warmup, fp8_unfused=False):
    """Allocate the workload's buffers and run warm-up + timed steps. Returns
    (timings, qkv) with per-step means in ms of the step and of its phases."""
    import torch

    from video_diffusion_transformer_amd import synth, wan_attn

    grid = (w.T, w.H, w.W)
    qkv = synth.make_qkv(w.B, w.S, w.heads, seed=w.seed, device=dev)
    pristine_qk = qkv[..., :2 * w.D].clone()  # V is never written
    gq, gk = synth.make_gammas(w.D, seed=w.seed, device=dev)
    out = torch.empty((w.B, w.S, w.D), dtype=torch.bfloat16, device=dev)
    fp8 = w.dtype == "fp8"
    f8 = wan_attn.fp8_buffers(w.B, w.S, w.heads, dev) if fp8 else None
    stream = torch.cuda.current_stream(dev)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(ev=None):
        qkv[..., :2 * w.D].copy_(pristine_qk)  # same input every step; before the step's first event
        if ev: ev[0].record(stream)
        if fp8 and not fp8_unfused:
            wan_attn.qknorm_rope_quant_fp8(qkv, gq, gk, grid, w.heads, out=f8)  # norm + RoPE + amax, quantise
            if ev: ev[1].record(stream)
            if ev: ev[2].record(stream)
        else:
            wan_attn.qknorm_rope(qkv, gq, gk, grid, w.heads)
            if ev: ev[1].record(stream)
            if fp8:
                wan_attn.qkv_quant_fp8(qkv, w.heads, out=f8)
            if ev: ev[2].record(stream)
        if fp8:
            wan_attn.attn_fwd_fp8(f8, out=out)
        else:
            wan_attn.attn_fwd(qkv, w.heads, out=out)
        if ev: ev[3].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[E() for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    t = {"step": sum(e[0].elapsed_time(e[3]) for e in evs) / steps,
         "norm": sum(e[0].elapsed_time(e[1]) for e in evs) / steps,
         "quant": sum(e[1].elapsed_time(e[2]) for e in evs) / steps,
         "attn": sum(e[2].elapsed_time(e[3]) for e in evs) / steps}
    if not fp8:
        # a plain device copy of the norm's bytes (Q and K read, then written):
        # the bandwidth the chip reaches on a read + write stream of this size
        dst = torch.empty_like(pristine_qk)
        dst.copy_(pristine_qk)
        torch.cuda.synchronize()
        e0, e1 = E(), E()
        reps = max(3, steps)
        e0.record(stream)
        for _ in range(reps):
            dst.copy_(pristine_qk)
        e1.record(stream)
        torch.cuda.synchronize()
        t["copy"] = e0.elapsed_time(e1) / reps
        del dst
    if fp8:
        # the single-pass producer with delayed scales, on the same raw input:
        # amax_prev from the last step (what the previous DiT step would report)
        qkv[..., :2 * w.D].copy_(pristine_qk)
        amax_prev = f8.amax.clone()
        g8 = wan_attn.fp8_buffers(w.B, w.S, w.heads, dev)
        wan_attn.qknorm_rope_quant_fp8_delayed(qkv, gq, gk, grid, w.heads, amax_prev, out=g8)
        torch.cuda.synchronize()
        e0, e1 = E(), E()
        reps = max(3, steps)
        e0.record(stream)
        for _ in range(reps):
            wan_attn.qknorm_rope_quant_fp8_delayed(qkv, gq, gk, grid, w.heads, amax_prev, out=g8)
        e1.record(stream)
        torch.cuda.synchronize()
        t["prep_delayed"] = e0.elapsed_time(e1) / reps
        del g8, amax_prev
    del pristine_qk, out, f8
    return t, qkv


def kernel_objects(w, t, fp8_unfused=False):
    """Roofline objects of the step's kernels from the measured times."""
    fp8 = w.dtype == "fp8"
    dtype = "fp8" if fp8 else "bf16"
    flop = w.attn_flop()
    attn_tflops = flop / (t["attn"] * 1e-3) / 1e12
    kname = "attn_fwd_fp8" if fp8 else "attn_fwd"
    objs = {"attention": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_TFLOPS[dtype],
                          "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_TFLOPS[dtype], 4),
                          "traffic": committed_traffic(kname, w.name), "kernel": kname,
                          "ms_per_launch": round(t["attn"], 4), "flop_per_launch": flop}}
    if fp8 and not fp8_unfused:
        # one call: norm + RoPE + amax (reads Q, K, V; writes Q, K), then the
        # quantisation (reads Q, K, V; writes e4m3 Q, K, V^T)
        prep_bytes = w.B * w.S * w.D * (8 + 2 + 6 + 3)
        gbs = prep_bytes / (t["norm"] * 1e-3) / 1e9
        objs["qknorm_rope_quant_fp8"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                         "ms_per_launch": round(t["norm"], 4), "bytes_per_launch": prep_bytes}
    if fp8 and "prep_delayed" in t:
        # reads Q, K, V (bf16), writes e4m3 Q, K, V^T: 9 bytes per token and channel
        d_bytes = w.B * w.S * w.D * 9
        gbs = d_bytes / (t["prep_delayed"] * 1e-3) / 1e9
        objs["qknorm_rope_quant_fp8_delayed"] = {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "ms_per_launch": round(t["prep_delayed"], 4),
            "bytes_per_launch": d_bytes,
            "note": "single-pass producer with delayed per-tensor scales (from the previous call's amax); not "
                    "the step's prep, which uses current scales"}
    else:
        gbs = w.norm_bytes() / (t["norm"] * 1e-3) / 1e9
        objs["qknorm_rope"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(gbs / PEAK_HBM_GBS, 4), "ms_per_launch": round(t["norm"], 4),
                               "bytes_per_launch": w.norm_bytes(),
                               "traffic": committed_traffic("qknorm_rope", w.name)}
        if "copy" in t:
            cbs = w.norm_bytes() / (t["copy"] * 1e-3) / 1e9
            objs["qknorm_rope"].update({"copy_GBps": round(cbs, 1), "frac_of_copy": round(gbs / cbs, 4),
                                        "copy_note": "device copy (torch copy_) of the same bytes: Q and K "
                                                     "of every token read once and written once"})
        if fp8:
            objs["quant_ms_per_launch"] = round(t["quant"], 4)
    return objs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="480p", choices=["480p", "720p", "720p_fp8", "long", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8-unfused", action="store_true",
                    help="fp8 workload: run norm + RoPE and the quantisation as two calls (separate amax pass) "
                         "instead of wan_qknorm_rope_quant_fp8")
    ap.add_argument("--ring-cp", type=int, default=8, metavar="CP",
                    help="also time one GPU's share of ring attention with the sequence split over CP ranks "
                         "(bf16 workloads; 0 to skip)")
    ap.add_argument("--proj-reps", type=int, default=10, metavar="N",
                    help="timed calls of the QKV projection on the workload's tokens (bf16 workloads; 0 to skip)")
    ap.add_argument("--skip-threshold", type=float, default=0.02, metavar="T",
                    help="also time Skip-Softmax attention at this threshold against dense attention on a "
                         "local-score input of the workload's shape (bf16 workloads; 0 to skip)")
    ap.add_argument("--config-steps", type=int, default=5, metavar="N",
                    help="timed steps of each other workload (720p, 720p_fp8, long) reported next to the 480p "
                         "headline; 0 to skip them")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the steps, run one plain device copy of MIB MiB (its hardware "
                         "counters scale FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (the multi-GPU "
              "path is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch

    from video_diffusion_transformer_amd.configs import WORKLOADS

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    t, qkv = run_steps(w, dev, args.steps, args.warmup, args.fp8_unfused)
    fp8 = w.dtype == "fp8"
    dtype = "fp8" if fp8 else "bf16"
    flop = w.attn_flop()
    objs = kernel_objects(w, t, args.fp8_unfused)
    rec = {
        "metric": "attention TFLOP/s per DiT self-attention step (QK-norm+RoPE then bidirectional attention)",
        "value": round(flop / (t["step"] * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"wan2.2-a14b-{w.name}", "B": w.B, "grid_THW": [w.T, w.H, w.W], "S": w.S,
                   "heads": w.heads, "head_dim": w.head_dim},
        "roofline": objs.pop("attention"),
    }
    rec.update(objs)
    props = torch.cuda.get_device_properties(dev)
    rec["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                     "compute_units": props.multi_processor_count,
                     "hbm_GiB": round(props.total_memory / 2**30, 1)}
    if args.ring_cp:
        ring = ring_share(w, qkv, args.ring_cp)
        if ring:
            rec["ring_share"] = ring
    del qkv
    torch.cuda.empty_cache()
    proj = qkv_proj(w, dev, args.proj_reps)
    if proj:
        rec["qkv_proj"] = proj
    torch.cuda.empty_cache()
    sk = skip_softmax(w, dev, args.skip_threshold)
    if sk:
        rec["skip_softmax"] = sk
        torch.cuda.empty_cache()
    if args.workload == "480p" and args.config_steps > 0:
        for name in EXTRA_WORKLOADS:
            x = WORKLOADS[name]
            tx, q = run_steps(x, dev, args.config_steps, 2)
            del q
            torch.cuda.empty_cache()
            sub = {"workload": f"wan2.2-a14b-{x.name}", "dtype": x.dtype, "B": x.B, "grid_THW": [x.T, x.H, x.W],
                   "S": x.S, "steps": args.config_steps, "warmup": 2, "ms_per_step": round(tx["step"], 4),
                   "step_tflops": round(x.attn_flop() / (tx["step"] * 1e-3) / 1e12, 2)}
            sub.update(kernel_objects(x, tx))
            rec[name] = sub
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
