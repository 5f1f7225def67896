"""Benchmark of one Wan2.2 DiT self-attention step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 480p|720p|720p_fp8|long]

A step is the whole hot path over one batch of synthetic input already resident
in HBM: in-place Q/K RMSNorm + bf16 rounding + 3-D RoPE on the packed [Q|K|V]
buffer, then bidirectional attention over every token (the fp8 workload adds
the per-tensor e4m3 quantisation, its amax taken in the norm pass, and runs
attention on fp8 MFMA). W untimed
warm-up steps, then K timed steps between device synchronisations. One JSON
line is printed.

  value       attention FLOP of one step (4 * B * heads * S^2 * 128) divided by
              the measured time of the whole step, in TFLOP/s.
  roofline    the dominant kernel (attention): algorithmic FLOP per launch over
              its average launch time from HIP events recorded on the stream it
              runs on, against the dense MFMA peak of its dtype; ``traffic`` is
              the HBM bytes per launch from the committed rocprofv3 counter
              summary when it was taken on the current kernel source, else null.
  cpu_baseline the fp64 numpy oracle on the host cores, on a bounded sample of
              the same workload (query rows of one head against all keys).
  ring_share  (bf16 workloads) one GPU's share of ring attention with the
              sequence split over --ring-cp ranks: S/cp queries against cp
              K/V chunks, each round folded into the accumulator by the
              log-sum-exp merge; not part of the step or of value.
  qkv_proj    (bf16 workloads) the QKV projection x W^T + b that produces the
              packed [Q|K|V] buffer the step reads: FLOP per launch over the
              launch time from HIP events on its stream, against the bf16
              MFMA peak; not part of the step or of value.
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
KERNEL_SOURCES = {"attn_fwd": "attn_fwd.hip", "attn_fwd_fp8": "attn_fwd_fp8.hip",
                  "qknorm_rope": "qknorm_rope.hip", "qkv_proj": "qkv_proj.hip"}


def kernel_source_hash(name):
    path = os.path.join(ROOT, "video_diffusion_transformer_amd", "csrc", KERNEL_SOURCES[name])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


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


def cpu_baseline(w, budget_s=12.0):
    """Time the oracle's attention on query rows of (b=0, h=0) against all S
    keys until about ``budget_s`` seconds of CPU work are done."""
    import numpy as np
    import torch

    from oracle import wan_ref
    from video_diffusion_transformer_amd import synth

    cores = len(os.sched_getaffinity(0))
    torch.manual_seed(0)
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
    del synth
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} query rows of head 0 x all {w.S} keys, fp64 numpy (BLAS threads = "
                      f"{cores}), {dt:.1f} s; full-step time extrapolated: "
                      f"{w.attn_flop() / (flop / dt):.0f} s"}


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
    fused weight [3D, D] plus bias into the packed [B, S, 3D] buffer. One
    warm-up call, then reps calls timed with HIP events on the stream."""
    import torch

    from video_diffusion_transformer_amd import synth, wan_attn

    if reps < 1 or w.dtype != "bf16":
        return None
    x = synth.make_tokens(w.B, w.S, w.D, seed=w.seed, device=dev)
    wq, bq = synth.make_qkv_weights(w.D, seed=w.seed, device=dev)
    out = torch.empty((w.B, w.S, 3 * w.D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    wan_attn.qkv_proj(x, wq, w.heads, bias=bq, out=out)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        wan_attn.qkv_proj(x, wq, w.heads, bias=bq, out=out)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    flop = 2.0 * w.B * w.S * 3 * w.D * w.D
    tf = flop / (ms * 1e-3) / 1e12
    del x, wq, bq, out
    return {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
            "frac": round(tf / PEAK_TFLOPS["bf16"], 4), "ms_per_launch": round(ms, 4), "flop_per_launch": flop,
            "traffic": committed_traffic("qkv_proj", w.name)}


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
    ap.add_argument("--proj-reps", type=int, default=3, metavar="N",
                    help="timed calls of the QKV projection on the workload's tokens (bf16 workloads; 0 to skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the steps, run one plain device copy of MIB MiB (its hardware "
                         "counters scale FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (the multi-GPU "
              "path is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch

    from video_diffusion_transformer_amd import synth, wan_attn
    from video_diffusion_transformer_amd.configs import WORKLOADS

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    grid = (w.T, w.H, w.W)
    qkv = synth.make_qkv(w.B, w.S, w.heads, seed=w.seed, device=dev)
    gq, gk = synth.make_gammas(w.D, seed=w.seed, device=dev)
    out = torch.empty((w.B, w.S, w.D), dtype=torch.bfloat16, device=dev)
    fp8 = w.dtype == "fp8"
    if fp8:
        f8 = wan_attn.fp8_buffers(w.B, w.S, w.heads, dev)
    stream = torch.cuda.current_stream(dev)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(ev=None):
        if ev: ev[0].record(stream)
        if fp8 and not args.fp8_unfused:
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

    if args.copy_calibration:
        n = args.copy_calibration * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[E() for _ in range(4)] for _ in range(args.steps)]
    t0 = E()
    t1 = E()
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    norm_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    quant_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    attn_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps

    dtype = "fp8" if fp8 else "bf16"
    flop = w.attn_flop()
    attn_tflops = flop / (attn_ms * 1e-3) / 1e12
    norm_gbs = w.norm_bytes() / (norm_ms * 1e-3) / 1e9
    kname = "attn_fwd_fp8" if fp8 else "attn_fwd"
    traffic = committed_traffic(kname, w.name)
    rec = {
        "metric": "attention TFLOP/s per DiT self-attention step (QK-norm+RoPE then bidirectional attention)",
        "value": round(flop / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"wan2.2-a14b-{w.name}", "B": w.B, "grid_THW": list(grid), "S": w.S,
                   "heads": w.heads, "head_dim": w.head_dim},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_TFLOPS[dtype],
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_TFLOPS[dtype], 4),
                     "traffic": traffic, "kernel": kname, "ms_per_launch": round(attn_ms, 4),
                     "flop_per_launch": flop},
        "qknorm_rope": {"bound": "hbm", "achieved": round(norm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(norm_gbs / PEAK_HBM_GBS, 4), "ms_per_launch": round(norm_ms, 4),
                        "bytes_per_launch": w.norm_bytes(),
                        "traffic": committed_traffic("qknorm_rope", w.name)},
    }
    if fp8 and not args.fp8_unfused:
        # one call: norm + RoPE + amax (reads Q, K, V; writes Q, K), then the
        # quantisation (reads Q, K, V; writes e4m3 Q, K, V^T)
        del rec["qknorm_rope"]
        prep_bytes = w.B * w.S * w.D * (8 + 2 + 6 + 3)
        rec["qknorm_rope_quant_fp8"] = {
            "bound": "hbm", "achieved": round(prep_bytes / (norm_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(prep_bytes / (norm_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "ms_per_launch": round(norm_ms, 4), "bytes_per_launch": prep_bytes}
    elif fp8:
        rec["quant_ms_per_launch"] = round(quant_ms, 4)
    if args.ring_cp:
        ring = ring_share(w, qkv, args.ring_cp)
        if ring:
            rec["ring_share"] = ring
    proj = qkv_proj(w, dev, args.proj_reps)
    if proj:
        rec["qkv_proj"] = proj
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
