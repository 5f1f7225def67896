"""bench.py's host-side contract (no GPU): more than one GPU is refused with a
message and a non-zero status before anything touches a device, the
committed counter summaries it reads parse, and the roofline objects follow
from the measured times by the stated arithmetic."""

import glob
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")


def test_committed_traffic_records_parse():
    files = glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json"))
    assert files
    for f in files:
        rec = json.load(open(f))
        assert rec["hbm_bytes_per_launch"] > 0
        assert len(rec["source_sha256_16"]) == 16
        assert all("rocprofv3 --pmc" in c for c in rec["commands"])


def _bench_module():
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402
    return bench


def test_kernel_objects_arithmetic():
    """The roofline objects of one step from given phase times: attention FLOP
    per launch over its time against the bf16 peak, the norm's algorithmic
    bytes over its time against 8 TB/s, and the norm against a device copy of
    the same bytes."""
    from video_diffusion_transformer_amd.configs import WORKLOADS
    bench = _bench_module()
    w = WORKLOADS["480p"]
    t = {"step": 33.0, "norm": 0.5, "quant": 0.0, "attn": 32.5, "copy": 0.6}
    o = bench.kernel_objects(w, t)
    a = o["attention"]
    flop = 4.0 * 2 * 40 * 32760 ** 2 * 128
    assert a["flop_per_launch"] == flop
    assert abs(a["achieved"] - flop / 32.5e-3 / 1e12) < 0.01
    assert abs(a["frac"] - a["achieved"] / 2500.0) < 1e-4
    n = o["qknorm_rope"]
    nbytes = 4.0 * 2 * 32760 * 5120 * 2
    assert n["bytes_per_launch"] == nbytes
    assert abs(n["achieved"] - nbytes / 0.5e-3 / 1e9) < 0.1
    assert abs(n["frac"] - n["achieved"] / 8000.0) < 1e-4
    assert abs(n["copy_GBps"] - nbytes / 0.6e-3 / 1e9) < 0.1
    assert abs(n["frac_of_copy"] - 0.6 / 0.5) < 1e-3


def test_kernel_objects_fp8():
    """The fp8 step: attention against the fp8 peak, the fused prep's bytes
    (norm + amax + quantisation) over its time."""
    from video_diffusion_transformer_amd.configs import WORKLOADS
    bench = _bench_module()
    w = WORKLOADS["720p_fp8"]
    t = {"step": 120.0, "norm": 2.7, "quant": 0.0, "attn": 115.0, "prep_delayed": 1.8}
    o = bench.kernel_objects(w, t)
    a = o["attention"]
    assert a["peak"] == 5000.0 and a["kernel"] == "attn_fwd_fp8"
    assert abs(a["frac"] - a["flop_per_launch"] / 115.0e-3 / 1e12 / 5000.0) < 1e-4
    p = o["qknorm_rope_quant_fp8"]
    assert p["bytes_per_launch"] == 2 * 75600 * 5120 * 19
    d = o["qknorm_rope_quant_fp8_delayed"]
    assert d["bytes_per_launch"] == 2 * 75600 * 5120 * 9
    assert "qknorm_rope" not in o
