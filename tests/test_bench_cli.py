"""bench.py's host-side contract (no GPU): more than one GPU is refused with a
message and a non-zero status before anything touches a device, and the
committed counter summaries it reads parse."""

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
