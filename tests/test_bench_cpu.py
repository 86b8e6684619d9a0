"""bench.py's contract checks that need no GPU: a request for more than one
GPU is refused with a message and exit status 2 before anything touches a
device, and the counter-derived traffic is reported only for the kernel
source it was measured on."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_only_for_the_measured_kernel_source():
    digest = bench.kernel_digest()
    with open(bench.TRAFFIC_FILE) as f:
        recorded = [l.split(":", 1)[1].strip() for l in f if l.startswith("kernel_digest:")]
    assert recorded, "the traffic summary names the kernel source it was taken on"
    t = bench.measured_traffic(digest)
    if recorded[0] == digest:
        assert t is not None and t > bench.algorithmic_bytes(_bench_workload())
    else:
        assert t is None
    assert bench.measured_traffic("0" * 16) is None


def _bench_workload():
    from mamba_selective_scan_causal_amd import inputs as gen
    return gen.MAMBA_2P8B
