"""Host-side checks of bench.py (CPU): the committed HBM-traffic summary is in
step with the kernel sources it was taken on, the traffic lookup only answers
for a matching source digest, and a multi-GPU request is refused."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

# the kernel-source set behind each workload's GEMM1 line in hbm_traffic.txt
WORKLOAD_SOURCES = {"decode": "small", "skew@1": "small", "prefill": "large", "fp8": "large_q",
                    "mxfp8": "large_q", "fp8@8192": "large_q", "mxfp8@8192": "large_q"}


def _traffic_lines():
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    return [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]


def test_traffic_summary_matches_current_sources():
    lines = _traffic_lines()
    seen = set()
    for f in lines:
        wl = f[0].split("/")[0]
        assert wl in WORKLOAD_SOURCES, f[0]
        assert f[1] == bench.kernel_source_digest(WORKLOAD_SOURCES[wl]), \
            f"{f[0]}: counters taken on other kernel sources (re-run the traffic passes)"
        seen.add(f[0])
    for wl in WORKLOAD_SOURCES:
        assert wl in seen and wl + "/gemm2" in seen, wl


def test_read_traffic_needs_the_digest():
    f = next(x for x in _traffic_lines() if x[0] == "decode")
    assert bench.read_traffic("decode", f[1]) == pytest.approx(float(f[3]))
    assert bench.read_traffic("decode", "0" * 16) is None
    assert bench.read_traffic("no-such-workload", f[1]) is None


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
