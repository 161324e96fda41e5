"""Host-side pieces of the benchmark (no GPU): the HBM traffic it reports comes from the
committed counter summary and only while that summary describes the current kernel sources;
a request for more than one GPU is refused with a message."""
import os
import subprocess
import sys

import bench


def test_measured_traffic_follows_the_committed_counters():
    for k in ("logits_lse", "probs", "dh_gemm"):
        b = bench.measured_traffic(k, True)
        assert b is not None and b > 1e9, (k, b)  # GB per launch, HBM side
    assert bench.measured_traffic("probs", False) is None  # another workload: not profiled
    assert bench.measured_traffic("no_such_kernel", True) is None


def test_measured_traffic_is_dropped_when_the_sources_change(tmp_path, monkeypatch):
    # a copy of the summary whose recorded hash no longer matches the sources
    text = open(bench.COUNTERS_MD).read().replace("sources_sha256 = ", "sources_sha256 = 0")
    p = tmp_path / "counters.md"
    p.write_text(text)
    monkeypatch.setattr(bench, "COUNTERS_MD", str(p))
    assert bench.measured_traffic("probs", True) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)
