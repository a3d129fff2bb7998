"""Host-side behaviour of bench.py that needs no GPU: the one-GPU contract and
the rule that recorded HBM counters are reported only for the kernel source
they were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line for a refused run


def test_traffic_reported_only_for_the_profiled_source(monkeypatch):
    import bench
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    kernel = "bwd_dkdv"
    assert kernel in rec and rec[kernel]["bytes_per_launch"] > 0
    monkeypatch.setattr(bench, "source_hash", lambda name: rec[kernel]["source_hash"])
    assert bench.traffic_for(kernel) == rec[kernel]["bytes_per_launch"]
    monkeypatch.setattr(bench, "source_hash", lambda name: "0" * 16)
    assert bench.traffic_for(kernel) is None


@pytest.mark.parametrize("kernel", ["fwd", "bwd_dkdv", "bwd_dq"])
def test_kernel_sources_exist(kernel):
    import bench
    path = os.path.join(ROOT, "io_aware_exact_20_amd", "csrc", bench.KERNEL_SOURCES[kernel])
    assert os.path.exists(path)
