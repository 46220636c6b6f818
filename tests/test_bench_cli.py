"""bench.py's command-line contract on the CPU: more than one GPU is
refused with a message and exit status 2, and the traffic lookup reports
nothing for workloads without committed counters."""

import os
import subprocess
import sys

from tests.conftest import ROOT


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_lookup_only_for_profiled_workloads():
    sys.path.insert(0, ROOT)
    import bench

    assert bench.measured_traffic("c1", "f16x3") is None
    assert bench.measured_traffic("c3", "bf16x3") is None  # the bf16 operand variant was not profiled
    v = bench.measured_traffic("c3", "f16x3")
    assert v is None or v > 1e8  # None once the library's sources change after the counters were taken
    assert len(bench.sources_digest()) == 64
