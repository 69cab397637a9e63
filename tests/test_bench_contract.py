"""CPU checks of bench.py's contract: one GPU only, the counter record in
profiles/ describes the executor sources as they stand, and the oracle
baseline leg returns what the JSON line carries."""
import os
import subprocess
import sys

import bench
from synth import WORKLOADS, make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_matches_the_executor_sources():
    # the HBM byte counters in profiles/ were taken on these exact sources;
    # an edit of the executor must come with new counters
    assert bench.measured_traffic("large", "token") is not None
    assert bench.measured_traffic("large", "expert") is not None
    assert bench.measured_traffic("large", "nonexistent") is None


def test_cpu_baseline_leg_reports_the_oracle():
    wl = WORKLOADS["tiny"]
    cpu = bench.cpu_baseline(make_inputs(wl), wl, target_s=0.05)
    assert cpu["kind"] == "oracle" and cpu["unit"] == "routed tokens/s"
    assert cpu["value"] > 0 and cpu["cores"] >= 1 and "tokens" in cpu["sample"]
