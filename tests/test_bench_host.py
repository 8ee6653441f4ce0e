"""Host-side parts of bench.py, checked without a GPU: the single-GPU refusal,
the counter-file lookup and the CPU-baseline record."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert r.stdout == ""  # no JSON line
    assert "exactly one GPU" in r.stderr


def test_traffic_lookup_follows_the_source_hash():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        data = json.load(f)
    for name, ent in data.items():
        got = bench.load_traffic(name)
        if ent.get("kernel_source_hash") == bench.kernel_source_hash():
            assert got == ent["bytes_per_launch"]
            # never far below the compulsory bytes (each operand read once, C
            # written once); the counters are scaled by a copy calibration
            assert got >= 0.95 * synth.WORKLOADS[name].compulsory_bytes, name
        else:
            assert got is None, name
    assert bench.load_traffic("no_such_workload") is None


@pytest.mark.parametrize("name", ["sq512_bf16_f32"])
def test_cpu_baseline_record(name):
    w = synth.WORKLOADS[name]
    rec = bench.cpu_baseline(w, target_s=0.2)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "%dx%dx%d" % (w.M, w.N, w.K) in rec["sample"]
