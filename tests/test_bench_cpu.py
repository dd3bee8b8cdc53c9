"""The parts of bench.py that run without a GPU: the refusal of more than one
GPU, and the per-element byte counts behind its roofline figures."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_step_bytes_per_element():
    # pass 1 reads the grad; pass 2 re-reads it, reads and writes master
    # (or the fp32 param), m and v, and writes a 16-bit param
    assert bench.pass_bytes("bf16", "bf16") == (2, 28)
    assert bench.pass_bytes("f16", "f16") == (2, 28)
    assert bench.pass_bytes("bf16", "f32") == (4, 30)
    assert bench.pass_bytes("f32", "f32") == (4, 28)
    assert sum(bench.pass_bytes("bf16", "bf16")) == 30 and sum(bench.pass_bytes("bf16", "f32")) == 34


def test_traffic_is_reported_only_for_the_measured_source():
    # the stored PMC traffic belongs to one version of the kernels' source
    for entry in bench.MEASURED_TRAFFIC.values():
        assert len(entry["src"]) == 16 and entry["bytes_per_launch"] > 0
    assert len(bench._src_sha()) == 16


def test_cpu_baseline_host_description():
    h = bench.host_cpu()
    assert h["cores_available"] >= 1 and isinstance(h["model"], str) and h["model"]
