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


def test_placement_summary_reports_the_distribution():
    class A:
        placement = {"candidates": 3, "pass2_ms": [5.9, 5.1, 6.2], "kept": 1,
                     "refined": [[0, "grad", 2, [5.1, 5.3, 5.0]], [0, "param", 1, [5.0, 5.4]]]}
    out = bench.placement_summary(A, 3.25)
    assert out["whole_sets"] == {"n": 3, "kept_ms": 5.1, "median_ms": 5.9, "worst_ms": 6.2, "all_ms": [5.9, 5.1, 6.2]}
    assert out["per_array"][0] == {"array": "0.grad", "n": 3, "kept_ms": 5.0, "median_ms": 5.1, "worst_ms": 5.3}
    assert out["kept_pass2_ms"] == 5.0 and out["seconds"] == 3.25

    class B:
        placement = None
    assert bench.placement_summary(B, 1.0) == {"candidates": 1, "seconds": 1.0}


def test_default_workload_is_the_largest_one_gpu_workload():
    import synth
    ap_default = [line for line in open(os.path.join(ROOT, "bench.py")) if '"--workload", default=' in line]
    assert ap_default and '"dense-7b"' in ap_default[0]
    w = synth.WORKLOADS["dense-7b"]
    assert w.dp_size == 1  # the whole model's state on one GPU


def test_placement_summary_of_region_search():
    class A:
        placement = {"kind": "regions", "buffers": [
            {"buffer": 0, "regions": 3, "region_elems": 1 << 27, "sweeps": 2,
             "last_sweep": [[0, 0.70, 0.61, 5], [1, 0.62, 0.61, 0], [2, 0.20, 0.19, 2]]}]}
    out = bench.placement_summary(A, 5.0)
    b = out["buffers"][0]
    assert out["kind"] == "regions" and b["regions"] == 3 and b["region_ms_kept"] == 1.41
    assert b["region_ms_before_last_sweep"] == 1.52 and b["candidates_last_sweep"] == 7
    assert b["fastest_region_ms"] == 0.19 and b["slowest_region_ms"] == 0.61


def test_pass2_kernel_label_follows_the_layout():
    """The roofline names the pass-2 kernel the library chose for each buffer
    (dopt_buffer_info.apply_bnd), each kernel once, in buffer order."""
    import sharded_mixed_precision_amd as D
    from synth import PARAM_LISTS, WORKLOADS

    class A:
        def __init__(self, L):
            self.info = L.infos()

    labels = {}
    for name in ("dense-7b", "llama3-8b", "llama3-70b"):
        w = WORKLOADS[name]
        L = D.dopt_build_ranges(PARAM_LISTS[w.model](), w.dp_size, w.dp_rank, w.bucket_size, w.pad_for_high_busbw)
        labels[name] = bench.pass2_kernels(A(L))
    assert labels == {"dense-7b": "k_apply", "llama3-8b": "k_apply", "llama3-70b": "k_apply_bnd"}


def test_traffic_entries_cover_the_headline():
    # counters for the headline workload are stored (reported while their
    # source hash is the library's)
    assert "dense-7b" in bench.MEASURED_TRAFFIC
