"""The C ABI driven by a native C++ program (tests/native/abi_step), with no
Python or PyTorch in the process that calls it: every device array is
hipMalloc'd by the program and the steps run on its own HIP stream (in one
mode through dopt_step, in the other through the fused reduce, the split
step, the state export and the scalar state).

The CPU test runs the program's layout mode (host-side mapper only) and
checks it against the Python binding's view of the same layout.  The GPU
tests feed it seeded synthetic params and grads (or received grad chunks)
through a file, run the steps, and compare the stats and every shard element
of the final state (and the reduced grads, the export and the scalar state)
with the oracle on the same inputs, to the bars of the other parity tests.
"""
import ctypes
import os
import struct
import subprocess

import numpy as np
import pytest

import oracle
import synth
from synth.models import ParamSpec
from tests import gpu_harness as H
from tests.oracle_harness import OracleRun, oracle_export, to_bits

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "native", "abi_step")
DT = {"f32": 0, "bf16": 1, "f16": 2}
ES = {"f32": 4, "bf16": 2, "f16": 2}

PARAMS = [ParamSpec("emb", 40_000, "bf16", "bf16", 0, 0), ParamSpec("w", 9_001, "bf16", "bf16", 0, 1),
          ParamSpec("norm", 700, "f32", "f32", 0, 0), ParamSpec("b", 333, "bf16", "bf16", 0, 1)]
N, R, BUCKET, STEPS, MAX_NORM = 3, 1, 20_000, 3, 1.0
HPS = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (3e-4, 0.8, 0.99, 1e-6, 0.0)]


def _exe():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built: run __graft_entry__.build()")
    return EXE


def _header(steps):
    h = struct.pack("<6i", 0x444F5054, len(PARAMS), N, R, steps, len(HPS))
    h += struct.pack("<q", BUCKET) + struct.pack("<d", MAX_NORM)
    for hp in HPS:
        h += struct.pack("<5d", *hp)
    for p in PARAMS:
        h += struct.pack("<q3i", p.numel, DT[p.param_dtype], DT[p.grad_dtype], p.hgroup)
    return h


def _binding_layout():
    import sharded_mixed_precision_amd as D
    return D, D.dopt_build_ranges(PARAMS, N, R, BUCKET)


def test_native_layout_mode_matches_binding(tmp_path):
    D, L = _binding_layout()
    f = tmp_path / "in.bin"
    f.write_bytes(_header(0))
    out = subprocess.run([_exe(), "layout", str(f)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    lines = out.stdout.split("\n")
    assert lines[0] == f"buffers {L.num_buffers} workspace {L.workspace_bytes}"
    for k in range(L.num_buffers):
        b = L.buffer(k)
        assert lines[1 + k] == f"buffer {k} arena_numel {b['arena_numel']} shard_numel {b['shard_numel']}"


@pytest.mark.gpu
def test_native_step_matches_oracle(tmp_path):
    D, L = _binding_layout()
    nb = L.num_buffers
    arena = [L.buffer(k)["arena_numel"] for k in range(nb)]
    run = OracleRun(PARAMS, N, R, BUCKET, arena_numel=arena)
    blob = [_header(STEPS), struct.pack(f"<{nb}q", *arena)]
    for k, b in enumerate(run.bufs):
        b["param"][:] = to_bits(synth.fill_normal(b["pd"], b["n"], 0, synth.weight_stream(k), 0, 0.02))
        blob.append(b["param"].tobytes())
    run.init_state()
    ref_stats = []
    for s in range(1, STEPS + 1):
        for k, b in enumerate(run.bufs):
            b["grad"][:] = to_bits(synth.fill_normal(b["gd"], b["n"], 0, synth.grad_stream(k), s, 1e-2))
            blob.append(b["grad"].tobytes())
        ref_stats.append(run.step(HPS, MAX_NORM))
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    fin.write_bytes(b"".join(blob))
    out = subprocess.run([_exe(), "run", str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    data = fout.read_bytes()
    sz = ctypes.sizeof(D.dopt_stats)
    off = 0
    for s, ref in enumerate(ref_stats):
        st = D.dopt_stats.from_buffer_copy(data[off:off + sz]).as_dict()
        off += sz
        H.check_stats(st, ref, s + 1)
    for k, b in enumerate(run.bufs):
        n = b["n"]
        valid = run.valid(k)
        keys = (["master"] if b["pd"] != "f32" else []) + ["m", "v"]
        for key in keys:
            got = np.frombuffer(data, np.float32, n, off)
            off += 4 * n
            H.check_f32(f"buffer {k} {key}", got[valid], b[key][valid])
        pdt = np.float32 if b["pd"] == "f32" else np.uint16
        got = np.frombuffer(data, pdt, n, off)
        off += ES[b["pd"]] * n
        H.check_param(f"buffer {k} param", got[valid].copy(), b["param"][valid].copy(), b["pd"])
    assert off == len(data)


@pytest.mark.gpu
def test_native_reduce_export_matches_oracle(tmp_path):
    """The reduce mode: per step the dp_size received bf16 chunks of each
    buffer go through dopt_reduce_prepare (fp32-accumulating reduce, scaled by
    1/dp_size, pass 1, finalize), dopt_step_apply and dopt_read_stats; then the
    state export and the scalar state.  Against the oracle's reduce and step
    on the same chunks: the stats, every reduced window slot and every shard
    element bit for bit, the export arrays bit for bit, and the step count."""
    D, L = _binding_layout()
    nb = L.num_buffers
    arena = [L.buffer(k)["arena_numel"] for k in range(nb)]
    run = OracleRun(PARAMS, N, R, BUCKET, arena_numel=arena)
    scale = 1.0 / N
    blob = [_header(STEPS), struct.pack(f"<{nb}q", *arena), struct.pack("<if", DT["bf16"], scale)]
    for k, b in enumerate(run.bufs):
        b["param"][:] = to_bits(synth.fill_normal(b["pd"], b["n"], 0, synth.weight_stream(k), 0, 0.02))
        blob.append(b["param"].tobytes())
    run.init_state()
    ref_stats = []
    for s in range(1, STEPS + 1):
        for k, b in enumerate(run.bufs):
            ch = synth.fill_normal("bf16", N * b["n"], 0, synth.chunk_stream(k), s, 1e-2)
            blob.append(to_bits(ch).tobytes())
            oracle.lib().or_reduce_chunks(run.L.handle, k, ch.data_ptr(), oracle.DTYPES["bf16"], N, b["n"],
                                          ctypes.c_float(scale), 0, b["n"], b["grad"].ctypes.data)
        ref_stats.append(run.step(HPS, MAX_NORM))
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    fin.write_bytes(b"".join(blob))
    out = subprocess.run([_exe(), "reduce", str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    data = fout.read_bytes()
    sz = ctypes.sizeof(D.dopt_stats)
    off = 0
    for s, ref in enumerate(ref_stats):
        st = D.dopt_stats.from_buffer_copy(data[off:off + sz]).as_dict()
        off += sz
        H.check_stats(st, ref, s + 1)
    for k, b in enumerate(run.bufs):
        n = b["n"]
        valid = run.valid(k)
        for key in (["master"] if b["pd"] != "f32" else []) + ["m", "v"]:
            got = np.frombuffer(data, np.float32, n, off)
            off += 4 * n
            H.check_f32(f"buffer {k} {key}", got[valid], b[key][valid])
        pdt = np.float32 if b["pd"] == "f32" else np.uint16
        got = np.frombuffer(data, pdt, n, off)
        off += ES[b["pd"]] * n
        H.check_param(f"buffer {k} param", got[valid].copy(), b["param"][valid].copy(), b["pd"])
    for k, b in enumerate(run.bufs):  # the last step's reduced grads, every window slot
        gdt = np.float32 if b["gd"] == "f32" else np.uint16
        got = np.frombuffer(data, gdt, b["n"], off)
        off += ES[b["gd"]] * b["n"]
        w = run.L.buffer(k)["window_numel"]  # the arena's tail past the window is tile padding
        assert np.array_equal(got[:w].view(np.uint8), b["grad"][:w].view(np.uint8)), f"buffer {k} reduced grad"
    sn = struct.unpack_from("<q", data, off)[0]
    off += 8
    assert sn == L.state_numel
    ref_ex = oracle_export(run)
    for key, ref in zip(("master", "exp_avg", "exp_avg_sq"), ref_ex):
        got = np.frombuffer(data, np.float32, sn, off)
        off += 4 * sn
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"export {key}"
    sc = struct.unpack_from("<qdqq", data, off)
    off += struct.calcsize("<qdqq")
    assert sc[0] == STEPS and sc[1] == 1.0, sc
    assert off == len(data)
