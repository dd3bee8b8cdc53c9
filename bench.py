"""Benchmark of the shard-local mixed-precision AdamW step on one MI355X.

A step is one call of dopt_step over one rank's shard: pass 1 (unscale,
inf/NaN, sum of squares, zero count), the one-workgroup fixed-order
reduction fused with the finalize (skip, norm, clip, loss scale, step
count), then pass 2 (clip + AdamW + bias correction + write-back).  Inputs
are synthetic (seeded model-shaped param lists) and resident in HBM before
the timed region.  The timed region holds the K steps and nothing else (an
event between two kernels adds a few microseconds on MI355X, so none is
recorded inside it).  The launch duration of pass 2 for the roofline comes
from K further steps, each running pass 2 APPLY_BATCH times back to back
between two HIP events on the launch stream (the repeats apply the step's
own scalars again: the same kernel, launch configuration and bytes), so the
events' own cost is spread over the batch.  Last, K steps run with the
256 MB last-level cache flushed before each (`llc_flushed`): back-to-back
steps of a small window find much of their data still in that cache.

Prints one JSON line.  The headline workload is the dense 7B list at N=1
(6.74e9 fp16 params with fp16 grads under a dynamic loss scale: the largest
workload that one GPU holds whole, 202 GB moved per step); the line also
carries, under "secondary", the GPT-2-small-shaped rank (N=8, rank 3) with its
step timed back to back and with the last-level cache flushed, and the
distribution of pass-2 times over the arena placements the start-up search
tried.  Inputs are seeded draws of PyTorch's device generator (the parity
tests use the host generator of synth/; the step's speed does not depend on
the values).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
METRIC = "shard AdamW step: Gparams/s and achieved HBM GB/s (% of peak), 1 MI355X"
ES = {"f32": 4, "bf16": 2, "f16": 2}
APPLY_BATCH = 10  # pass-2 launches between one pair of events (roofline timing)
SMALL_WINDOW = 64 << 20  # shard elements up to which the default step counts are large
REGION_ELEMS = 1 << 27  # arena elements per placement region

# HBM traffic of pass 2 (k_apply, or k_apply_bnd for Llama-3-70B, whose window
# has boundary tiles) measured with rocprofv3 PMC counters (FETCH_SIZE,
# WRITE_SIZE) and scaled by the same counters on a plain copy of known size;
# reported only while the kernel source is the one that was measured.
# bytes_per_launch = FETCH_SIZE * 2.0 + WRITE_SIZE * 1.0 (KiB -> B), the scale
# factors read off a 1 GiB fp32 copy.
MEASURED_TRAFFIC = {
    # FETCH_SIZE 106,556.68 KiB * 2.0 + WRITE_SIZE 213,569.33 KiB * 1.0, averaged over 523 dispatches
    # (profiles/k_apply_gpt2-small_kernel_trace.md)
    "gpt2-small": {"src": "53d67aba3946e0d0", "bytes_per_launch": 436923071},
    # FETCH_SIZE 46,269,131.90 KiB * 2.0 + WRITE_SIZE 92,127,420.10 KiB * 1.0, averaged over the 37
    # full-window dispatches that were not overflow-skipped (profiles/k_apply_dense-7b_kernel_trace.md)
    "dense-7b": {"src": "53d67aba3946e0d0", "bytes_per_launch": 189097660323},
    # k_apply_bnd: FETCH_SIZE 7,569,690.44 KiB * 2.0 + WRITE_SIZE 15,072,217.06 KiB * 1.0, averaged over 37
    # dispatches (profiles/k_apply_llama3-70b_kernel_trace.md)
    "llama3-70b": {"src": "53d67aba3946e0d0", "bytes_per_launch": 30936676290},
    # both buffers' launches of one step (the bf16-param / fp32-grad window and the fp32 norms):
    # FETCH_SIZE 7,872,477.81 + 310.13 KiB * 2.0 + WRITE_SIZE 13,723,600.49 + 390.00 KiB * 1.0, averaged
    # over 37 dispatches each (profiles/k_apply_llama3-8b_kernel_trace.md)
    "llama3-8b": {"src": "53d67aba3946e0d0", "bytes_per_launch": 30176835961},
}


def progress(msg: str):
    """A progress line on stderr (the JSON result is the only stdout line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _src_sha() -> str:
    h = hashlib.sha256()
    for f in ("sharded_mixed_precision_amd/csrc/step.hip", "sharded_mixed_precision_amd/csrc/internal.h"):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pass_bytes(pd: str, gd: str):
    """Algorithmic HBM bytes per shard element: (pass 1, pass 2).

    Pass 1 reads the grad.  Pass 2 reads grad, master (or the fp32 param),
    m, v and writes master, m, v and, for 16-bit params, the param."""
    p1 = ES[gd]
    p2 = ES[gd] + 12 + 12 + (ES[pd] if pd != "f32" else 0)
    return p1, p2


def host_cpu() -> dict:
    """The host's processor model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "cores_available": len(os.sched_getaffinity(0))}


def cpu_baseline(workload, seconds: float):
    """The oracle (plain single-threaded C) on a bounded sample of the same
    workload, with the calling thread pinned to one core for the timing."""
    mask = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {min(mask)})
    try:
        res = _cpu_baseline(workload, seconds)
    finally:
        os.sched_setaffinity(0, mask)
    res["host"] = host_cpu()
    res["host"]["pinned_core"] = min(mask)
    threads = min(16, len(mask))
    if threads > 1:
        th = _cpu_threaded(workload, seconds / 2, threads)
        if th is not None:
            res["threaded"] = th
    return res


def _large_sample(workload):
    """The oracle's inputs for the first 2^24 arena slots of buffer 0 of a
    large rank window (seeded like the GPU run's inputs); None for a window
    of at most 2^25 shard elements."""
    import numpy as np
    import oracle
    import synth
    from tests.oracle_harness import to_bits

    params = synth.PARAM_LISTS[workload.model]()
    O = oracle.Layout(params, workload.dp_size, workload.dp_rank, workload.bucket_size)
    if sum(O.buffer(k)["shard_numel"] for k in range(O.num_buffers)) <= (1 << 25):
        return None  # a small window: the baseline runs whole oracle steps instead
    lib = oracle.lib()
    b0 = O.buffer(0)
    pd, gd = {0: "f32", 1: "bf16", 2: "f16"}[b0["param_dtype"]], {0: "f32", 1: "bf16", 2: "f16"}[b0["grad_dtype"]]
    n = min(1 << 24, b0["window_numel"])
    g = to_bits(synth.fill_normal(gd, n, 0, synth.grad_stream(0), 1, workload.grad_sigma)).copy()
    p = to_bits(synth.fill_normal(pd, n, 0, synth.weight_stream(0), 0, 0.02)).copy()
    master = np.zeros(n, np.float32)
    if pd == "bf16":
        lib.or_bf16_to_f32_n(p.ctypes.data, master.ctypes.data, n)
    elif pd == "f16":
        lib.or_f16_to_f32_n(p.ctypes.data, master.ctypes.data, n)
    return {"O": O, "lib": lib, "pd": pd, "gd": gd, "n": n, "g": g, "p": p, "master": master,
            "m": np.zeros(n, np.float32), "v": np.zeros(n, np.float32), "hg": np.zeros(n, np.int32)}


def _cpu_threaded(workload, seconds: float, threads: int):
    """Context beside the oracle, not the oracle itself: the oracle's range
    functions on `threads` disjoint slices of the same large-window sample,
    run on host threads (the library releases the interpreter lock), the
    statistics of the slices added in slice order.  None for small windows."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor

    S = _large_sample(workload)
    if S is None:
        return None
    lib, n = S["lib"], S["n"]
    ES_ = {"f32": 4, "bf16": 2, "f16": 2}
    eg, ep = ES_[S["gd"]], ES_[S["pd"]]
    cut = [(n * i // threads) // 2048 * 2048 for i in range(threads)] + [n]
    ranges = [(cut[i], cut[i + 1]) for i in range(threads) if cut[i + 1] > cut[i]]
    hp = [(workload.lr, workload.beta1, workload.beta2, workload.eps, workload.weight_decay)]
    sc = oracle.make_scaler(workload.dynamic_scale, workload.initial_scale)
    t = ctypes.c_int64(0)
    inv = lib.or_inv_scale(ctypes.byref(sc))

    def stats(r):
        st = oracle.Stats()
        lib.or_grad_stats_range(S["O"].handle, 0, S["g"].ctypes.data, inv, r[0], r[1], ctypes.byref(st))
        return st

    def apply(r, s):
        lo, cnt = r[0], r[1] - r[0]
        lib.or_apply_elems(oracle.DTYPES[S["pd"]], oracle.DTYPES[S["gd"]], cnt, S["hg"].ctypes.data + 4 * lo,
                           S["g"].ctypes.data + eg * lo, S["master"].ctypes.data + 4 * lo, S["m"].ctypes.data + 4 * lo,
                           S["v"].ctypes.data + 4 * lo, S["p"].ctypes.data + ep * lo, ctypes.byref(s))

    steps, t0 = 0, time.perf_counter()
    with ThreadPoolExecutor(len(ranges)) as pool:
        while True:
            parts = list(pool.map(stats, ranges))
            st = oracle.Stats()
            for q in parts:
                st.sumsq += q.sumsq
                st.zeros += q.zeros
                st.found_inf = st.found_inf or q.found_inf
            s = oracle.Scalars()
            lib.or_decide(ctypes.byref(st), ctypes.byref(sc), ctypes.byref(t), oracle.make_hparams(hp), 1,
                          workload.max_grad_norm, ctypes.byref(s))
            list(pool.map(lambda r: apply(r, s), ranges))
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": round(n * steps / el / 1e9, 6), "unit": "Gparams/s", "threads": len(ranges),
            "kind": "the oracle's range functions on disjoint slices of the sample, on host threads; "
                    "context beside the oracle, not the oracle",
            "sample": f"first {n} arena slots of buffer 0, {steps} stats+update passes in {el:.1f}s"}


def _cpu_baseline(workload, seconds: float):
    import oracle
    import synth
    from tests.oracle_harness import OracleRun, to_bits

    params = synth.PARAM_LISTS[workload.model]()
    O = oracle.Layout(params, workload.dp_size, workload.dp_rank, workload.bucket_size)
    E = sum(O.buffer(k)["shard_numel"] for k in range(O.num_buffers))
    hp = [(workload.lr, workload.beta1, workload.beta2, workload.eps, workload.weight_decay)]
    if E <= (1 << 25):
        run = OracleRun(params, workload.dp_size, workload.dp_rank, workload.bucket_size)
        for k, b in enumerate(run.bufs):
            b["param"][:] = to_bits(synth.fill_normal(b["pd"], b["n"], 0, synth.weight_stream(k), 0, 0.02))
            b["grad"][:] = to_bits(synth.fill_normal(b["gd"], b["n"], 0, synth.grad_stream(k), 1, workload.grad_sigma))
        run.init_state()
        steps, t0 = 0, time.perf_counter()
        while True:
            run.step(hp, workload.max_grad_norm)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        return {"value": round(E * steps / el / 1e9, 6), "unit": "Gparams/s", "cores": 1, "kind": "oracle",
                "sample": f"whole rank window ({E} shard elements), {steps} full oracle steps in {el:.1f}s, "
                          f"1 thread"}
    # large windows: the oracle's per-element stats + update on the first
    # 2^24 arena slots of buffer 0 (same arithmetic per element as a full step)
    S = _large_sample(workload)
    lib, n, pd, gd = S["lib"], S["n"], S["pd"], S["gd"]
    g, p, master, m, v, hg = S["g"], S["p"], S["master"], S["m"], S["v"], S["hg"]
    sc = oracle.make_scaler(workload.dynamic_scale, workload.initial_scale)
    t = ctypes.c_int64(0)
    steps, t0 = 0, time.perf_counter()
    while True:
        st = oracle.Stats()
        lib.or_grad_stats_range(S["O"].handle, 0, g.ctypes.data, lib.or_inv_scale(ctypes.byref(sc)), 0, n,
                                ctypes.byref(st))
        s = oracle.Scalars()
        lib.or_decide(ctypes.byref(st), ctypes.byref(sc), ctypes.byref(t), oracle.make_hparams(hp), 1,
                      workload.max_grad_norm, ctypes.byref(s))
        lib.or_apply_elems(oracle.DTYPES[pd], oracle.DTYPES[gd], n, hg.ctypes.data, g.ctypes.data,
                           master.ctypes.data, m.ctypes.data, v.ctypes.data, p.ctypes.data, ctypes.byref(s))
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(n * steps / el / 1e9, 6), "unit": "Gparams/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} arena slots of buffer 0 of the rank window, {steps} oracle stats+update "
                      f"passes in {el:.1f}s, 1 thread"}


def skip_step(L, A, step, K: int, stream):
    """An overflow step: one grad element of the first shard set to +inf, so
    pass 1 finds it and pass 2 writes nothing.  Timed over K steps with
    nothing else in the timed region; the bytes are pass 1's (the grad)."""
    import torch
    import sharded_mixed_precision_amd as D

    p0 = next(L.param(p) for p in range(L.n_params) if L.param(p)["has_shard"])
    A.bufs[p0["buffer"]]["grad"][p0["arena_offset"]] = float("inf")
    step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(K):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    st = D.dopt_read_stats(L, A.workspace, stream)
    assert st["skipped"] == 1 and st["found_inf"] == 1, st
    ms = t0.elapsed_time(t1) / K
    nbytes = sum(ES[info["gd"]] * info["shard_numel"] for info in A.info)
    return {"ms_per_step": round(ms, 5), "bytes_per_step": nbytes, "hbm_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "steps": K}


def bench_reduce(args, w, L, A, bufs_c, hp_c, stream):
    """The local half of a reduce-scatter with fp32 accumulation fused with
    pass 1: dp_size bf16 chunks per window slot are summed in fp32 and written
    to the grad arena, and the stats run on the stored value."""
    import torch
    import sharded_mixed_precision_amd as D

    N = w.dp_size
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    chunks = []
    bytes_call = 0
    for k, info in enumerate(A.info):
        t = torch.empty(N * info["n"], dtype=torch.bfloat16, device="cuda")
        t.normal_(0.0, w.grad_sigma, generator=gen)  # seeded synthetic chunks, drawn on the device
        chunks.append(t)
        bytes_call += info["window_numel"] * (N * 2 + ES[info["gd"]])
    for _ in range(args.warmup):
        D.dopt_reduce_prepare(L, bufs_c, chunks, "bf16", N, 1.0, hp_c, w.max_grad_norm, A.workspace, stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev:
        a.record(stream)
        D.dopt_reduce_prepare(L, bufs_c, chunks, "bf16", N, 1.0, hp_c, w.max_grad_norm, A.workspace, stream)
        b.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    gbps = bytes_call / (ms * 1e-3) / 1e9
    E = sum(info["window_numel"] for info in A.info)
    print(json.dumps({
        "metric": "fused local fp32-accumulating reduce of dp_size bf16 chunks + pass 1, 1 MI355X",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_call": round(ms, 5), "higher_is_better": True, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: rank {w.dp_rank} of N={N}, {E} window slots, {N} bf16 chunks each",
                   "bytes_per_call": bytes_call},
        "roofline": {"bound": "hbm", "kernel": "k_reduce_stats (+ k_finish)", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None, "algorithmic_bytes_per_call": bytes_call},
    }), flush=True)


def bench_check(args, w, L, A, stream):
    """The pre-communication scan of every bucket of the rank's whole local
    grad buffers (read only)."""
    import torch
    import sharded_mixed_precision_amd as D

    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    bufs, outs, total = [], [], 0
    for k in range(L.num_buffers):
        info = L.buffer(k)
        gd = D.DTYPE_NAMES[info["grad_dtype"]]
        t = torch.empty(info["numel"], dtype={"f32": torch.float32, "bf16": torch.bfloat16,
                                              "f16": torch.float16}[gd], device="cuda")
        t.normal_(0.0, w.grad_sigma, generator=gen)  # seeded synthetic local grads, drawn on the device
        bufs.append(t)
        outs.append(torch.zeros(info["n_buckets"] * D.BUCKET_CHECK_BYTES, dtype=torch.uint8, device="cuda"))
        total += info["numel"] * ES[gd]

    def call():
        for k in range(L.num_buffers):
            D.dopt_check_grads(L, k, bufs[k], 1.0, outs[k], A.workspace, stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    gbps = total / (ms * 1e-3) / 1e9
    numel = sum(L.buffer(k)["numel"] for k in range(L.num_buffers))
    print(json.dumps({
        "metric": "whole-bucket NaN/Inf/large-grad scan of a rank's local grad buffers, 1 MI355X",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_call": round(ms, 5), "higher_is_better": True, "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"{w.name}: {numel} buffer elements, "
                               f"{sum(L.buffer(k)['n_buckets'] for k in range(L.num_buffers))} buckets",
                   "bytes_per_call": total},
        "roofline": {"bound": "hbm", "kernel": "k_check (+ k_check_finish)", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None, "algorithmic_bytes_per_call": total},
    }), flush=True)


def bench_checkpoint(args, w, L, A, bufs_c, stream):
    """Model-space export of the rank's (master, m, v) shards and the import
    back (which also rewrites the 16-bit params from the master)."""
    import torch
    import sharded_mixed_precision_amd as D

    n = L.state_numel
    ex = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    exp_bytes = imp_bytes = 0
    for info in A.info:
        exp_bytes += 24 * info["shard_numel"]  # read master, m, v; write three fp32 exports
        imp_bytes += (24 + (ES[info["pd"]] if info["pd"] != "f32" else 0)) * info["shard_numel"]

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / len(ev)

    ms_e = timed(lambda: D.dopt_state_export(L, bufs_c, *ex, A.workspace, stream))
    ms_i = timed(lambda: D.dopt_state_import(L, bufs_c, *ex, A.workspace, stream))
    ge = exp_bytes / (ms_e * 1e-3) / 1e9
    gi = imp_bytes / (ms_i * 1e-3) / 1e9
    print(json.dumps({
        "metric": "model-space optimizer-state export of a rank's (master, m, v) shards, 1 MI355X",
        "value": round(ge, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_call": round(ms_e, 5), "higher_is_better": True, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: rank {w.dp_rank} of N={w.dp_size}, {n} shard elements",
                   "bytes_per_call": exp_bytes},
        "roofline": {"bound": "hbm", "kernel": "k_state_copy (export)", "achieved": round(ge, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ge / HBM_PEAK_GBPS, 4),
                     "traffic": None, "algorithmic_bytes_per_call": exp_bytes},
        "import": {"ms_per_call": round(ms_i, 5), "GBps": round(gi, 1), "frac": round(gi / HBM_PEAK_GBPS, 4),
                   "algorithmic_bytes_per_call": imp_bytes},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 500 on windows of up to 64M shard elements, else 20)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: 200 on windows of up to 64M shard elements, else 3)")
    ap.add_argument("--workload", default="dense-7b",
                    help="the headline workload (default: the 7B dense list at N=1, the largest one-GPU workload)")
    ap.add_argument("--secondary", default="gpt2-small",
                    help="step mode: a second workload measured after the first and reported under 'secondary' "
                         "with its own default step counts ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=["step", "reduce", "check", "checkpoint"], default="step",
                    help="step: the optimizer step (default); reduce: the fused local fp32-accumulating reduce of "
                         "dp_size received bf16 chunks + pass 1 (dopt_reduce_prepare); check: the whole-bucket "
                         "NaN/Inf/large scan of the rank's full local grad buffers (dopt_check_grads); checkpoint: the "
                         "model-space export and import of the rank's optimizer state (dopt_state_export / _import)")
    ap.add_argument("--placement", choices=["auto", "regions", "sets"], default="auto",
                    help="arena placement search: 'regions' backs each large buffer's arrays region by region "
                         "(2^27 elements) and keeps, per region, the fastest of the candidate backings for pass 2; "
                         "'sets' allocates whole candidate arena sets; auto: regions when a buffer spans at least "
                         "4 regions, else sets")
    # A one-time search of about 40-50 s for the 108 GB dense-7B state: against 2 sweeps, 1% and 8 candidates
    # (6-7 s) it took that workload's pass 2 from 30.82-30.84 to 30.66-30.67 ms, two runs each on one box.
    ap.add_argument("--region-sweeps", type=int, default=3, help="region search: passes over the regions")
    ap.add_argument("--region-tolerance", type=float, default=0.003,
                    help="region search: a region within this fraction of the fastest region rate seen is kept")
    ap.add_argument("--placement-tries", type=int, default=12,
                    help="candidate arena placements tried at start-up, the fastest for pass 2 kept (1: plain "
                         "allocation); capped by free device memory")
    ap.add_argument("--flush-llc", action="store_true",
                    help="step mode: read a 512 MiB buffer before each timed step, so that no step data is left in "
                         "the 256 MB last-level cache; each step is then timed on its own with HIP events and "
                         "ms_per_step is their mean")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="instead of the step: copy an fp32 buffer of this many MiB (a plain copy of known size, "
                         "used to scale the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the step; runs on more than one GPU are not supported.",
              file=sys.stderr)
        sys.exit(2)

    progress("importing torch")
    import torch
    progress(f"torch {torch.__version__}, device {torch.cuda.get_device_name(0) if torch.cuda.is_available() else None}")
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        dst.copy_(src)
        torch.cuda.synchronize()
        ev[0].record()
        reps = 5
        for _ in range(reps):
            dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        print(json.dumps({"calibration": "fp32 copy", "bytes_read": 4 * n, "bytes_written": 4 * n,
                          "ms": round(ms, 5), "GBps": round(8 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return
    import synth

    w = synth.WORKLOADS[args.workload]
    if args.mode != "step":
        run_other_mode(args, w)
        return
    res = measure_step(w, args.steps, args.warmup, args.placement_tries, args.flush_llc, args.placement,
                       (args.region_sweeps, args.region_tolerance))
    out = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "Gparams/s",
        "n_gpus": 1,
        "steps": res["steps"],
        "warmup": res["warmup"],
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded draws on the device)",
        "config": res["config"],
        "hbm_GBps_step": res["hbm_GBps_step"],
        "hbm_frac_step": res["hbm_frac_step"],
        "roofline": res["roofline"],
    }
    for key in ("skip_step", "llc_flushed"):
        if key in res:
            out[key] = res[key]
    if args.secondary and args.secondary != args.workload:
        # the GPT-2-small rank: a window whose 249 MB of step data nearly fits
        # the 256 MB last-level cache, so its back-to-back figure is
        # cache-assisted; its flushed figure is the HBM-bound one
        import torch
        torch.cuda.empty_cache()
        sw = synth.WORKLOADS[args.secondary]
        sec = measure_step(sw, None, None, args.placement_tries, False, args.placement)
        out["secondary"] = {k: sec[k] for k in ("value", "ms_per_step", "steps", "warmup", "hbm_GBps_step",
                                                 "hbm_frac_step", "roofline", "llc_flushed")}
        out["secondary"]["workload"] = sec["config"]["workload"]
        out["secondary"]["llc"] = "warm (steps back to back): the step's data nearly fits the 256 MB last-level " \
                                  "cache, so value and roofline are cache-assisted; llc_flushed is HBM-bound"
    if not args.no_cpu_baseline:
        progress("oracle CPU baseline")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def fill_device(t, sigma: float, seed: int, scale: float = 1.0, zero_frac: float = 0.0, chunk: int = 1 << 28):
    """Seeded synthetic values drawn on the device into t: storage(scale *
    N(0, sigma^2)) by PyTorch's device generator, with exact zeros at the
    given fraction (an independent uniform draw per element)."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(seed)
    for s in range(0, t.numel(), chunk):
        part = t[s:s + chunk]
        part.normal_(0.0, sigma * scale, generator=g)
        if zero_frac > 0.0:
            part.masked_fill_(torch.rand(part.numel(), device=t.device, generator=g) < zero_frac, 0.0)


def setup(w, placement_tries: int, placement: str = "auto", region=(2, 0.01)):
    """Layout, arenas (with the placement search) and seeded inputs of one
    workload, state initialised; returns (L, A, bufs_c, hp_c, sizes, alloc_seconds)."""
    import torch
    import sharded_mixed_precision_amd as D
    import synth
    from sharded_mixed_precision_amd.arena import DeviceArenas

    params = synth.PARAM_LISTS[w.model]()
    L = D.dopt_build_ranges(params, w.dp_size, w.dp_rank, w.bucket_size, w.pad_for_high_busbw)
    if placement == "auto":
        big = max(L.buffer(k)["arena_numel"] for k in range(L.num_buffers))
        placement = "regions" if big >= 4 * REGION_ELEMS else "sets"
    t_alloc = time.perf_counter()
    A = DeviceArenas(L, placement_tries=placement_tries, placement=placement, region_elems=REGION_ELEMS,
                     region_sweeps=region[0], region_tolerance=region[1])
    torch.cuda.synchronize()
    t_alloc = time.perf_counter() - t_alloc
    sizes = {"E": 0, "bytes_step": 0, "apply_bytes": 0, "n_params": len(params)}
    for k, info in enumerate(A.info):
        p1, p2 = pass_bytes(info["pd"], info["gd"])
        sizes["E"] += info["shard_numel"]
        sizes["bytes_step"] += (p1 + p2) * info["shard_numel"]
        sizes["apply_bytes"] += p2 * info["shard_numel"]
        fill_device(A.bufs[k]["param"], w.weight_sigma, 1_000_003 * w.seed + 2 * k)
        fill_device(A.bufs[k]["grad"], w.grad_sigma, 1_000_003 * w.seed + 2 * k + 1, w.initial_scale, w.zero_frac)
    stream = torch.cuda.current_stream()
    D.dopt_init_state(L, A.bufs, D.scaler_cfg(w.dynamic_scale, w.initial_scale), A.workspace, stream)
    bufs_c = D.tensors(L, A.bufs)
    hp_c = D.hparams_array([(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)])
    return L, A, bufs_c, hp_c, sizes, t_alloc


def placement_summary(A, seconds: float) -> dict:
    """The distribution of pass-2 times over the placements the search tried:
    whole arena sets, then each array's candidates with the others fixed."""
    p = A.placement
    if p is None:
        return {"candidates": 1, "seconds": round(seconds, 3)}
    if p.get("kind") == "regions":
        out = {"kind": "regions", "seconds": round(seconds, 3), "buffers": []}
        for b in p["buffers"]:
            reg = b["last_sweep"]
            out["buffers"].append({
                "buffer": b["buffer"], "regions": b["regions"], "region_elems": b["region_elems"],
                "sweeps": b["sweeps"], "region_ms_before_last_sweep": round(sum(r[1] for r in reg), 4),
                "region_ms_kept": round(sum(r[2] for r in reg), 4),
                "candidates_last_sweep": sum(r[3] for r in reg),
                "fastest_region_ms": min(r[2] for r in reg), "slowest_region_ms": max(r[2] for r in reg[:-1] or reg)})
        return out
    whole = p["pass2_ms"]
    out = {"whole_sets": {"n": len(whole), "kept_ms": whole[p["kept"]], "median_ms": round(statistics.median(whole), 4),
                          "worst_ms": max(whole), "all_ms": whole},
           "per_array": [], "seconds": round(seconds, 3)}
    for k, key, n, ms_list in p["refined"]:
        out["per_array"].append({"array": f"{k}.{key}", "n": len(ms_list), "kept_ms": min(ms_list),
                                 "median_ms": round(statistics.median(ms_list), 4), "worst_ms": max(ms_list)})
    out["kept_pass2_ms"] = min(p["refined"][-1][3]) if p["refined"] else whole[p["kept"]]
    return out


def pass2_kernels(A) -> str:
    """The pass-2 kernel of each buffer, as the library chose it (k_apply_bnd
    for a grid-stride window that holds boundary tiles)."""
    names = []
    for info in A.info:
        name = "k_apply_bnd" if info.get("apply_bnd") else "k_apply"
        if name not in names:
            names.append(name)
    return " + ".join(names)


def measure_step(w, steps, warmup, placement_tries: int, flush_llc: bool, placement: str = "auto",
                 region=(2, 0.01)) -> dict:
    """Time K back-to-back steps of one workload (or K steps each after an
    LLC flush), then pass 2 on its own, the flushed steps, and the skipped
    step for a dynamically scaled workload."""
    import torch
    import sharded_mixed_precision_amd as D

    L, A, bufs_c, hp_c, sz, t_alloc = setup(w, placement_tries, placement, region)
    stream = torch.cuda.current_stream()
    E, bytes_step, apply_bytes = sz["E"], sz["bytes_step"], sz["apply_bytes"]
    progress(f"{w.name}: arenas placed in {t_alloc:.1f}s, inputs drawn, state initialised")
    # A small window's step lasts tens of microseconds: hundreds of warm-up
    # steps let the clocks settle, and hundreds of timed steps keep the timed
    # region in the tens of milliseconds.  A large window's step lasts
    # milliseconds.
    small = E <= SMALL_WINDOW
    K = steps if steps is not None else (500 if small else 20)
    W = warmup if warmup is not None else (200 if small else 3)

    def step():
        D.dopt_step(L, bufs_c, hp_c, w.max_grad_norm, A.workspace, stream, want_stats=False)

    # dopt_step = dopt_step_prepare + dopt_step_apply; called as its two
    # halves so that events can bracket the apply pass (APPLY_BATCH launches).
    def step_bracketed(ev_a, ev_b):
        D.dopt_step_prepare(L, bufs_c, hp_c, w.max_grad_norm, A.workspace, stream)
        ev_a.record(stream)
        for _ in range(APPLY_BATCH):
            D.dopt_step_apply(L, bufs_c, A.workspace, stream)
        ev_b.record(stream)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    flush = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")  # 512 MiB
    torch.cuda.synchronize()

    def evict():
        """Read 512 MiB: the 256 MB last-level cache then holds none of the
        step's data, only clean lines (a write would leave dirty lines whose
        write-back the next step would pay for)."""
        flush.sum()

    def flushed_steps():
        """K steps, each timed on its own right after evict(); their ms."""
        ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        for i in range(K):
            evict()
            ev_s[i].record(stream)
            step()
            ev_e[i].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in zip(ev_s, ev_e)]

    per_step = None  # each step's ms where steps are timed one by one
    if flush_llc:
        per_step = flushed_steps()
        total_ms = sum(per_step)
    else:
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        for i in range(K):
            step()
        t_end.record(stream)
        torch.cuda.synchronize()
        total_ms = t_start.elapsed_time(t_end)
    # pass-2 launch duration: K more steps, events bracketing APPLY_BATCH applies
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for i in range(K):
        if flush_llc:
            evict()
        step_bracketed(ev_a[i], ev_b[i])
    torch.cuda.synchronize()
    apply_ms = sum(a.elapsed_time(b) for a, b in zip(ev_a, ev_b)) / (K * APPLY_BATCH)
    progress(f"{w.name}: {K} steps at {total_ms / K:.4f} ms, pass 2 at {apply_ms:.4f} ms")
    # the same steps with the last-level cache flushed before each (reported
    # beside the back-to-back figure; a training step runs after forward and
    # backward have passed far more than 256 MB through the cache)
    flushed = None if flush_llc else flushed_steps()
    flushed_ms = None if flushed is None else sum(flushed) / K
    st = D.dopt_read_stats(L, A.workspace, stream)
    assert st["skipped"] == 0 and st["step_count"] == W + (2 if flush_llc else 3) * K, st
    skip = skip_step(L, A, step, K, stream) if w.dynamic_scale else None
    ms = total_ms / K
    gbps = bytes_step / (ms * 1e-3) / 1e9
    ach = apply_bytes / (apply_ms * 1e-3) / 1e9
    tr = MEASURED_TRAFFIC.get(w.name)
    traffic = tr["bytes_per_launch"] if tr and tr.get("src") == _src_sha() else None
    res = {
        "value": round(E / (ms * 1e-3) / 1e9, 3), "steps": K, "warmup": W, "ms_per_step": round(ms, 5),
        "config": {"workload": f"{w.name}: {sz['n_params']}-param list, rank {w.dp_rank} of N={w.dp_size}, "
                               f"bucket {w.bucket_size}, {E} shard elements",
                   "shard_elements": E, "bytes_per_step": bytes_step,
                   "llc": "flushed before each step" if flush_llc else "warm (steps back to back)",
                   "arena_placement": placement_summary(A, t_alloc)},
        "hbm_GBps_step": round(gbps, 1),
        "hbm_frac_step": round(gbps / HBM_PEAK_GBPS, 4),
        **({"ms_per_step_median": round(statistics.median(per_step), 5), "ms_per_step_best": round(min(per_step), 5)}
           if per_step else {}),
        "roofline": {"bound": "hbm", "kernel": pass2_kernels(A) + " (pass 2)", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "launch_ms": round(apply_ms, 5), "launches_timed": K * APPLY_BATCH,
                     "algorithmic_bytes_per_launch": apply_bytes},
    }
    if skip is not None:
        res["skip_step"] = skip
    if flushed_ms is not None:
        res["llc_flushed"] = {"ms_per_step": round(flushed_ms, 5), "value": round(E / (flushed_ms * 1e-3) / 1e9, 3),
                              "unit": "Gparams/s", "hbm_GBps_step": round(bytes_step / (flushed_ms * 1e-3) / 1e9, 1),
                              "hbm_frac_step": round(bytes_step / (flushed_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                              "ms_per_step_median": round(statistics.median(flushed), 5),
                              "ms_per_step_best": round(min(flushed), 5)}
    del A, bufs_c, flush
    return res


def run_other_mode(args, w):
    import torch
    import sharded_mixed_precision_amd as D

    L, A, bufs_c, hp_c, sz, _ = setup(w, args.placement_tries, args.placement)
    stream = torch.cuda.current_stream()
    if args.steps is None:
        args.steps = 50 if sz["E"] <= SMALL_WINDOW else 10
    if args.warmup is None:
        args.warmup = 10 if sz["E"] <= SMALL_WINDOW else 2
    if args.mode == "reduce":
        bench_reduce(args, w, L, A, bufs_c, hp_c, stream)
    elif args.mode == "check":
        bench_check(args, w, L, A, stream)
    else:
        bench_checkpoint(args, w, L, A, bufs_c, stream)


if __name__ == "__main__":
    main()
