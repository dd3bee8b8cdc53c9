"""Parity harness: runs the HIP path (through the C ABI) and the oracle on the
same seeded inputs and compares them.

Tolerances (fixed for this method): integer results bit-exact; fp32 master,
m and v within max(1e-6 * |oracle|, 1e-9); grad norm within 1e-5 relative;
16-bit params within 1 ulp.

Inputs are keyed by (seed, stream, step, arena index): weights N(0, sigma_w)
narrowed to the param dtype; per-step grads N(0, sigma_g) (times the loss
scale the step's grads carry) narrowed to the grad dtype; optional exact
zeros; optionally one +inf at a seeded shard element.
"""
from __future__ import annotations

import ctypes
import math
import sys
import time
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

import oracle
import synth
from tests.oracle_harness import (NP_STORE, OracleRun, export_to_model, model_to_export, place_in_arenas,
                                  shard_pieces, to_bits, to_torch)

MASTER_RTOL, MASTER_ATOL = 1e-6, 1e-9
NORM_RTOL = 1e-5
PARAM_ULPS = 1


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class Case:
    name: str
    params: Sequence
    dp_size: int
    dp_rank: int
    bucket_size: int = 0
    busbw: int = 0
    steps: int = 3
    grad_sigma: float = 1e-2
    weight_sigma: float = 0.02
    zero_frac: float = 0.0
    dynamic: bool = False
    initial_scale: float = 1.0
    inf_step: Optional[int] = None
    inf_value: float = math.inf
    seed: int = 0
    hparams: List = field(default_factory=lambda: [(1e-3, 0.9, 0.999, 1e-8, 0.01)])
    max_norm: float = 1.0
    const_grad: Optional[float] = None  # all grads equal to this value
    instances: int = 1
    # grads produced by the fp32-accumulating local reduce of `chunks` received
    # chunks in the `wire` dtype (0: grads drawn directly)
    chunks: int = 0
    wire: str = "bf16"
    reduce_scale: float = 1.0
    reduce_split: bool = False
    # slots after each received chunk, filled with NaN and never read: chunk
    # j of an n-slot arena starts at j * (n + chunk_pad)
    chunk_pad: int = 0
    placement_tries: int = 1  # DeviceArenas placement search (1: plain allocation)
    placement: str = "sets"  # "regions": large buffers backed region by region (dopt_vmm.h)
    region_elems: int = 1 << 27

    def scale_at(self, step: int) -> float:
        if not self.dynamic:
            return self.initial_scale
        s = self.initial_scale
        if self.inf_step is not None and step > self.inf_step:
            s *= 0.5
        return s


def case_from_workload(w) -> Case:
    return Case(w.name, synth.PARAM_LISTS[w.model](), w.dp_size, w.dp_rank, w.bucket_size, w.pad_for_high_busbw,
                w.steps, w.grad_sigma, w.weight_sigma, w.zero_frac, w.dynamic_scale, w.initial_scale, w.inf_step,
                seed=w.seed, hparams=[(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)], max_norm=w.max_grad_norm)


# ---------------------------------------------------------------- inputs ----

def host_weights(case: Case, k: int, dt: str, n: int, out=None):
    return synth.fill_normal(dt, n, case.seed, synth.weight_stream(k), 0, case.weight_sigma,
                             out=out)


def host_grads(case: Case, k: int, dt: str, n: int, step: int, out=None):
    if case.const_grad is not None:
        t = out if out is not None else torch.empty(n, dtype=synth.torch_dtype(dt))
        t.fill_(case.const_grad)
        return t
    return synth.fill_normal(dt, n, case.seed, synth.grad_stream(k), step, case.grad_sigma,
                             scale=case.scale_at(step), zero_frac=case.zero_frac, out=out)


def host_chunks(case: Case, k: int, n: int, step: int, out=None):
    """case.chunks received chunks of an n-slot arena, back to back, in the wire dtype."""
    return synth.fill_normal(case.wire, case.chunks * n, case.seed, synth.chunk_stream(k), step, case.grad_sigma,
                             zero_frac=case.zero_frac, out=out)


def padded_chunks(case: Case, packed: torch.Tensor, n: int) -> torch.Tensor:
    """The chunks at a stride of n + case.chunk_pad, the gaps filled with NaN."""
    stride = n + case.chunk_pad
    out = torch.full((case.chunks * stride,), math.nan, dtype=packed.dtype)
    for j in range(case.chunks):
        out[j * stride:j * stride + n] = packed[j * n:(j + 1) * n]
    return out


def inf_position(case: Case, O: oracle.Layout):
    """(buffer, arena index) of the seeded overflow element: the j-th shard element in buffer/arena order."""
    total = sum(O.buffer(k)["shard_numel"] for k in range(O.num_buffers))
    j = synth.uniform_index(case.seed, synth.STREAM_INF_POS, case.inf_step, 0, total)
    for k in range(O.num_buffers):
        s, ln, _ = O.segments(k)
        if j < int(ln.sum()):
            c = np.cumsum(ln)
            q = int(np.searchsorted(c, j, side="right"))
            before = int(c[q - 1]) if q > 0 else 0
            return k, int(s[q]) + (j - before)
        j -= int(ln.sum())
    raise AssertionError("no shard element")


# ------------------------------------------------------------ comparisons ---

def ulp_dist(a_bits: np.ndarray, b_bits: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f32":
        a = a_bits.view(np.int32).astype(np.int64)
        b = b_bits.view(np.int32).astype(np.int64)
        sign = np.int64(1 << 31)
        mag = np.int64(0x7fffffff)
    else:
        a = a_bits.view(np.uint16).astype(np.int64)
        b = b_bits.view(np.uint16).astype(np.int64)
        sign = np.int64(0x8000)
        mag = np.int64(0x7fff)
    oa = np.where(a & sign, -(a & mag), a & mag)
    ob = np.where(b & sign, -(b & mag), b & mag)
    return np.abs(oa - ob)


def check_f32(name: str, dev: np.ndarray, ref: np.ndarray) -> dict:
    dev = dev.astype(np.float64)
    ref = ref.astype(np.float64)
    with np.errstate(invalid="ignore"):  # inf - inf where both overflowed
        err = np.abs(dev - ref)
    tol = np.maximum(MASTER_RTOL * np.abs(ref), MASTER_ATOL)
    bad = ~((err <= tol) | (dev == ref))  # equal infinities (an overflowed v) match
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} outside tolerance; idx {i} dev {dev[i]} ref {ref[i]}")
    rel = np.where(dev == ref, 0.0, err / np.maximum(np.abs(ref), 1e-30))
    return {"n": int(dev.size), "bit_exact": float(np.mean(dev == ref)) if dev.size else 1.0,
            "max_rel": float(np.max(rel)) if dev.size else 0.0}


def check_param(name: str, dev_bits: np.ndarray, ref_bits: np.ndarray, dt: str) -> dict:
    d = ulp_dist(dev_bits, ref_bits, dt)
    if d.size and d.max() > PARAM_ULPS:
        i = np.flatnonzero(d > PARAM_ULPS)[:5]
        raise AssertionError(f"{name}: {int((d > PARAM_ULPS).sum())} params beyond {PARAM_ULPS} ulp; idx {i}")
    return {"n": int(d.size), "bit_exact": float(np.mean(d == 0)) if d.size else 1.0, "max_ulp": int(d.max()) if d.size else 0}


def check_stats(dev: dict, ref: oracle.Stats, step: int):
    where = f"step {step}"
    assert dev["found_inf"] == ref.found_inf, where
    assert dev["skipped"] == ref.skipped, where
    assert dev["step_count"] == ref.t, where
    assert dev["num_zeros"] == ref.zeros, (where, dev["num_zeros"], ref.zeros)
    assert dev["loss_scale_used"] == ref.scale_used and dev["loss_scale_next"] == ref.scale_next, where
    if math.isfinite(ref.sumsq):
        assert math.isclose(dev["grad_norm"], ref.norm, rel_tol=NORM_RTOL, abs_tol=0.0) or \
            (ref.norm == 0.0 and dev["grad_norm"] == 0.0), (where, dev["grad_norm"], ref.norm)
        assert dev["clip_applied"] == ref.clip_applied, where
        if ref.clip_applied:
            assert math.isclose(dev["clip_coef"], ref.clip_coef, rel_tol=NORM_RTOL), where
    else:
        assert not math.isfinite(dev["sumsq"]), where


# ---------------------------------------------------------------- device ----

def _dopt():
    import sharded_mixed_precision_amd as D
    return D


class DeviceRun:
    def __init__(self, case: Case):
        D = _dopt()
        from sharded_mixed_precision_amd.arena import DeviceArenas
        self.D = D
        self.L = D.dopt_build_ranges(case.params, case.dp_size, case.dp_rank, case.bucket_size, case.busbw,
                                     case.instances)
        self.A = DeviceArenas(self.L, placement_tries=case.placement_tries, placement=case.placement,
                              region_elems=case.region_elems)
        self.stream = torch.cuda.current_stream()
        self.case = case

    def init(self, host_params: List[torch.Tensor]):
        for k, t in enumerate(host_params):
            self.A.bufs[k]["param"].copy_(t)
        c = self.case
        sc = self.D.scaler_cfg(c.dynamic, c.initial_scale)
        self.D.dopt_init_state(self.L, self.A.bufs, sc, self.A.workspace, self.stream)

    def step(self, host_grads: List[torch.Tensor], split: bool = False, halves: bool = False) -> dict:
        for k, t in enumerate(host_grads):
            self.A.bufs[k]["grad"].copy_(t)
        c = self.case
        if halves:
            self.D.dopt_step_prepare(self.L, self.A.bufs, c.hparams, c.max_norm, self.A.workspace, self.stream)
            self.D.dopt_step_apply(self.L, self.A.bufs, self.A.workspace, self.stream)
            return self.D.dopt_read_stats(self.L, self.A.workspace, self.stream)
        if split:
            self.D.dopt_step_stats(self.L, self.A.bufs, self.A.workspace, self.stream)
            self.D.dopt_step_finalize(self.L, c.hparams, c.max_norm, self.A.workspace, self.stream)
            self.D.dopt_step_apply(self.L, self.A.bufs, self.A.workspace, self.stream)
            return self.D.dopt_read_stats(self.L, self.A.workspace, self.stream)
        return self.D.dopt_step(self.L, self.A.bufs, c.hparams, c.max_norm, self.A.workspace, self.stream)

    def step_reduce(self, host_chunks: List[torch.Tensor]) -> dict:
        """The step with its grads formed on the device by dopt_reduce_prepare."""
        c = self.case
        if not hasattr(self, "dev_chunks"):
            self.dev_chunks = [torch.empty(t.numel(), dtype=t.dtype, device="cuda") for t in host_chunks]
        for d, t in zip(self.dev_chunks, host_chunks):
            d.copy_(t)
        strides = [inf["arena_numel"] + c.chunk_pad for inf in self.L.infos()] if c.chunk_pad else None
        if c.reduce_split:
            self.D.dopt_reduce_prepare(self.L, self.A.bufs, self.dev_chunks, c.wire, c.chunks, c.reduce_scale, None,
                                       c.max_norm, self.A.workspace, self.stream, chunk_strides=strides)
            self.D.dopt_step_finalize(self.L, c.hparams, c.max_norm, self.A.workspace, self.stream)
        else:
            self.D.dopt_reduce_prepare(self.L, self.A.bufs, self.dev_chunks, c.wire, c.chunks, c.reduce_scale,
                                       c.hparams, c.max_norm, self.A.workspace, self.stream, chunk_strides=strides)
        self.D.dopt_step_apply(self.L, self.A.bufs, self.A.workspace, self.stream)
        return self.D.dopt_read_stats(self.L, self.A.workspace, self.stream)

    def host(self, k: int, key: str) -> np.ndarray:
        t = self.A.bufs[k][key]
        return to_bits(t.cpu())

    def gather(self, k: int, key: str, idx_dev: torch.Tensor) -> np.ndarray:
        t = self.A.bufs[k][key]
        return to_bits(t.index_select(0, idx_dev).cpu())


# ------------------------------------------------------------ full parity ---

def run_full(case: Case, split_steps: Sequence[int] = (), half_steps: Sequence[int] = ()) -> List[dict]:
    """Every element compared after every step."""
    t0 = time.time()
    dev = DeviceRun(case)
    arena = [dev.L.buffer(k)["arena_numel"] for k in range(dev.L.num_buffers)]
    orc = OracleRun(case.params, case.dp_size, case.dp_rank, case.bucket_size, case.busbw, arena_numel=arena,
                    instances=case.instances)
    for k in range(orc.nb):
        w = orc.L.buffer(k)["window_numel"]
        assert arena[k] == -(-max(w, 1) // dev.D.DOPT_ARENA_ALIGN) * dev.D.DOPT_ARENA_ALIGN
    orc.scaler = oracle.make_scaler(case.dynamic, case.initial_scale)
    hp = [orc.bufs[k] for k in range(orc.nb)]
    params0 = []
    for k, b in enumerate(hp):
        t = host_weights(case, k, b["pd"], b["n"])
        b["param"][:] = to_bits(t)
        params0.append(t)
    dev.init(params0)
    orc.init_state()
    masks = [orc.valid(k) for k in range(orc.nb)]
    init_bits = [to_bits(p).copy() for p in params0]
    pos = inf_position(case, orc.L) if case.inf_step else None
    report = []
    for s in range(1, case.steps + 1):
        grads, chunks = [], []
        for k, b in enumerate(hp):
            if case.chunks:
                ch = host_chunks(case, k, b["n"], s)
                if case.chunk_pad:
                    ch = padded_chunks(case, ch, b["n"])
                chunks.append(ch)
                oracle.lib().or_reduce_chunks(orc.L.handle, k, ch.data_ptr(), oracle.DTYPES[case.wire], case.chunks,
                                              b["n"] + case.chunk_pad, case.reduce_scale, 0, b["n"],
                                              b["grad"].ctypes.data)
                continue
            g = host_grads(case, k, b["gd"], b["n"], s)
            if pos is not None and s == case.inf_step and pos[0] == k:
                g[pos[1]] = case.inf_value
            b["grad"][:] = to_bits(g)
            grads.append(g)
        ref = orc.step(case.hparams, case.max_norm)
        if case.chunks:
            got = dev.step_reduce(chunks)
        else:
            got = dev.step(grads, split=s in split_steps, halves=s in half_steps)
        check_stats(got, ref, s)
        rep = {"step": s, "norm_dev": got["grad_norm"], "norm_ref": ref.norm}
        if case.chunks:  # the reduced grad window, every slot, bit for bit
            for k, b in enumerate(hp):
                w = orc.L.buffer(k)["window_numel"]
                gdev = dev.host(k, "grad")[:w]
                assert np.array_equal(gdev.view(np.uint8), b["grad"][:w].view(np.uint8)), f"step {s}: reduced grad[{k}]"
        for k, b in enumerate(hp):
            m = masks[k]
            if b["pd"] != "f32":
                rep[f"master{k}"] = check_f32(f"{case.name} step {s} master[{k}]", dev.host(k, "master")[m],
                                              b["master"][m])
            rep[f"m{k}"] = check_f32(f"{case.name} step {s} m[{k}]", dev.host(k, "exp_avg")[m], b["m"][m])
            rep[f"v{k}"] = check_f32(f"{case.name} step {s} v[{k}]", dev.host(k, "exp_avg_sq")[m], b["v"][m])
            pdev = dev.host(k, "param")
            rep[f"param{k}"] = check_param(f"{case.name} step {s} param[{k}]", pdev[m], b["param"][m], b["pd"])
            # slots that hold no param element are never written
            assert np.array_equal(pdev[~m], init_bits[k][~m]), f"step {s}: param arena gap written"
        report.append(rep)
        log(f"[parity] {case.name} step {s}: every element compared ({time.time() - t0:.1f}s)")
    log(f"[parity] {case.name}: {case.steps} steps full compare ok in {time.time() - t0:.1f}s; last {report[-1]}")
    return report


# ------------------------------------------------- full parity, chunked ---

def _valid_ranges(O: oracle.Layout, k: int):
    s, ln, _ = O.segments(k)
    return list(zip(s.tolist(), (s + ln).tolist()))


def _gaps(ranges, n):
    """Arena slots [lo, hi) between and after the shard segments."""
    out, cur = [], 0
    for a, b in ranges:
        if a > cur:
            out.append((cur, a))
        cur = max(cur, b)
    if cur < n:
        out.append((cur, n))
    return out


def run_full_chunked(case: Case, workers: int = 16, chunk: int = 1 << 26) -> List[dict]:
    """Every shard element compared after every step at full size, with the
    oracle split into disjoint arena ranges run on host threads: the
    statistics by or_grad_stats_range (partials added in range order), the
    update by or_apply_range (each element's update depends on its own values
    only), both pinned on the CPU to equal the whole-window calls.  The device
    arrays are copied back range by range and compared with the oracle's."""
    t0 = time.time()
    lib = oracle.lib()
    dev = DeviceRun(case)
    O = oracle.Layout(case.params, case.dp_size, case.dp_rank, case.bucket_size, case.busbw, case.instances)
    nb = O.num_buffers
    infos = []
    for k in range(nb):
        b = O.buffer(k)
        pd, gd = {0: "f32", 1: "bf16", 2: "f16"}[b["param_dtype"]], {0: "f32", 1: "bf16", 2: "f16"}[b["grad_dtype"]]
        n = dev.L.buffer(k)["arena_numel"]
        assert n == -(-max(b["window_numel"], 1) // 2048) * 2048
        infos.append((pd, gd, n))
    ranges = [_valid_ranges(O, k) for k in range(nb)]
    host, params0, gap_bits = [], [], []
    for k, (pd, gd, n) in enumerate(infos):
        p = host_weights(case, k, pd, n)
        params0.append(p)
        pbits = to_bits(p)
        gap_bits.append([(lo, hi, pbits[lo:hi].copy()) for lo, hi in _gaps(ranges[k], n)])
        master = np.zeros(n, np.float32) if pd != "f32" else None
        host.append({"param": pbits, "master": master, "m": np.zeros(n, np.float32), "v": np.zeros(n, np.float32),
                     "grad": torch.empty(n, dtype=synth.torch_dtype(gd), pin_memory=torch.cuda.is_available())})
    dev.init(params0)
    jobs = [(k, lo, min(lo + chunk, infos[k][2])) for k in range(nb) for lo in range(0, infos[k][2], chunk)]

    def init_master(job):
        k, lo, hi = job
        pd = infos[k][0]
        h = host[k]
        if pd == "bf16":
            lib.or_bf16_to_f32_n(h["param"][lo:].ctypes.data, h["master"][lo:].ctypes.data, hi - lo)
        elif pd == "f16":
            lib.or_f16_to_f32_n(h["param"][lo:].ctypes.data, h["master"][lo:].ctypes.data, hi - lo)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(init_master, jobs))
    arrays = (oracle.Arrays * nb)()
    for k, h in enumerate(host):
        arrays[k] = oracle.arrays(h["grad"], h["param"], h["master"], h["m"], h["v"])
    log(f"[fullsize] {case.name}: init done {time.time() - t0:.1f}s, arenas {[i[2] for i in infos]}")
    scaler = oracle.make_scaler(case.dynamic, case.initial_scale)
    t = ctypes.c_int64(0)
    hpa = oracle.make_hparams(case.hparams)
    pos = inf_position(case, O) if case.inf_step else None
    keys = [("master", "master"), ("exp_avg", "m"), ("exp_avg_sq", "v"), ("param", "param")]
    report = []
    for s in range(1, case.steps + 1):
        ts = time.time()
        for k, (pd, gd, n) in enumerate(infos):
            host_grads(case, k, gd, n, s, out=host[k]["grad"])
            if pos is not None and s == case.inf_step and pos[0] == k:
                host[k]["grad"][pos[1]] = case.inf_value
        tg = time.time()
        st = oracle_stats_parallel(O, [h["grad"] for h in host], float(np.float32(1.0 / scaler.scale)), workers)
        sc = oracle.Scalars()
        assert lib.or_decide(ctypes.byref(st), ctypes.byref(scaler), ctypes.byref(t), hpa, len(case.hparams),
                             case.max_norm, ctypes.byref(sc)) == 0

        def apply(job):
            k, lo, hi = job
            lib.or_apply_range(O.handle, k, arrays, ctypes.byref(sc), lo, hi)

        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(apply, jobs))
        to = time.time()
        got = dev.step([h["grad"] for h in host])
        check_stats(got, st, s)

        def compare(job):
            """(elements compared, bit-identical, max param ulp) of one range;
            raises on a value outside the tolerance."""
            k, lo, hi = job
            pd = infos[k][0]
            out = []
            for dkey, hkey in keys:
                if hkey == "master" and pd == "f32":
                    continue
                d = to_bits(dev.A.bufs[k][dkey][lo:hi].cpu())
                r = host[k][hkey][lo:hi]
                valid = [(max(a, lo) - lo, min(b, hi) - lo) for a, b in ranges[k] if a < hi and b > lo]
                cnt = sum(b - a for a, b in valid)
                if np.array_equal(d.view(np.uint8), r.view(np.uint8)):
                    out.append((hkey, cnt, cnt, 0))
                    continue
                m = np.zeros(hi - lo, bool)
                for a, b in valid:
                    m[a:b] = True
                same = int(np.count_nonzero((d.view(np.uint8).reshape(hi - lo, -1) ==
                                             r.view(np.uint8).reshape(hi - lo, -1)).all(axis=1) & m))
                if hkey == "param" and pd != "f32":
                    res = check_param(f"{case.name} s{s} {hkey}[{k}] [{lo},{hi})", d[m], r[m], pd)
                    out.append((hkey, cnt, same, res["max_ulp"]))
                else:
                    check_f32(f"{case.name} s{s} {hkey}[{k}] [{lo},{hi})", d[m], r[m])
                    out.append((hkey, cnt, same, 0))
            return out

        with ThreadPoolExecutor(max_workers=8) as ex:
            parts = [x for part in ex.map(compare, jobs) for x in part]
        rep = {"step": s, "norm_dev": got["grad_norm"], "norm_ref": st.norm, "skipped": got["skipped"]}
        for hkey in ("master", "m", "v", "param"):
            sel = [p for p in parts if p[0] == hkey]
            if sel:
                n_el, n_same = sum(p[1] for p in sel), sum(p[2] for p in sel)
                rep[hkey] = {"n": n_el, "bit_exact": n_same / max(n_el, 1), "max_ulp": max(p[3] for p in sel)}
        for k, gaps in enumerate(gap_bits):  # slots that hold no param element are never written
            pdev = dev.A.bufs[k]["param"]
            for lo, hi, bits in gaps:
                assert np.array_equal(to_bits(pdev[lo:hi].cpu()).view(np.uint8), bits.view(np.uint8)), \
                    f"step {s}: param arena gap [{lo},{hi}) of buffer {k} written"
        report.append(rep)
        log(f"[fullsize] {case.name} step {s}: gen {tg - ts:.1f}s oracle {to - tg:.1f}s device+compare "
            f"{time.time() - to:.1f}s; {rep}")
    log(f"[fullsize] {case.name}: every element compared after each of {case.steps} steps in {time.time() - t0:.1f}s")
    return report


# --------------------------------------------------------- sampled parity ---

def _pick_samples(O: oracle.Layout, k: int, n_rand: int, seed: int) -> np.ndarray:
    s, ln, _ = O.segments(k)
    if len(s) == 0:
        return np.zeros(0, np.int64)
    c = np.cumsum(ln)
    total = int(c[-1])
    rng = np.random.default_rng(seed + 17 * k)
    j = rng.integers(0, total, size=min(n_rand, total))
    q = np.searchsorted(c, j, side="right")
    before = np.where(q > 0, c[np.maximum(q - 1, 0)], 0)
    idx = s[q] + (j - before)
    # every shard element of every boundary tile: the 2048-slot tiles that
    # hold a segment's first or last element or a bucket window's first or
    # last slot (the tiles the kernels take element by element)
    ends = np.concatenate([s, s + ln - 1])
    nbk = O.buffer(k)["n_buckets"]
    wins = []
    for b in range(nbk):
        bk = O.bucket(k, b)
        if bk["shard"] > 0:
            wins += [bk["arena_offset"], bk["arena_offset"] + bk["shard"] - 1]
    # and the tiles on both sides of every multiple of 2^26 slots, where a
    # pass launched over ranges of the arena (the fused reduce's ranges are
    # multiples of it) starts a new range
    cuts = np.arange(1 << 26, int(O.buffer(k)["window_numel"]), 1 << 26, dtype=np.int64)
    tiles = np.unique(np.concatenate([ends, np.array(wins, np.int64), cuts - 1, cuts]) // 2048)
    tb = []
    for tl in tiles.tolist():
        lo, hi = tl * 2048, tl * 2048 + 2048
        first = max(int(np.searchsorted(s + ln, lo, side="right")), 0)
        for q in range(first, len(s)):
            a, b = int(s[q]), int(s[q] + ln[q])
            if a >= hi:
                break
            tb.append(np.arange(max(a, lo), min(b, hi), dtype=np.int64))
    tb = np.concatenate(tb) if tb else np.zeros(0, np.int64)
    return np.unique(np.concatenate([idx, ends, tb]).astype(np.int64))


def oracle_stats_parallel(O: oracle.Layout, grads: List[torch.Tensor], inv_scale: float, workers: int = 16,
                          chunk: int = 1 << 26) -> oracle.Stats:
    """The oracle's S2 over all shard elements, split into disjoint arena
    ranges run on host threads (each range is one plain single-threaded oracle
    call); partials are added in range order."""
    lib = oracle.lib()
    jobs = []
    for k, g in enumerate(grads):
        n = g.numel()
        for lo in range(0, n, chunk):
            jobs.append((k, lo, min(lo + chunk, n)))

    def run(job):
        k, lo, hi = job
        st = oracle.Stats()
        lib.or_grad_stats_range(O.handle, k, grads[k].data_ptr(), inv_scale, lo, hi, ctypes.byref(st))
        return st.sumsq, st.zeros, st.found_inf

    with ThreadPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(run, jobs))
    out = oracle.Stats()
    out.sumsq = 0.0
    for sq, z, fi in parts:
        out.sumsq += sq
        out.zeros += z
        out.found_inf |= fi
    return out


def oracle_reduce_parallel(O: oracle.Layout, k: int, chunks: torch.Tensor, wire: str, n_chunks: int, stride: int,
                           scale: float, grad_out: torch.Tensor, workers: int = 16, chunk: int = 1 << 24):
    """The oracle's local fp32 reduce over disjoint slot ranges on host threads
    (each range one plain single-threaded oracle call; every slot is computed
    exactly once, so the result does not depend on the split)."""
    lib = oracle.lib()
    n = grad_out.numel()

    def run(lo):
        lib.or_reduce_chunks(O.handle, k, chunks.data_ptr(), oracle.DTYPES[wire], n_chunks, stride, scale, lo,
                             min(lo + chunk, n), grad_out.data_ptr())

    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(run, range(0, n, chunk)))


def oracle_check_parallel(O: oracle.Layout, k: int, grad: torch.Tensor, thr: float, workers: int = 16,
                          chunk: int = 1 << 24) -> List[dict]:
    """The oracle's whole-bucket check of buffer k; each bucket split into
    disjoint element ranges run on host threads and combined in range order."""
    lib = oracle.lib()
    nb = O.buffer(k)["n_buckets"]
    jobs = []
    for b in range(nb):
        bk = O.bucket(k, b)
        for lo in range(bk["offset"], bk["offset"] + bk["numel"], chunk):
            jobs.append((b, lo, min(lo + chunk, bk["offset"] + bk["numel"])))

    def run(job):
        b, lo, hi = job
        s, m, f = ctypes.c_double(), ctypes.c_float(), (ctypes.c_int32 * 3)()
        lib.or_check_bucket(O.handle, k, b, grad.data_ptr(), lo, hi, thr, ctypes.byref(s), ctypes.byref(m), f)
        return b, s.value, m.value, tuple(f)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(run, jobs))
    out = [{"sumsq": 0.0, "max_abs": 0.0, "has_nan": 0, "has_inf": 0, "large": 0} for _ in range(nb)]
    for b, s, m, f in parts:
        o = out[b]
        o["sumsq"] += s
        o["max_abs"] = max(o["max_abs"], m)
        o["has_nan"] |= f[0]
        o["has_inf"] |= f[1]
        o["large"] |= f[2]
    return out


def check_bucket_results(dev: List[dict], ref: List[dict], where: str):
    assert len(dev) == len(ref), where
    for b, (x, y) in enumerate(zip(dev, ref)):
        for key in ("has_nan", "has_inf", "large"):
            assert x[key] == y[key], (where, b, key, x, y)
        assert np.float32(x["max_abs"]) == np.float32(y["max_abs"]), (where, b, x, y)
        if math.isfinite(y["sumsq"]):
            assert math.isclose(x["sumsq"], y["sumsq"], rel_tol=1e-10, abs_tol=0.0), (where, b, x, y)
        else:
            assert math.isnan(x["sumsq"]) == math.isnan(y["sumsq"]) and not math.isfinite(x["sumsq"]), (where, b)


def run_check(case: Case, thr: float, injections=()) -> List[List[dict]]:
    """Whole local grad buffers through dopt_check_grads and the oracle.
    injections: (buffer, element index, value) written into the buffer first."""
    D = _dopt()
    from sharded_mixed_precision_amd.arena import DeviceArenas
    t0 = time.time()
    L = D.dopt_build_ranges(case.params, case.dp_size, case.dp_rank, case.bucket_size, case.busbw, case.instances)
    O = oracle.Layout(case.params, case.dp_size, case.dp_rank, case.bucket_size, case.busbw, case.instances)
    A = DeviceArenas(L)
    stream = torch.cuda.current_stream()
    D.dopt_init_state(L, A.bufs, D.scaler_cfg(), A.workspace, stream)
    results = []
    for k in range(L.num_buffers):
        info = L.buffer(k)
        gd = {0: "f32", 1: "bf16", 2: "f16"}[info["grad_dtype"]]
        n = info["numel"]
        host = synth.fill_normal(gd, n, case.seed, synth.local_grad_stream(k), 1, case.grad_sigma,
                                 zero_frac=case.zero_frac, out=torch.empty(n, dtype=synth.torch_dtype(gd),
                                                                           pin_memory=True))
        for kk, i, val in injections:
            if kk == k:
                host[i] = val
        dev = torch.empty(n, dtype=host.dtype, device="cuda")
        dev.copy_(host)
        nb = info["n_buckets"]
        out = torch.zeros(nb * D.BUCKET_CHECK_BYTES, dtype=torch.uint8, device="cuda")
        D.dopt_check_grads(L, k, dev, thr, out, A.workspace, stream)
        got = D.bucket_checks(out.cpu().numpy().tobytes(), nb)
        ref = oracle_check_parallel(O, k, host, thr)
        check_bucket_results(got, ref, f"{case.name} buffer {k}")
        results.append(got)
        del dev
    log(f"[check] {case.name}: {sum(len(r) for r in results)} buckets ok in {time.time() - t0:.1f}s")
    return results


def run_sampled(case: Case, n_samples: int = 1 << 20) -> List[dict]:
    """Full-size run on the device; the oracle computes the exact per-step
    stats over all shard elements and the trajectories of sampled elements."""
    t0 = time.time()
    lib = oracle.lib()
    dev = DeviceRun(case)
    O = oracle.Layout(case.params, case.dp_size, case.dp_rank, case.bucket_size, case.busbw, case.instances)
    nb = O.num_buffers
    infos = []
    for k in range(nb):
        b = O.buffer(k)
        pd, gd = {0: "f32", 1: "bf16", 2: "f16"}[b["param_dtype"]], {0: "f32", 1: "bf16", 2: "f16"}[b["grad_dtype"]]
        n = dev.L.buffer(k)["arena_numel"]
        assert n == -(-max(b["window_numel"], 1) // 2048) * 2048
        infos.append((pd, gd, n))
    samples, hgs, dev_idx = [], [], []
    st_master, st_m, st_v, st_param = [], [], [], []
    params0 = []
    for k, (pd, gd, n) in enumerate(infos):
        p = host_weights(case, k, pd, n)
        params0.append(p)
        idx = _pick_samples(O, k, n_samples, case.seed)
        samples.append(idx)
        hgs.append(O.hgroup_at(k, idx).astype(np.int32))
        dev_idx.append(torch.from_numpy(idx).cuda())
        pbits = to_bits(p)[idx].copy()
        mas = np.zeros(idx.size, np.float32)
        if pd == "bf16":
            lib.or_bf16_to_f32_n(pbits.ctypes.data, mas.ctypes.data, idx.size)
        elif pd == "f16":
            lib.or_f16_to_f32_n(pbits.ctypes.data, mas.ctypes.data, idx.size)
        else:
            mas[:] = pbits.view(np.float32)
        st_master.append(mas)
        st_m.append(np.zeros(idx.size, np.float32))
        st_v.append(np.zeros(idx.size, np.float32))
        st_param.append(pbits.copy())
    dev.init(params0)
    del params0
    log(f"[parity] {case.name}: init done {time.time() - t0:.1f}s, samples {[s.size for s in samples]}")
    scaler = oracle.make_scaler(case.dynamic, case.initial_scale)
    t = ctypes.c_int64(0)
    hpa = oracle.make_hparams(case.hparams)
    pos = inf_position(case, O) if case.inf_step else None
    grads = [torch.empty(n, dtype=synth.torch_dtype(gd), pin_memory=True) for (pd, gd, n) in infos]
    chunks = [torch.empty(case.chunks * n, dtype=synth.torch_dtype(case.wire), pin_memory=True)
              for (pd, gd, n) in infos] if case.chunks else None
    report = []
    for s in range(1, case.steps + 1):
        ts = time.time()
        for k, (pd, gd, n) in enumerate(infos):
            if case.chunks:
                host_chunks(case, k, n, s, out=chunks[k])
                oracle_reduce_parallel(O, k, chunks[k], case.wire, case.chunks, n, case.reduce_scale, grads[k])
                continue
            host_grads(case, k, gd, n, s, out=grads[k])
            if pos is not None and s == case.inf_step and pos[0] == k:
                grads[k][pos[1]] = case.inf_value
        tg = time.time()
        st = oracle_stats_parallel(O, grads, float(np.float32(1.0 / scaler.scale)))
        sc = oracle.Scalars()
        assert lib.or_decide(ctypes.byref(st), ctypes.byref(scaler), ctypes.byref(t), hpa, len(case.hparams),
                             case.max_norm, ctypes.byref(sc)) == 0
        for k, (pd, gd, n) in enumerate(infos):
            gs = np.ascontiguousarray(to_bits(grads[k])[samples[k]])
            lib.or_apply_elems(oracle.DTYPES[pd], oracle.DTYPES[gd], samples[k].size, hgs[k].ctypes.data,
                               gs.ctypes.data, st_master[k].ctypes.data, st_m[k].ctypes.data, st_v[k].ctypes.data,
                               st_param[k].ctypes.data, ctypes.byref(sc))
        to = time.time()
        got = dev.step_reduce(chunks) if case.chunks else dev.step(grads)
        if case.chunks:  # sampled slots of the reduced grad window, bit for bit
            for k in range(nb):
                gd_dev = dev.gather(k, "grad", dev_idx[k])
                assert np.array_equal(gd_dev.view(np.uint8), to_bits(grads[k])[samples[k]].view(np.uint8)), \
                    f"step {s}: reduced grad[{k}] samples"
        check_stats(got, st, s)
        rep = {"step": s, "norm_dev": got["grad_norm"], "norm_ref": st.norm, "skipped": got["skipped"]}
        for k, (pd, gd, n) in enumerate(infos):
            if pd != "f32":
                rep[f"master{k}"] = check_f32(f"{case.name} s{s} master[{k}]", dev.gather(k, "master", dev_idx[k]),
                                              st_master[k])
            rep[f"m{k}"] = check_f32(f"{case.name} s{s} m[{k}]", dev.gather(k, "exp_avg", dev_idx[k]), st_m[k])
            rep[f"v{k}"] = check_f32(f"{case.name} s{s} v[{k}]", dev.gather(k, "exp_avg_sq", dev_idx[k]), st_v[k])
            pdev = dev.gather(k, "param", dev_idx[k])
            if pd == "f32":
                rep[f"param{k}"] = check_f32(f"{case.name} s{s} param[{k}]", pdev, st_master[k])
            else:
                rep[f"param{k}"] = check_param(f"{case.name} s{s} param[{k}]", pdev, st_param[k], pd)
        report.append(rep)
        log(f"[parity] {case.name} step {s}: gen {tg - ts:.1f}s oracle {to - tg:.1f}s device+check "
            f"{time.time() - to:.1f}s; {rep}")
    log(f"[parity] {case.name}: sampled compare ok in {time.time() - t0:.1f}s")
    return report


# --------------------------------------------------- multi-rank and reshard ---

class DeviceRanks:
    """All N ranks of a data-parallel job on the one device, each with its own
    layout, arenas and workspace, joined through the library's cross-rank seam:
    dopt_step_stats on every rank, the grad-stats records summed over ranks in
    rank order (the all-reduce a real job makes), dopt_step_finalize and
    dopt_step_apply on every rank."""

    def __init__(self, params, dp_size, bucket_size=0, scaler=(False, 1.0)):
        D = _dopt()
        from sharded_mixed_precision_amd.arena import DeviceArenas
        self.D, self.params = D, list(params)
        self.layouts = [D.dopt_build_ranges(self.params, dp_size, r, bucket_size) for r in range(dp_size)]
        self.arenas = [DeviceArenas(L) for L in self.layouts]
        self.stream = torch.cuda.current_stream()
        self.scaler = scaler
        self.rec_off = self.layouts[0].stats_record_offset

    def _host_arenas(self, A, key, dtkey):
        return [np.zeros(info["n"], NP_STORE[info[dtkey]]) for info in A.info]

    def init(self, weights):
        for L, A in zip(self.layouts, self.arenas):
            host = self._host_arenas(A, "param", "pd")
            place_in_arenas(L, len(self.params), [to_bits(w) for w in weights], host)
            for k, h in enumerate(host):
                A.bufs[k]["param"].copy_(to_torch(h, A.info[k]["pd"]))
            self.D.dopt_init_state(L, A.bufs, self.D.scaler_cfg(*self.scaler), A.workspace, self.stream)

    def _record(self, A):
        return A.workspace[self.rec_off:self.rec_off + 16].view(torch.float64)

    def step(self, grads, hparams, max_norm) -> dict:
        D = self.D
        gbits = [to_bits(g) for g in grads]
        for L, A in zip(self.layouts, self.arenas):
            host = self._host_arenas(A, "grad", "gd")
            place_in_arenas(L, len(self.params), gbits, host)
            for k, h in enumerate(host):
                A.bufs[k]["grad"].copy_(to_torch(h, A.info[k]["gd"]))
            D.dopt_step_stats(L, A.bufs, A.workspace, self.stream)
        sumsq, zeros = 0.0, 0.0
        for A in self.arenas:  # rank order
            r = self._record(A).cpu().tolist()
            sumsq += r[0]
            zeros += r[1]
        total = torch.tensor([sumsq, zeros], dtype=torch.float64)
        for L, A in zip(self.layouts, self.arenas):
            self._record(A).copy_(total)
            D.dopt_step_finalize(L, hparams, max_norm, A.workspace, self.stream)
            D.dopt_step_apply(L, A.bufs, A.workspace, self.stream)
        stats = [D.dopt_read_stats(L, A.workspace, self.stream) for L, A in zip(self.layouts, self.arenas)]
        for s in stats[1:]:
            assert s == stats[0], "ranks disagree on the step's scalars"
        return stats[0]

    def model_state(self):
        full = {key: [np.full(p.numel, np.nan, np.float32) for p in self.params] for key in ("master", "m", "v")}
        for L, A in zip(self.layouts, self.arenas):
            n = L.state_numel
            ex = [torch.empty(max(n, 1), dtype=torch.float32, device="cuda") for _ in range(3)]
            self.D.dopt_state_export(L, A.bufs, *ex, A.workspace, self.stream)
            export_to_model(L, len(self.params), tuple(e[:n].cpu().numpy() for e in ex), full)
        return full

    def model_params(self):
        full = [np.zeros(p.numel, NP_STORE[p.param_dtype]) for p in self.params]
        for L, A in zip(self.layouts, self.arenas):
            host = [to_bits(b["param"].cpu()) for b in A.bufs]
            for p, k, a, lo, hi, _ in shard_pieces(L, len(self.params)):
                full[p][lo:hi] = host[k][a:a + hi - lo]
        return full

    def scalars(self):
        s = self.D.dopt_state_scalars_get(self.layouts[0], self.arenas[0].workspace, self.stream)
        return {"t": s["step_count"], "scale": s["loss_scale"], "growth_tracker": s["growth_tracker"],
                "hysteresis_tracker": s["hysteresis_tracker"]}

    def load(self, full, scalars):
        sc = {"step_count": scalars["t"], "loss_scale": scalars["scale"],
              "growth_tracker": scalars["growth_tracker"], "hysteresis_tracker": scalars["hysteresis_tracker"]}
        for L, A in zip(self.layouts, self.arenas):
            ex = [torch.from_numpy(e).to("cuda") if e.size else torch.zeros(1, device="cuda")
                  for e in model_to_export(L, len(self.params), full)]
            self.D.dopt_state_import(L, A.bufs, *ex, A.workspace, self.stream)
            self.D.dopt_state_scalars_set(L, A.workspace, sc, self.stream)
        torch.cuda.synchronize()


def check_model_state(name, dev, ref):
    out = {}
    for key in ("master", "m", "v"):
        out[key] = check_f32(f"{name} {key}", np.concatenate(dev[key]), np.concatenate(ref[key]))
    return out


def check_model_params(name, params, dev, ref):
    out = {}
    for p, x, y in zip(params, dev, ref):
        out[p.name] = check_param(f"{name} param {p.name}", x, y, p.param_dtype)["max_ulp"]
    return out
