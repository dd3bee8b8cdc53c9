"""Device memory for one rank's step.

Per flat buffer: the grad window arena (read by the step), the param window
arena (written back), and the fp32 master / Adam m / Adam v arenas, all of
``arena_numel`` elements; plus the workspace.  Allocation only; the step runs
in the library.

Placement.  The step's second pass reads four arrays and writes four at the
same index at once, and on MI355X how fast it runs depends on where the
arrays' physical pages sit relative to each other: the same kernel took
4.9-5.9 ms on the Llama-3-8B rank from one allocation to the next.  Plain
streams on the same arrays show that the placement decides the writes: five
arrays written at once ran at 5.5 TB/s on an ordinary allocation and 7.2 TB/s
on a fast one, while five read at once stayed near 6 TB/s on both; pass 2 ran
at 5.1 and 6.1 TB/s.  Which pages are fast cannot be read from user space, so
it is measured:

- ``placement="regions"`` (large buffers): each array is a reserved address
  range backed region by region (``dopt_vmm.h``; regions of 2^27 elements).
  For every region and array, candidate backings are mapped in turn and
  pass 2 is timed on that region alone; the fastest is kept.  Per region the
  times fall into two groups (about 5.4 and 6.1 TB/s); enough candidates and
  sweeps bring every region to the faster one (see DeviceArenas).  The search holds at most one region of memory per
  candidate and took 0.3-9 s for the Llama-3 ranks and the 108 GB dense-7B
  state with 2 sweeps, 8 candidates and a 1% tolerance (40-50 s for dense-7B
  with 3 sweeps, 12 candidates and 0.3%, which gained another 0.5%).
- ``placement="sets"``: up to n whole candidate sets of arenas, each allocated
  while the earlier ones are held, the fastest for pass 2 kept, then refined
  one array at a time.  It finds the same 6.1 TB/s plateau when a fast set
  turns up, but needs room for several copies of the state (two for
  dense-7B) and took 18-20 s there.

Either search runs once, before any data is loaded; the arenas then serve
every step.  Without a search (the default) the arrays are plain PyTorch
allocations.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import torch

from . import DOPT_MAX_HGROUPS, DTYPE_NAMES, Layout

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
ES = {"f32": 4, "bf16": 2, "f16": 2}


KEYS = ("grad", "param", "master", "exp_avg", "exp_avg_sq")
# __cuda_array_interface__ type strings; bf16 has none and is viewed from int16
_TYPESTR = {"f32": ("<f4", None), "f16": ("<f2", None), "bf16": ("<i2", torch.bfloat16)}


class _Backing:
    """A reserved device address range whose regions are backed by physical
    allocations of their own (dopt_vmm.h).  Unmapped and released when the
    last tensor viewing it goes away (the tensors hold a reference)."""

    def __init__(self, nbytes: int, region_bytes: int, gran: int):
        from . import dopt_vmm_create, dopt_vmm_map, dopt_vmm_reserve, dopt_vmm_set_access
        # whole regions only (the tail of the last one is backed but unused):
        # the access call on a remapped region was refused on MI355X for a
        # region shorter than the others
        region_bytes = -(-region_bytes // gran) * gran
        self.nbytes = -(-nbytes // region_bytes) * region_bytes
        self.region_bytes = region_bytes
        self.va = dopt_vmm_reserve(self.nbytes, gran)
        self.handles: List[int] = []
        self.mapped = 0
        try:
            for off in range(0, self.nbytes, region_bytes):
                size = min(region_bytes, self.nbytes - off)
                h = dopt_vmm_create(size)
                self.handles.append(h)
                dopt_vmm_map(self.va + off, size, h)
                self.mapped += 1
            dopt_vmm_set_access(self.va, self.nbytes)
        except Exception:
            self.close()
            raise

    def region(self, j: int) -> Tuple[int, int]:
        off = j * self.region_bytes
        return self.va + off, min(self.region_bytes, self.nbytes - off)

    def replace(self, j: int, h: int):
        """Back region j with h (the caller keeps the old handle)."""
        from . import DoptError, dopt_vmm_map, dopt_vmm_set_access, dopt_vmm_unmap
        torch.cuda.synchronize()
        va, size = self.region(j)
        dopt_vmm_unmap(va, size)
        dopt_vmm_map(va, size, h)
        try:
            dopt_vmm_set_access(va, size)
        except DoptError:
            dopt_vmm_set_access(self.va, self.nbytes)
        self.handles[j] = h

    def close(self):
        from . import dopt_vmm_free, dopt_vmm_release, dopt_vmm_unmap
        if getattr(self, "va", None) is None:
            return
        torch.cuda.synchronize()
        for j in range(self.mapped):
            va, size = self.region(j)
            dopt_vmm_unmap(va, size)
        for h in self.handles:
            dopt_vmm_release(h)
        dopt_vmm_free(self.va, self.nbytes)
        self.va = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class _View:
    def __init__(self, backing: _Backing, n: int, typestr: str):
        self.backing = backing  # kept alive by every tensor made from this view
        self.__cuda_array_interface__ = {"shape": (n,), "typestr": typestr, "data": (backing.va, False),
                                         "version": 3, "strides": None}


def _tensor_over(backing: _Backing, n: int, dt: str) -> torch.Tensor:
    ts, view_as = _TYPESTR[dt]
    t = torch.as_tensor(_View(backing, n, ts), device="cuda")
    return t.view(view_as) if view_as is not None else t


def search_regions(ops, nreg: int, keys, tries: int, sweeps: int, tol: float) -> List:
    """The region search's policy, on an `ops` object that backs and times
    regions: ops.region_ms(j) -> (ms, elements) times pass 2 on region j;
    ops.create(key, j) -> a new backing for that region of that array (or
    None when memory runs out); ops.current(key, j); ops.use(key, j, h) maps h
    there; ops.release(h) frees a backing that is not mapped.

    For every region, up to `tries` candidates per array are mapped in turn
    and timed; the fastest backing is kept.  Rejected and replaced backings
    are held until the array's candidates are done (so that each try gets
    other memory) and then released.  A region whose time per element is
    within `tol` of the best region rate seen so far is not searched further.
    Returns, for the last sweep, [region, ms before, ms after, candidates
    tried] per region."""
    best_rate = None  # ms per element of the fastest region so far

    def near_best(ms, m):
        return best_rate is not None and ms / m <= (1.0 + tol) * best_rate

    regions = []
    for sweep in range(sweeps):
        for j in range(nreg):
            first, m = ops.region_ms(j)
            best, tried = first, 0
            for key in keys:
                if near_best(best, m):
                    break
                held = []
                for _ in range(tries):
                    h = ops.create(key, j)
                    if h is None:
                        break
                    old = ops.current(key, j)
                    ops.use(key, j, h)
                    ms, _ = ops.region_ms(j)
                    tried += 1
                    if ms < best:
                        best = ms
                        held.append(old)
                    else:
                        ops.use(key, j, old)
                        held.append(h)
                    if near_best(best, m):
                        break
                for h in held:
                    ops.release(h)
            best_rate = best / m if best_rate is None else min(best_rate, best / m)
            if sweep == sweeps - 1:
                regions.append([j, round(first, 4), round(best, 4), tried])
    return regions


class _VmmRegionOps:
    """search_regions' operations on one buffer's region-backed arrays: new
    backings through dopt_vmm.h, pass 2 timed on one region through the C
    ABI (a one-param layout of the region's length over the same memory)."""

    def __init__(self, inf, back: Dict[str, _Backing], tensors, region_elems: int, launches: int, device):
        from . import DOPT_MAX_HGROUPS as NH, hparams_array
        self.inf, self.back, self.tensors = inf, back, tensors
        self.region_elems, self.launches, self.device = region_elems, launches, device
        self.es = {key: ES[inf["gd"]] if key == "grad" else ES[inf["pd"]] if key == "param" else 4
                   for key in back}
        self.layouts = {}
        self.hp = hparams_array([(1e-3, 0.9, 0.999, 1e-8, 0.0)] * NH)
        self.stream = torch.cuda.current_stream()

    def _span(self, j):
        lo = j * self.region_elems
        return lo, min(self.region_elems, self.inf["n"] - lo)

    def region_ms(self, j):
        from . import dopt_build_ranges, dopt_init_state, dopt_step_apply, dopt_step_prepare, scaler_cfg
        lo, m = self._span(j)
        if m not in self.layouts:
            inf = self.inf

            class _P:
                numel, param_dtype, grad_dtype = m, inf["pd"], inf["gd"]

            Lr = dopt_build_ranges([_P()], 1, 0, 0)
            self.layouts[m] = (Lr, torch.zeros(Lr.workspace_bytes, dtype=torch.uint8, device=self.device))
        Lr, wsr = self.layouts[m]
        rb = [{key: self.back[key].va + lo * self.es[key] for key in self.back}]
        if self.inf["pd"] == "f32":
            rb[0]["master"] = None
        s = self.stream
        dopt_init_state(Lr, rb, scaler_cfg(False, 1.0), wsr, s)
        dopt_step_prepare(Lr, rb, self.hp, 0.0, wsr, s)
        dopt_step_apply(Lr, rb, wsr, s)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(self.launches):
            dopt_step_apply(Lr, rb, wsr, s)
        b.record(s)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / self.launches, m

    def create(self, key, j):
        from . import DoptError, dopt_vmm_create
        try:
            return dopt_vmm_create(self.back[key].region(j)[1])
        except DoptError:
            return None  # out of device memory for candidates

    def current(self, key, j):
        return self.back[key].handles[j]

    def use(self, key, j, h):
        self.back[key].replace(j, h)
        lo, m = self._span(j)
        self.tensors[key][lo:lo + m].zero_()

    def release(self, h):
        from . import dopt_vmm_release
        torch.cuda.synchronize()
        dopt_vmm_release(h)


class DeviceArenas:
    """placement "sets": up to placement_tries whole arena sets, then array by
    array (below); "regions": the large buffers' arrays backed region by
    region through dopt_vmm.h, each region's backing chosen by timing pass 2
    on that region (region_search), with up to placement_tries candidates per
    array and region.

    How many candidates the region search needs depends on where the
    process's memory comes from.  Five 2^30-element arrays allocated first
    in a process started with every region in the slow group (5.1 TB/s for
    pass 2); 8 candidates, 2 sweeps and a 1% tolerance stayed there (the
    first region found no fast backing, and the others were then within the
    tolerance of it), while 16 candidates, 3 sweeps and 0.3% reached the fast
    group (6.1 TB/s) in 4-9 s.  The same arrays allocated after 128 GiB of
    other memory started in the fast group.  The defaults below are the
    sweeps and tolerance that escaped; pass placement_tries of 12 or more."""

    def __init__(self, layout: Layout, device: str = "cuda", placement_tries: int = 1,
                 timed_launches: int = 5, placement: str = "sets", region_elems: int = 1 << 27,
                 region_sweeps: int = 3, region_tolerance: float = 0.003):
        self.layout = layout
        self.device = device
        self.info = []
        for k in range(layout.num_buffers):
            b = layout.buffer(k)
            pd, gd = DTYPE_NAMES[b["param_dtype"]], DTYPE_NAMES[b["grad_dtype"]]
            self.info.append({"pd": pd, "gd": gd, "n": b["arena_numel"], **b})
        self.placement: Optional[Dict] = None
        if placement == "regions":
            self.bufs, self.workspace = self._region_search(placement_tries, timed_launches, region_elems,
                                                            region_sweeps, region_tolerance)
        elif placement_tries > 1:
            self.bufs, self.workspace = self._search(placement_tries, timed_launches)
        else:
            self.bufs, self.workspace = self._alloc()

    def _alloc_buffer(self, inf) -> Dict[str, torch.Tensor]:
        n, pd, gd = inf["n"], inf["pd"], inf["gd"]
        return {
            "grad": torch.zeros(n, dtype=TORCH_DTYPES[gd], device=self.device),
            "param": torch.zeros(n, dtype=TORCH_DTYPES[pd], device=self.device),
            "master": torch.zeros(n, dtype=torch.float32, device=self.device) if pd != "f32" else None,
            "exp_avg": torch.zeros(n, dtype=torch.float32, device=self.device),
            "exp_avg_sq": torch.zeros(n, dtype=torch.float32, device=self.device),
        }

    def _alloc(self) -> Tuple[List[Dict[str, torch.Tensor]], torch.Tensor]:
        bufs = [self._alloc_buffer(inf) for inf in self.info]
        ws = torch.zeros(self.layout.workspace_bytes, dtype=torch.uint8, device=self.device)
        return bufs, ws

    def arena_bytes(self) -> int:
        tot = self.layout.workspace_bytes
        for inf in self.info:
            per = ES[inf["gd"]] + ES[inf["pd"]] + 8 + (4 if inf["pd"] != "f32" else 0)
            tot += per * inf["n"]
        return tot

    def _pass2_ms(self, bufs, ws, launches: int) -> float:
        """Average duration of the second pass on these arenas (zeroed data:
        a not-skipped step with zero grads), from HIP events on the stream."""
        from . import dopt_init_state, dopt_step_apply, dopt_step_prepare, hparams_array, scaler_cfg, tensors
        stream = torch.cuda.current_stream()
        dopt_init_state(self.layout, bufs, scaler_cfg(False, 1.0), ws, stream)
        t = tensors(self.layout, bufs)
        hp = hparams_array([(1e-3, 0.9, 0.999, 1e-8, 0.0)] * DOPT_MAX_HGROUPS)
        dopt_step_prepare(self.layout, t, hp, 0.0, ws, stream)
        dopt_step_apply(self.layout, t, ws, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(launches):
            dopt_step_apply(self.layout, t, ws, stream)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / launches

    def _search(self, tries: int, launches: int):
        free, _ = torch.cuda.mem_get_info()
        cap = max(1, min(tries, int(0.9 * free) // max(self.arena_bytes(), 1)))
        cands, times = [], []
        for _ in range(cap):
            bufs, ws = self._alloc()
            times.append(self._pass2_ms(bufs, ws, launches))
            cands.append((bufs, ws))
        best = min(range(len(times)), key=times.__getitem__)
        kept = cands[best]
        # the kept arenas are handed over zeroed, as a plain allocation is
        for t in kept[0]:
            for v in t.values():
                if v is not None:
                    v.zero_()
        kept[1].zero_()
        del cands, bufs, ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        self.placement = {"candidates": len(times), "pass2_ms": [round(x, 4) for x in times], "kept": best}
        self.placement["refined"] = self._refine(kept, tries, launches)
        for t in kept[0]:
            for v in t.values():
                if v is not None:
                    v.zero_()
        kept[1].zero_()
        return kept

    def _refine(self, kept, tries: int, launches: int) -> List:
        """Array-by-array refinement of a kept set: for each array, candidates
        allocated while the earlier ones are held, the fastest kept."""
        bufs, ws = kept
        steps = []
        for k in range(len(bufs)):
            for key in ("grad", "param", "master", "exp_avg", "exp_avg_sq"):
                cur = bufs[k][key]
                if cur is None:
                    continue
                best_t, best_ms = cur, self._pass2_ms(bufs, ws, launches)
                times = [best_ms]
                free, _ = torch.cuda.mem_get_info()
                nbytes = cur.numel() * cur.element_size()
                n = max(0, min(tries, int(0.9 * free) // max(nbytes, 1)))
                held = []
                for _ in range(n):
                    held.append(torch.zeros_like(cur))
                    bufs[k][key] = held[-1]
                    ms = self._pass2_ms(bufs, ws, launches)
                    times.append(ms)
                    if ms < best_ms:
                        best_t, best_ms = held[-1], ms
                bufs[k][key] = best_t
                held.clear()
                cur = None
                # [buffer, array, candidates tried, pass-2 ms of the current
                # array then of each candidate]
                steps.append([k, key, n, [round(x, 4) for x in times]])
                torch.cuda.synchronize()
                torch.cuda.empty_cache()
        return steps

    def _region_search(self, tries: int, launches: int, region_elems: int, sweeps: int, tol: float = 0.01):
        """Buffers of at least 4 regions get their five arrays (four for fp32
        params) as reserved address ranges backed region by region, the
        backings chosen by search_regions with pass 2 timed on one region at
        a time; smaller buffers get plain allocations."""
        from . import dopt_vmm_granularity
        gran = dopt_vmm_granularity(0)
        bufs = [self._alloc_buffer(inf) if inf["n"] < 4 * region_elems else {} for inf in self.info]
        ws = torch.zeros(self.layout.workspace_bytes, dtype=torch.uint8, device=self.device)
        report = []
        self._backings = []
        for k, inf in enumerate(self.info):
            n = inf["n"]
            if n < 4 * region_elems:
                continue
            keys = [key for key in KEYS if not (key == "master" and inf["pd"] == "f32")]
            dts = {"grad": inf["gd"], "param": inf["pd"], "master": "f32", "exp_avg": "f32", "exp_avg_sq": "f32"}
            back = {}
            bufs[k] = {key: None for key in KEYS}
            for key in keys:
                back[key] = _Backing(n * ES[dts[key]], region_elems * ES[dts[key]], gran)
                bufs[k][key] = _tensor_over(back[key], n, dts[key])
                bufs[k][key].zero_()
            self._backings.append(back)
            ops = _VmmRegionOps(inf, back, bufs[k], region_elems, launches, self.device)
            regions = search_regions(ops, -(-n // region_elems), keys, tries, sweeps, tol)
            report.append({"buffer": k, "regions": -(-n // region_elems), "region_elems": region_elems,
                           "sweeps": sweeps, "last_sweep": regions})
        for b in bufs:
            for v in b.values():
                if v is not None:
                    v.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        self.placement = {"kind": "regions", "buffers": report}
        return bufs, ws

    def state_bytes(self) -> int:
        tot = 0
        for t in self.bufs:
            for v in t.values():
                if v is not None:
                    tot += v.numel() * v.element_size()
        return tot + self.workspace.numel()
