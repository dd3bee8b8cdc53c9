"""Device memory for one rank's step, allocated with PyTorch.

Per flat buffer: the grad window arena (read by the step), the param window
arena (written back), and the fp32 master / Adam m / Adam v arenas, all of
``arena_numel`` elements; plus the workspace.  Allocation only; the step runs
in the library.

Placement search.  On MI355X the speed of the step's second pass (half reads,
half writes, five arrays streamed at once) depends on where the driver puts
the arrays' pages in HBM: re-allocating the same arenas in one process moved
that pass between 4.9 and 5.9 ms on the Llama-3-8B rank, with the same kernel.
With ``placement_tries = n > 1`` the allocator creates up to n candidate sets
of arenas, each while the earlier ones are still held (so each gets other
pages), times the second pass on each (zeroed data, through the C ABI), keeps
the fastest and frees the rest.  The number of whole sets is capped by the
free device memory.  The kept set is then refined one array at a time: up to
n candidates for that array, the others fixed, the fastest kept.  (Whole sets
found the fast placements of the 16 GB Llama-3 ranks, which refining array by
array alone did not; refining the best whole set took their step a further
0.5-1% faster, and the 108 GB dense-7B state, of which only two sets fit,
from 34.4 to 31.2 ms.)  The search runs once, before any data is loaded; the
arenas then serve every step of the run.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import torch

from . import DOPT_MAX_HGROUPS, DTYPE_NAMES, Layout

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
ES = {"f32": 4, "bf16": 2, "f16": 2}


class DeviceArenas:
    def __init__(self, layout: Layout, device: str = "cuda", placement_tries: int = 1,
                 timed_launches: int = 5):
        self.layout = layout
        self.device = device
        self.info = []
        for k in range(layout.num_buffers):
            b = layout.buffer(k)
            pd, gd = DTYPE_NAMES[b["param_dtype"]], DTYPE_NAMES[b["grad_dtype"]]
            self.info.append({"pd": pd, "gd": gd, "n": b["arena_numel"], **b})
        self.placement: Optional[Dict] = None
        if placement_tries > 1:
            self.bufs, self.workspace = self._search(placement_tries, timed_launches)
        else:
            self.bufs, self.workspace = self._alloc()

    def _alloc(self) -> Tuple[List[Dict[str, torch.Tensor]], torch.Tensor]:
        bufs = []
        for inf in self.info:
            n, pd, gd = inf["n"], inf["pd"], inf["gd"]
            bufs.append({
                "grad": torch.zeros(n, dtype=TORCH_DTYPES[gd], device=self.device),
                "param": torch.zeros(n, dtype=TORCH_DTYPES[pd], device=self.device),
                "master": torch.zeros(n, dtype=torch.float32, device=self.device) if pd != "f32" else None,
                "exp_avg": torch.zeros(n, dtype=torch.float32, device=self.device),
                "exp_avg_sq": torch.zeros(n, dtype=torch.float32, device=self.device),
            })
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

    def state_bytes(self) -> int:
        tot = 0
        for t in self.bufs:
            for v in t.values():
                if v is not None:
                    tot += v.numel() * v.element_size()
        return tot + self.workspace.numel()
