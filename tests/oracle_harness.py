"""Test-side helpers that drive the oracle on host arrays (numpy).

Arrays are held per flat buffer in window-arena coordinates; 16-bit values
are kept as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

NP_STORE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16}
DT_NAME = {0: "f32", 1: "bf16", 2: "f16"}


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Host torch tensor -> numpy array in the oracle's storage (uint16 bits for 16-bit types)."""
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def to_torch(a: np.ndarray, dt: str) -> torch.Tensor:
    if dt == "f32":
        return torch.from_numpy(a)
    return torch.from_numpy(a.view(np.int16)).view(synth.torch_dtype(dt))


def as_f32(a: np.ndarray, dt: str) -> np.ndarray:
    """Exact fp32 value of stored elements (upcast through torch)."""
    return to_torch(np.ascontiguousarray(a), dt).float().numpy()


class OracleRun:
    """Holds a layout, its arena arrays and the scaler / step state."""

    def __init__(self, params, dp_size, dp_rank, bucket_size=0, pad_busbw=0, arena_numel=None, instances=1):
        self.L = oracle.Layout(params, dp_size, dp_rank, bucket_size, pad_busbw, instances)
        self.nb = self.L.num_buffers
        self.bufs = []
        for k in range(self.nb):
            b = self.L.buffer(k)
            pd, gd = DT_NAME[b["param_dtype"]], DT_NAME[b["grad_dtype"]]
            n = arena_numel[k] if arena_numel else max(b["window_numel"], 1)
            self.bufs.append({
                "pd": pd, "gd": gd, "n": n,
                "grad": np.zeros(n, NP_STORE[gd]), "param": np.zeros(n, NP_STORE[pd]),
                "master": np.zeros(n, np.float32) if pd != "f32" else None,
                "m": np.zeros(n, np.float32), "v": np.zeros(n, np.float32),
            })
        self.t = 0
        self.scaler = oracle.make_scaler(False, 1.0)

    def arrays(self):
        arr = (oracle.Arrays * self.nb)()
        for k, b in enumerate(self.bufs):
            arr[k] = oracle.arrays(b["grad"], b["param"], b["master"], b["m"], b["v"])
        return arr

    def init_state(self):
        oracle.lib().or_init_state(self.L.handle, self.arrays())

    def step(self, hparams, max_norm):
        import ctypes
        st = oracle.Stats()
        t = ctypes.c_int64(self.t)
        hp = oracle.make_hparams(hparams)
        rc = oracle.lib().or_step(self.L.handle, self.arrays(), ctypes.byref(self.scaler), ctypes.byref(t), hp,
                                  len(hparams), max_norm, ctypes.byref(st))
        assert rc == 0
        self.t = t.value
        return st

    def valid(self, k):
        return self.L.valid_mask(k, self.bufs[k]["n"])


# ------------------------------------------------------- model-space state ---
#
# A model-space copy holds, per param in model order, full-length arrays
# (param coordinates).  A rank's layout places its shard of param p at arena
# slots [arena_offset, arena_offset + hi - lo) of its buffer, where (lo, hi) is
# the shard's param range; the export holds the rank's shards back to back in
# model order.  These helpers work with any layout object whose ``param(p)``
# reports buffer, has_shard, param and arena_offset (the oracle's and the
# library's both do).


def shard_pieces(L, n_params):
    """[(p, buffer, arena_offset, lo, hi, export_offset)] for the rank's shards, model order."""
    out, x = [], 0
    for p in range(n_params):
        d = L.param(p)
        if not d["has_shard"]:
            continue
        lo, hi = d["param"]
        out.append((p, d["buffer"], d["arena_offset"], lo, hi, x))
        x += hi - lo
    return out


def place_in_arenas(L, n_params, full, arenas):
    """arenas[k][arena slots of p's shard] = full[p][lo:hi] for every shard of the rank."""
    for p, k, a, lo, hi, _ in shard_pieces(L, n_params):
        arenas[k][a:a + hi - lo] = full[p][lo:hi]


def export_to_model(L, n_params, exports, full):
    """Write one rank's export arrays (a tuple of three) into model-space arrays full[key][p]."""
    for p, _, _, lo, hi, x in shard_pieces(L, n_params):
        for key, e in zip(("master", "m", "v"), exports):
            full[key][p][lo:hi] = e[x:x + hi - lo]


def model_to_export(L, n_params, full):
    """The rank's export arrays read from model-space state."""
    pieces = shard_pieces(L, n_params)
    n = sum(hi - lo for _, _, _, lo, hi, _ in pieces)
    outs = tuple(np.zeros(n, np.float32) for _ in range(3))
    for p, _, _, lo, hi, x in pieces:
        for key, e in zip(("master", "m", "v"), outs):
            e[x:x + hi - lo] = full[key][p][lo:hi]
    return outs


def oracle_export(run: "OracleRun"):
    n = sum(run.L.buffer(k)["shard_numel"] for k in range(run.nb))
    outs = tuple(np.zeros(max(n, 1), np.float32) for _ in range(3))
    got = oracle.lib().or_state_export(run.L.handle, run.arrays(), *(o.ctypes.data for o in outs))
    assert got == n
    return tuple(o[:n] for o in outs)


def oracle_import(run: "OracleRun", exports):
    ex = tuple(np.ascontiguousarray(e, dtype=np.float32) for e in exports)
    oracle.lib().or_state_import(run.L.handle, run.arrays(), *(e.ctypes.data for e in ex))


class OracleRanks:
    """All N ranks of a data-parallel job on the oracle, joined the way the
    ranks of a real job are: each rank forms its grad-stats partial over its
    own shard, the partials are summed over ranks (sumsq in rank order),
    every rank decides on the sum and updates its own shard."""

    def __init__(self, params, dp_size, bucket_size=0, pad_busbw=0):
        self.params = list(params)
        self.runs = [OracleRun(self.params, dp_size, r, bucket_size, pad_busbw) for r in range(dp_size)]

    def init(self, weights, scaler_args=(False, 1.0)):
        for run in self.runs:
            place_in_arenas(run.L, len(self.params), [to_bits(w) for w in weights],
                            [b["param"] for b in run.bufs])
            run.scaler = oracle.make_scaler(*scaler_args)
            run.init_state()

    def step(self, grads, hparams, max_norm):
        import ctypes
        lib = oracle.lib()
        parts = []
        for run in self.runs:
            for b in run.bufs:
                b["grad"][:] = 0
            place_in_arenas(run.L, len(self.params), [to_bits(g) for g in grads], [b["grad"] for b in run.bufs])
            st = oracle.Stats()
            lib.or_grad_stats(run.L.handle, run.arrays(), lib.or_inv_scale(ctypes.byref(run.scaler)),
                              ctypes.byref(st))
            parts.append(st)
        sumsq, zeros, found = 0.0, 0, 0
        for st in parts:
            sumsq += st.sumsq
            zeros += st.zeros
            found |= st.found_inf
        hp = oracle.make_hparams(hparams)
        out = None
        for run in self.runs:
            st = oracle.Stats()
            st.sumsq, st.zeros, st.found_inf = sumsq, zeros, found
            sc = oracle.Scalars()
            t = ctypes.c_int64(run.t)
            assert lib.or_decide(ctypes.byref(st), ctypes.byref(run.scaler), ctypes.byref(t), hp, len(hparams),
                                 max_norm, ctypes.byref(sc)) == 0
            run.t = t.value
            lib.or_apply(run.L.handle, run.arrays(), ctypes.byref(sc))
            out = st
        return out

    def model_state(self):
        """Model-space (master, m, v) assembled from every rank's export."""
        full = {key: [np.full(p.numel, np.nan, np.float32) for p in self.params] for key in ("master", "m", "v")}
        for run in self.runs:
            export_to_model(run.L, len(self.params), oracle_export(run), full)
        return full

    def model_params(self):
        """Model-space 16/32-bit params (storage bits) assembled from every rank's param window."""
        full = [np.zeros(p.numel, NP_STORE[p.param_dtype]) for p in self.params]
        for run in self.runs:
            for p, k, a, lo, hi, _ in shard_pieces(run.L, len(self.params)):
                full[p][lo:hi] = run.bufs[k]["param"][a:a + hi - lo]
        return full

    def load(self, full, scalars):
        """Import model-space state into every rank, and its scalar state."""
        for run in self.runs:
            oracle_import(run, model_to_export(run.L, len(self.params), full))
            run.t = scalars["t"]
            for key in ("scale", "growth_tracker", "hysteresis_tracker"):
                setattr(run.scaler, key, scalars[key])

    def scalars(self):
        run = self.runs[0]
        return {"t": run.t, "scale": run.scaler.scale, "growth_tracker": run.scaler.growth_tracker,
                "hysteresis_tracker": run.scaler.hysteresis_tracker}
