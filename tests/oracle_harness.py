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
