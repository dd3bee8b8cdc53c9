"""ORACLE -- test infrastructure only.

ctypes binding of ``oracle.c``, the plain single-threaded C statement of the
shard-local mixed-precision AdamW step.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import this package; the
product library never does.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, List, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F16 = 0, 1, 2
DTYPES = {"f32": F32, "bf16": BF16, "f16": F16}
GROUP_KINDS = {"model_float16": 0, "model_fp32": 1, "shard_float16": 2,
               "shard_fp32_from_float16": 3, "shard_fp32": 4}
MAX_HGROUPS = 16

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain C, no contraction)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.run(["gcc", *CFLAGS, os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _SO)
    return _SO


class Param(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("param_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
                ("requires_new_bucket", ctypes.c_int32), ("hgroup", ctypes.c_int32)]


class HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


class Scaler(ctypes.Structure):
    _fields_ = [("dynamic", ctypes.c_int32), ("hysteresis", ctypes.c_int32), ("growth_interval", ctypes.c_int64),
                ("growth_factor", ctypes.c_double), ("backoff_factor", ctypes.c_double),
                ("min_scale", ctypes.c_double), ("scale", ctypes.c_double), ("growth_tracker", ctypes.c_int64),
                ("hysteresis_tracker", ctypes.c_int64)]


class Stats(ctypes.Structure):
    _fields_ = [("found_inf", ctypes.c_int32), ("skipped", ctypes.c_int32), ("clip_applied", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("sumsq", ctypes.c_double), ("norm", ctypes.c_double),
                ("clip_coef", ctypes.c_double), ("zeros", ctypes.c_uint64), ("scale_used", ctypes.c_double),
                ("scale_next", ctypes.c_double), ("t", ctypes.c_int64)]


_F16 = ctypes.c_float * MAX_HGROUPS


class Scalars(ctypes.Structure):
    _fields_ = [("skip", ctypes.c_int32), ("clip_on", ctypes.c_int32), ("inv_scale", ctypes.c_float),
                ("clip", ctypes.c_float), ("decay", _F16), ("beta1", _F16), ("omb1", _F16), ("beta2", _F16),
                ("omb2", _F16), ("eps", _F16), ("step_size", _F16), ("sqrt_bc2", _F16)]


class Arrays(ctypes.Structure):
    _fields_ = [("grad", ctypes.c_void_p), ("param", ctypes.c_void_p), ("master", ctypes.c_void_p),
                ("m", ctypes.c_void_p), ("v", ctypes.c_void_p)]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    L = ctypes.CDLL(_SO)
    P, I32, I64, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    sig = {
        "or_build": ([P(Param), I64, I32, I32, I64, I32, P(VP)], ctypes.c_int),
        "or_build_instances": ([P(Param), I64, I32, I32, I32, I64, I32, P(VP)], ctypes.c_int),
        "or_free": ([VP], None),
        "or_error": ([], ctypes.c_char_p),
        "or_num_buffers": ([VP], I32),
        "or_buffer": ([VP, I32, P(I64)], ctypes.c_int),
        "or_bucket": ([VP, I32, I32, P(I64)], ctypes.c_int),
        "or_param_info": ([VP, I64, P(I64)], ctypes.c_int),
        "or_group": ([VP, I32, I32, VP, I64], I64),
        "or_segments": ([VP, I32, VP, VP, VP, I64], I64),
        "or_bf16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
        "or_f16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
        "or_f32_to_bf16": ([ctypes.c_float], ctypes.c_uint16),
        "or_f32_to_f16": ([ctypes.c_float], ctypes.c_uint16),
        "or_f32_to_bf16_n": ([VP, VP, I64], None),
        "or_f32_to_f16_n": ([VP, VP, I64], None),
        "or_bf16_to_f32_n": ([VP, VP, I64], None),
        "or_f16_to_f32_n": ([VP, VP, I64], None),
        "or_init_state": ([VP, P(Arrays)], None),
        "or_reduce_chunks": ([VP, I32, VP, I32, I32, I64, ctypes.c_float, I64, I64, VP], None),
        "or_check_bucket": ([VP, I32, I32, VP, I64, I64, ctypes.c_double, P(ctypes.c_double), P(ctypes.c_float),
                             P(I32)], None),
        "or_grad_stats": ([VP, P(Arrays), ctypes.c_float, P(Stats)], None),
        "or_grad_stats_range": ([VP, I32, VP, ctypes.c_float, I64, I64, P(Stats)], None),
        "or_decide": ([P(Stats), P(Scaler), P(I64), P(HParams), I32, ctypes.c_double, P(Scalars)], ctypes.c_int),
        "or_apply": ([VP, P(Arrays), P(Scalars)], None),
        "or_apply_elems": ([I32, I32, I64, VP, VP, VP, VP, VP, VP, P(Scalars)], None),
        "or_apply_range": ([VP, I32, P(Arrays), P(Scalars), I64, I64], None),
        "or_step": ([VP, P(Arrays), P(Scaler), P(I64), P(HParams), I32, ctypes.c_double, P(Stats)], ctypes.c_int),
        "or_inv_scale": ([P(Scaler)], ctypes.c_float),
        "or_state_export": ([VP, P(Arrays), VP, VP, VP], I64),
        "or_state_import": ([VP, P(Arrays), VP, VP, VP], None),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def lib():
    return _load()


class OracleError(RuntimeError):
    pass


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        assert a.flags.c_contiguous
        return a.ctypes.data
    return a.data_ptr()  # torch CPU tensor


class Layout:
    """The oracle's shard layout for one rank (integer results)."""

    def __init__(self, params: Sequence, dp_size: int, dp_rank: int, bucket_size: int = 0, pad_busbw: int = 0,
                 instances: int = 1):
        L = _load()
        n = len(params)
        arr = (Param * n)()
        for i, p in enumerate(params):
            arr[i].numel = p.numel
            arr[i].param_dtype = DTYPES[p.param_dtype]
            arr[i].grad_dtype = DTYPES[p.grad_dtype]
            arr[i].requires_new_bucket = int(getattr(p, "requires_new_bucket", 0))
            arr[i].hgroup = int(getattr(p, "hgroup", 0))
        h = ctypes.c_void_p()
        if instances == 1:
            rc = L.or_build(arr, n, dp_size, dp_rank, bucket_size, pad_busbw, ctypes.byref(h))
        else:
            rc = L.or_build_instances(arr, n, dp_size, dp_rank, instances, bucket_size, pad_busbw, ctypes.byref(h))
        if rc != 0:
            raise OracleError(L.or_error().decode())
        self._h = h
        self._free = L.or_free  # kept so that freeing works during interpreter shutdown
        self.dp_size, self.dp_rank, self.n_params = dp_size, dp_rank, n

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None:
            self._free(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    @property
    def num_buffers(self) -> int:
        return int(_lib.or_num_buffers(self._h))

    def buffer(self, k: int) -> Dict[str, int]:
        o = (ctypes.c_int64 * 8)()
        if _lib.or_buffer(self._h, k, o) != 0:
            raise OracleError(_lib.or_error().decode())
        keys = ["param_dtype", "grad_dtype", "n_buckets", "n_params", "numel", "numel_unpadded",
                "window_numel", "shard_numel"]
        return dict(zip(keys, list(o)))

    def bucket(self, k: int, b: int) -> Dict[str, int]:
        o = (ctypes.c_int64 * 7)()
        if _lib.or_bucket(self._h, k, b, o) != 0:
            raise OracleError(_lib.or_error().decode())
        keys = ["offset", "numel", "numel_unpadded", "shard", "window_start", "arena_offset", "n_params"]
        return dict(zip(keys, list(o)))

    def param(self, p: int) -> Dict:
        o = (ctypes.c_int64 * 15)()
        if _lib.or_param_info(self._h, p, o) != 0:
            raise OracleError(_lib.or_error().decode())
        v = list(o)
        return {"buffer": v[0], "bucket": v[1], "start": v[2], "end": v[3], "has_shard": v[4], "hgroup": v[5],
                "gbuf_world": (v[6], v[7]), "gbuf_world_in_bucket": (v[8], v[9]), "gbuf_local": (v[10], v[11]),
                "param": (v[12], v[13]), "arena_offset": v[14]}

    def group(self, kind: str, hgroup: int = 0) -> List[int]:
        k = GROUP_KINDS[kind]
        n = _lib.or_group(self._h, k, hgroup, None, 0)
        buf = np.zeros(max(n, 1), dtype=np.int64)
        _lib.or_group(self._h, k, hgroup, buf.ctypes.data, n)
        return buf[:n].tolist()

    def segments(self, k: int):
        n = _lib.or_segments(self._h, k, None, None, None, 0)
        s = np.zeros(max(n, 1), np.int64)
        ln = np.zeros(max(n, 1), np.int64)
        pr = np.zeros(max(n, 1), np.int64)
        _lib.or_segments(self._h, k, s.ctypes.data, ln.ctypes.data, pr.ctypes.data, n)
        return s[:n], ln[:n], pr[:n]

    def valid_mask(self, k: int, n: int) -> np.ndarray:
        """Boolean mask over ``n`` arena slots of buffer k: True where a param element lives."""
        m = np.zeros(n, dtype=bool)
        s, ln, _ = self.segments(k)
        for a, b in zip(s.tolist(), ln.tolist()):
            m[a:a + b] = True
        return m

    def hgroup_at(self, k: int, idx: np.ndarray) -> np.ndarray:
        """Hyper-group of the param owning each arena index (which must be valid)."""
        s, ln, pr = self.segments(k)
        pos = np.searchsorted(s, idx, side="right") - 1
        hg = np.array([self.param(int(p))["hgroup"] for p in pr.tolist()], dtype=np.int32) if len(pr) else \
            np.zeros(0, np.int32)
        assert np.all(pos >= 0) and np.all(idx < s[pos] + ln[pos]), "index not owned by a param"
        return hg[pos]


def arrays(grad=None, param=None, master=None, m=None, v=None) -> Arrays:
    a = Arrays()
    a.grad, a.param, a.master, a.m, a.v = _ptr(grad), _ptr(param), _ptr(master), _ptr(m), _ptr(v)
    return a


def make_scaler(dynamic: bool, scale: float, growth_factor: float = 2.0, backoff_factor: float = 0.5,
                growth_interval: int = 1000, hysteresis: int = 1, min_scale: float = 1.0) -> Scaler:
    s = Scaler()
    s.dynamic = int(dynamic)
    s.hysteresis = hysteresis
    s.growth_interval = growth_interval
    s.growth_factor, s.backoff_factor, s.min_scale = growth_factor, backoff_factor, min_scale
    s.scale = scale
    s.growth_tracker = 0
    s.hysteresis_tracker = hysteresis
    return s


def make_hparams(hps) -> ctypes.Array:
    arr = (HParams * len(hps))()
    for i, h in enumerate(hps):
        arr[i].lr, arr[i].beta1, arr[i].beta2, arr[i].eps, arr[i].weight_decay = h
    return arr
