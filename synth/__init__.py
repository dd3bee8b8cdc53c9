"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This package generates inputs only: model-shaped parameter lists, initial
weights, per-step gradients, zero masks and the index of an injected
overflow.  It contains none of the optimizer step's arithmetic.  Random draws
come from the counter-based generator in ``gen.c`` (SplitMix64 + Box-Muller),
so any sub-range of any array can be produced on its own.  Narrowing a drawn
fp32 value to bf16/fp16 storage is done by PyTorch's CPU cast.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .models import PARAM_LISTS, ParamSpec  # noqa: F401
from .workloads import WORKLOADS, Workload  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

# Stream ids: each kind of draw has its own stream so that draws never alias.
STREAM_WEIGHT = 1
STREAM_GRAD = 2
STREAM_ZERO_MASK = 3
STREAM_INF_POS = 4
STREAM_CHUNK = 5
STREAM_LOCAL_GRAD = 6
_BUFFER_STRIDE = 64  # stream offset between flat buffers


def build(force: bool = True) -> str:
    """Compile gen.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "gen.c")
        tmp = _SO + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        lib.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                         ctypes.c_int64, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                         ctypes.c_uint64, ctypes.c_void_p]
        lib.synth_normal_f32.restype = None
        lib.synth_uniform_index.argtypes = [ctypes.c_uint64] * 5
        lib.synth_uniform_index.restype = ctypes.c_uint64
        _lib = lib
    return _lib


def normal_f32(seed: int, stream: int, step: int, index0: int, n: int, sigma: float,
               mean: float = 0.0, zero_frac: float = 0.0, out: np.ndarray | None = None) -> np.ndarray:
    """fp32 draws of N(mean, sigma^2) for indices [index0, index0+n)."""
    lib = _load()
    if out is None:
        out = np.empty(n, dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size >= n
    lib.synth_normal_f32(seed, stream, step, index0, n, mean, sigma, zero_frac, STREAM_ZERO_MASK,
                         out.ctypes.data)
    return out


def uniform_index(seed: int, stream: int, step: int, index: int, bound: int) -> int:
    return int(_load().synth_uniform_index(seed, stream, step, index, bound))


def buffer_stream(stream: int, buffer_index: int) -> int:
    return stream + _BUFFER_STRIDE * buffer_index


def weight_stream(buffer_index: int) -> int:
    return buffer_stream(STREAM_WEIGHT, buffer_index)


def grad_stream(buffer_index: int) -> int:
    return buffer_stream(STREAM_GRAD, buffer_index)


def local_grad_stream(buffer_index: int) -> int:
    """Stream of a rank's whole local (pre-communication) grad buffer."""
    return buffer_stream(STREAM_LOCAL_GRAD, buffer_index)


def chunk_stream(buffer_index: int) -> int:
    """Stream of the received (pre-reduction) grad chunks of one buffer."""
    return buffer_stream(STREAM_CHUNK, buffer_index)


_TORCH_DTYPES = None


def torch_dtype(name: str):
    global _TORCH_DTYPES
    import torch
    if _TORCH_DTYPES is None:
        _TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    return _TORCH_DTYPES[name]


def fill_normal(dtype: str, n: int, seed: int, stream: int, step: int, sigma: float, scale: float = 1.0,
                zero_frac: float = 0.0, chunk: int = 1 << 26, out=None):
    """Host tensor of ``n`` elements of ``dtype`` holding storage(scale * N(0, sigma^2)).

    The draw is made in fp32 by the C generator (x = (float)(sigma*Z)); when
    ``scale`` != 1 the fp32 value is multiplied by ``scale`` in fp32 first
    (loss-scaled gradients use a power-of-two scale, so this is exact).  The
    result is narrowed to ``dtype`` by torch's round-to-nearest-even cast.
    """
    import torch
    tdt = torch_dtype(dtype)
    if out is None:
        out = torch.empty(n, dtype=tdt)
    assert out.dtype == tdt and out.numel() >= n
    buf = np.empty(min(chunk, max(n, 1)), dtype=np.float32)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        normal_f32(seed, stream, step, s, m, sigma, zero_frac=zero_frac, out=buf[:m])
        t = torch.from_numpy(buf[:m])
        if scale != 1.0:
            t = t * np.float32(scale)
        out[s:s + m].copy_(t)
    return out
