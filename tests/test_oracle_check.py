"""Pins for the oracle's whole-bucket pre-communication check
("Megatron-LM distributed 包深度解析…" §2.4 check_grads, §3.2
check_for_nan_in_grad / check_for_large_grads).

Closed forms: constant grads give n*a^2 and |a|; a NaN sets has_nan and is
ignored by the maximum; an infinity sets has_inf and is the maximum;
"large" is max |g| > threshold (strict); splitting a bucket into ranges and
combining them gives the same result; the sum of squares equals the library
two-norm squared; bucket padding (zeros) is part of the scan and changes
nothing."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from synth.models import ParamSpec
from tests.oracle_harness import to_bits


def _check(L, k, b, grad_bits, lo, hi, thr):
    s, m, f = ctypes.c_double(), ctypes.c_float(), (ctypes.c_int32 * 3)()
    oracle.lib().or_check_bucket(L.handle, k, b, grad_bits.ctypes.data, lo, hi, thr, ctypes.byref(s),
                                 ctypes.byref(m), f)
    return s.value, m.value, tuple(f)


def _buf(L, values: np.ndarray, dt: str):
    n = L.buffer(0)["numel"]
    x = np.zeros(n, np.float32)
    x[:len(values)] = values
    return to_bits(torch.from_numpy(x).to({"bf16": torch.bfloat16, "f16": torch.float16,
                                            "f32": torch.float32}[dt])).copy()


def test_constant_grads_closed_form():
    L = oracle.Layout([ParamSpec("w", 4096, "bf16", "bf16")], 1, 0)
    g = _buf(L, np.full(4096, -0.25, np.float32), "bf16")
    s, m, f = _check(L, 0, 0, g, 0, 1 << 40, 0.0)
    assert s == 4096 * 0.0625 and m == 0.25 and f == (0, 0, 0)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_nan_inf_and_large(dt):
    L = oracle.Layout([ParamSpec("w", 1000, dt, dt)], 1, 0)
    base = np.linspace(-1, 1, 1000).astype(np.float32)
    g = _buf(L, base, dt)
    s0, m0, f0 = _check(L, 0, 0, g, 0, 1 << 40, 0.5)
    assert f0 == (0, 0, 1) and m0 == 1.0
    assert _check(L, 0, 0, g, 0, 1 << 40, 1.0)[2] == (0, 0, 0)  # strict: max == threshold is not large
    v = base.copy()
    v[10] = np.nan
    s, m, f = _check(L, 0, 0, _buf(L, v, dt), 0, 1 << 40, 0.0)
    assert math.isnan(s) and f == (1, 0, 0) and m == 1.0  # NaN ignored by the maximum
    v[20] = -np.inf
    s, m, f = _check(L, 0, 0, _buf(L, v, dt), 0, 1 << 40, 0.0)
    assert math.isnan(s) and f == (1, 1, 0) and math.isinf(m)
    w = base.copy()
    w[999] = np.inf
    s, m, f = _check(L, 0, 0, _buf(L, w, dt), 0, 1 << 40, 2.0)
    assert math.isinf(s) and f == (0, 1, 1) and math.isinf(m)


def test_ranges_combine_and_library_norm():
    L = oracle.Layout([ParamSpec("a", 50000, "f32", "f32"), ParamSpec("b", 777, "f32", "f32")], 4, 1, 20000)
    n = L.buffer(0)["numel"]
    x = np.random.default_rng(0).standard_normal(n).astype(np.float32)
    g = x.copy()
    for b in range(L.buffer(0)["n_buckets"]):
        bk = L.bucket(0, b)
        lo, hi = bk["offset"], bk["offset"] + bk["numel"]
        whole = _check(L, 0, b, g, 0, n, 0.0)
        parts = [_check(L, 0, b, g, a, min(a + 997, hi), 0.0) for a in range(lo, hi, 997)]
        assert whole[1] == max(p[1] for p in parts)
        assert math.isclose(whole[0], sum(p[0] for p in parts), rel_tol=1e-12)
        ref = float(np.linalg.norm(x[lo:hi].astype(np.float64))) ** 2
        assert math.isclose(whole[0], ref, rel_tol=1e-12)
        assert whole[1] == np.abs(x[lo:hi]).max()


def test_padding_is_scanned_and_adds_nothing():
    # 100 elements at N=4 pad to a 128-element bucket; the padding slots are
    # part of the bucket and hold zeros
    L = oracle.Layout([ParamSpec("w", 100, "bf16", "bf16")], 4, 0)
    assert L.bucket(0, 0)["numel"] == 128
    g = _buf(L, np.full(100, 0.5, np.float32), "bf16")
    s, m, f = _check(L, 0, 0, g, 0, 1 << 40, 0.0)
    assert s == 100 * 0.25 and m == 0.5
