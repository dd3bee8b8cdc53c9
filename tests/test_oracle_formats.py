"""Pins for the oracle's numeric-format conversions.

The fp32 master is written back to the 16-bit param with round-to-nearest-
even ("Megatron-LM distrib_optimizer.py 源码精读", the master-to-model copy in
the data-flow walk-through; read as the IEEE default rounding).  Checked
exhaustively over all 2^32 binary32 patterns against PyTorch's cast (a
library routine), and on a sample against an exact-arithmetic formulation
written with Python fractions.
"""
from fractions import Fraction
import math
import random

import numpy as np
import pytest
import torch

import oracle

FMT = {  # significand bits (incl. hidden), min normal exponent, max exponent
    "bf16": (8, -126, 127),
    "f16": (11, -14, 15),
}


def _exact_round(x: float, fmt: str):
    """Nearest value of the format to x (ties to even), by exact arithmetic; None for NaN."""
    p, emin, emax = FMT[fmt]
    if math.isnan(x):
        return None
    if math.isinf(x) or x == 0.0:
        return x
    a = Fraction(abs(x))
    e = math.frexp(abs(x))[1] - 1  # abs(x) in [2^e, 2^(e+1))
    q = Fraction(2) ** (max(e, emin) - (p - 1))
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * q
    if r >= Fraction(2) ** (emax + 1):
        return math.copysign(math.inf, x)
    return math.copysign(float(r), x)


def _decode(bits: int, fmt: str) -> float:
    L = oracle.lib()
    return L.or_bf16_to_f32(bits) if fmt == "bf16" else L.or_f16_to_f32(bits)


def test_upcast_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    out = np.empty(65536, np.float32)
    oracle.lib().or_bf16_to_f32_n(h.ctypes.data, out.ctypes.data, 65536)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(out), nan)
    assert np.array_equal(out.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])
    oracle.lib().or_f16_to_f32_n(h.ctypes.data, out.ctypes.data, 65536)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(out), nan)
    assert np.array_equal(out.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_downcast_exhaustive_vs_library(fmt):
    L = oracle.lib()
    fn = L.or_f32_to_bf16_n if fmt == "bf16" else L.or_f32_to_f16_n
    tdt = torch.bfloat16 if fmt == "bf16" else torch.float16
    chunk = 1 << 26
    y = np.empty(chunk, np.uint16)
    base = np.arange(chunk, dtype=np.uint32)
    u = np.empty(chunk, np.uint32)
    ref_t = torch.empty(chunk, dtype=tdt)
    ref = ref_t.view(torch.int16).numpy().view(np.uint16)
    xnan = np.empty(chunk, bool)
    same = np.empty(chunk, bool)
    for c in range(0, 1 << 32, chunk):
        np.add(base, np.uint32(c), out=u)
        x = u.view(np.float32)
        fn(x.ctypes.data, y.ctypes.data, chunk)
        ref_t.copy_(torch.from_numpy(x))
        np.isnan(x, out=xnan)
        np.equal(y, ref, out=same)
        np.logical_or(same, xnan, out=same)
        if not same.all():
            bad = np.flatnonzero(~same)[:5]
            raise AssertionError(f"{fmt}: mismatch at {u[bad]} oracle {y[bad]} ref {ref[bad]}")
        # NaN in -> NaN out (sign and payload are not compared)
        exp_mask, man_mask = (0x7f80, 0x7f) if fmt == "bf16" else (0x7c00, 0x3ff)
        yn = y[xnan]
        assert np.all(((yn & exp_mask) == exp_mask) & ((yn & man_mask) != 0))


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_downcast_exact_arithmetic(fmt):
    L = oracle.lib()
    fn = L.or_f32_to_bf16 if fmt == "bf16" else L.or_f32_to_f16
    rng = random.Random(1234)
    cases = []
    for _ in range(6000):
        cases.append(np.uint32(rng.getrandbits(32)).view(np.float32).item())
    # ties and boundaries of the target format
    p, emin, emax = FMT[fmt]
    for e in list(range(emin - p - 2, emin + 3)) + [0, 1, emax - 1, emax]:
        for k in range(0, 8):
            base = 2.0 ** e
            q = 2.0 ** (max(e, emin) - (p - 1))
            for v in (base + k * q, base + k * q + q / 2, base + k * q + q / 4, base + k * q + 3 * q / 4):
                f = np.float32(v)
                if np.isfinite(f):
                    cases += [float(f), -float(f)]
    big = (2 - 2.0 ** (1 - p)) * 2.0 ** emax
    cases += [float(np.float32(big)), float(np.float32(big + 2.0 ** (emax - p))), 0.0, -0.0, math.inf, -math.inf]
    for x in cases:
        want = _exact_round(x, fmt)
        got = _decode(fn(x), fmt)
        if want is None:
            assert math.isnan(got)
            continue
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (fmt, x, got, want)
