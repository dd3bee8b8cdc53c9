"""Pins for the oracle's local half of the fp32-accumulating reduce-scatter
("Megatron-LM distributed 包深度解析…" §3.2, reduce_scatter_with_fp32_accumulation:
low precision on the wire, fp32 accumulation on the receiving rank).

Closed forms: sums of small integers are exact; the accumulation is fp32
(not the wire precision); the sum runs in chunk order (a cancellation case
that depends on the order); the scale multiplies once; N = 1 is a copy."""
import numpy as np
import pytest
import torch

import oracle
from synth.models import ParamSpec
from tests.oracle_harness import as_f32, to_bits

WIRE = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _layout(n, gd, N=1, r=0):
    return oracle.Layout([ParamSpec("w", n, "bf16", gd)], N, r, 0)


def _reduce(L, chunks_f32: np.ndarray, wire: str, gd: str, scale=1.0):
    """chunks_f32: (N, n) values exactly representable in the wire dtype."""
    N, n = chunks_f32.shape
    wire_arr = to_bits(torch.from_numpy(np.ascontiguousarray(chunks_f32.reshape(-1))).to(WIRE[wire])).copy()
    out = np.zeros(n, np.float32 if gd == "f32" else np.uint16)
    oracle.lib().or_reduce_chunks(L.handle, 0, wire_arr.ctypes.data, oracle.DTYPES[wire], N, n, scale, 0, n,
                                  out.ctypes.data)
    return as_f32(out, gd)


@pytest.mark.parametrize("wire,gd", [("bf16", "f32"), ("f16", "f32"), ("bf16", "bf16"), ("f32", "f32")])
def test_integer_sums_are_exact(wire, gd):
    rng = np.random.default_rng(0)
    n, N = 4096, 8
    x = rng.integers(-64, 65, size=(N, n)).astype(np.float32)
    got = _reduce(_layout(n, gd, 1, 0), x, wire, gd)
    exact = torch.from_numpy(x.astype(np.int64).sum(0).astype(np.float32))  # |sum| <= 512: exact in fp32
    assert np.array_equal(got, exact.to(WIRE[gd]).float().numpy())  # then stored in the grad dtype


def test_accumulation_is_fp32_not_wire_precision():
    # 1 + 7 * 2^-8 is exact in fp32; added in bf16 (8-bit significand) every
    # 2^-8 step would round back to 1.  Stored as fp32 it stays exact; stored
    # as bf16 the exact sum 1 + 3.5 * 2^-7 rounds to even: 1 + 4 * 2^-7.
    n = 128
    x = np.zeros((8, n), np.float32)
    x[0] = 1.0
    x[1:] = 2.0 ** -8
    assert np.all(_reduce(_layout(n, "f32"), x, "bf16", "f32") == np.float32(1 + 7 * 2.0 ** -8))
    assert np.all(_reduce(_layout(n, "bf16"), x, "bf16", "bf16") == np.float32(1 + 4 * 2.0 ** -7))


def test_summation_runs_in_chunk_order():
    # (2^25 + 1) rounds to 2^25 in fp32, so chunk order [2^25, 1, -2^25] gives 0
    # while [2^25, -2^25, 1] gives 1.
    n = 64
    a = np.zeros((3, n), np.float32)
    a[0], a[1], a[2] = 2.0 ** 25, 1.0, -(2.0 ** 25)
    assert np.all(_reduce(_layout(n, "f32"), a, "f32", "f32") == 0.0)
    b = a[[0, 2, 1]]
    assert np.all(_reduce(_layout(n, "f32"), b, "f32", "f32") == 1.0)


def test_scale_once_and_single_chunk_copy():
    rng = np.random.default_rng(1)
    n = 1024
    x = rng.integers(-256, 257, size=(8, n)).astype(np.float32)  # exact on a bf16 wire
    got = _reduce(_layout(n, "f32"), x, "bf16", "f32", scale=0.125)
    assert np.array_equal(got, (x.astype(np.int64).sum(0) / 8).astype(np.float32))
    y = torch.randn(1, n).to(torch.bfloat16).float().numpy()
    assert np.array_equal(_reduce(_layout(n, "f32"), y, "bf16", "f32"), y[0])
    assert np.array_equal(_reduce(_layout(n, "bf16"), y, "bf16", "bf16"), y[0])


def test_covers_padding_slots_of_the_window():
    # 100 elements at N=4: window of rank 1 is [32, 64) of a 128-element bucket;
    # every window slot (param or padding) gets the reduced value
    L = _layout(100, "f32", 4, 3)
    w = L.buffer(0)["window_numel"]
    assert w == 32
    x = np.ones((4, w), np.float32)
    assert np.all(_reduce(L, x, "bf16", "f32") == 4.0)
