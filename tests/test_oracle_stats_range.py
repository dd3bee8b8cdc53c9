"""Pins for the oracle's grad statistics restricted to a range of arena slots
(or_grad_stats_range), which checks the norm, the zero count and the
overflow flag of the largest workloads split over host threads.

What the statistics are comes from "Megatron-LM distrib_optimizer.py 源码精读",
section "三层继承体系": the first layer takes the grad norm and counts zeros
over the optimizer's (sharded) params, the second unscales the grads and
detects inf/NaN.  Which arena slots hold a shard element comes from the same
page's "Bucket 级别的均等切分" (rank r owns the r-th of N equal parts of each
bucket) and "Range 类：四种视角的统一抽象".

The reference values here are computed without the oracle's segment walk:
every element of every flat buffer is enumerated, its owner rank is
(element - bucket offset) div (bucket size / N) and its param is found from
the params' buffer ranges; the statistics are then taken over the owned
param elements with an exactly rounded sum (math.fsum).  Values that belong
to no param (alignment gaps, bucket padding, the arena tail) are filled with
inf and NaN, so a range that leaks outside the shard elements fails.
"""
import ctypes
import math
import random

import numpy as np
import pytest

import oracle
from synth.models import ParamSpec, tiny
from tests.oracle_harness import OracleRun

U = 2.0 ** -53  # unit roundoff of binary64
NP_DT = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16}
DT_NAME = {0: "f32", 1: "bf16", 2: "f16"}


def _arena_n(L, k):
    return -(-max(L.buffer(k)["window_numel"], 1) // 2048) * 2048


def _owned_arena_slots(L, params, k, r, N):
    """Arena slots of buffer k that hold an element of a param on rank r,
    found by enumerating every element of the buffer."""
    info = L.buffer(k)
    numel = info["numel"]
    elem_param = np.full(numel, -1, np.int64)
    for i in range(len(params)):
        p = L.param(i)
        if p["buffer"] == k:
            elem_param[p["start"]:p["end"]] = i
    bk = [L.bucket(k, b) for b in range(info["n_buckets"])]
    offs = np.array([b["offset"] for b in bk], np.int64)
    e = np.arange(numel, dtype=np.int64)
    b_of = np.searchsorted(offs, e, side="right") - 1
    shard = np.array([b["numel"] // N for b in bk], np.int64)
    owner = (e - offs[b_of]) // shard[b_of]
    arena_off = np.concatenate([[0], np.cumsum(shard)[:-1]])
    slot = arena_off[b_of] + (e - offs[b_of] - r * shard[b_of])
    mine = (owner == r) & (elem_param >= 0)
    return np.sort(slot[mine])


def _as_f32(bits, dt):
    if dt == "f32":
        return bits.view(np.float32)
    out = np.empty(bits.size, np.float32)
    if dt == "bf16":
        oracle.lib().or_bf16_to_f32_n(bits.ctypes.data, out.ctypes.data, bits.size)
    else:
        oracle.lib().or_f16_to_f32_n(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def _reference(g32, slots, inv):
    """Exactly rounded statistics of the owned slots (fp32 unscale, as the
    method states; the sum of squares in exact arithmetic, rounded once)."""
    x = g32[slots] * np.float32(inv)
    fin = np.isfinite(x)
    found_inf = int(not fin.all())
    sq = [float(v) * float(v) for v in x[fin].tolist()]
    return math.fsum(sq), int(np.count_nonzero(x == 0)), found_inf, len(slots)


def _fill(rng, dt, n, owned, plant_inf_owned):
    """Grad bits: N(0,1e-2)-ish values, 3% exact zeros, a few subnormal-sized
    values; inf and NaN in every slot that holds no shard element."""
    nr = np.random.default_rng(rng.randrange(1 << 30))
    x = (nr.standard_normal(n) * 1e-2).astype(np.float32)
    x[nr.random(n) < 0.03] = 0.0
    tiny_idx = nr.random(n) < 0.01
    x[tiny_idx] = np.float32(1e-39) if dt == "f32" else np.float32(3e-8)
    not_owned = np.ones(n, bool)
    not_owned[owned] = False
    bad = np.flatnonzero(not_owned)
    x[bad[0::2]] = np.inf
    x[bad[1::2]] = np.nan
    if plant_inf_owned and owned.size:
        x[owned[nr.integers(0, owned.size)]] = -np.inf
    if dt == "f32":
        return x.view(np.uint32).view(np.float32).copy()
    out = np.empty(n, np.uint16)
    f = oracle.lib().or_f32_to_bf16_n if dt == "bf16" else oracle.lib().or_f32_to_f16_n
    f(x.ctypes.data, out.ctypes.data, n)
    return out


def _range_stats(L, k, g, inv, lo, hi):
    st = oracle.Stats()
    oracle.lib().or_grad_stats_range(L.handle, k, g.ctypes.data, inv, lo, hi, ctypes.byref(st))
    return st.sumsq, st.zeros, st.found_inf


def _cuts(rng, L, k, n):
    """Cut points: inside segments, on segment ends, inside gaps and padding,
    on 2048-slot tile edges and next to them, and random ones."""
    s, ln, _ = L.segments(k)
    pts = {0, n}
    for a, b in zip(s.tolist(), (s + ln).tolist()):
        pts |= {a, b, (a + b) // 2, a + 1 if b - a > 1 else a}
        if rng.random() < 0.5:
            pts.add(b + rng.randrange(1, 64))  # in the gap / padding after the segment
    for t in range(0, n + 1, 2048):
        pts |= {t, max(t - 1, 0), min(t + 1, n)}
    pts |= {rng.randrange(n + 1) for _ in range(20)}
    pts = sorted(p for p in pts if 0 <= p <= n)
    keep = [p for p in pts if rng.random() < 0.6]
    return sorted({0, n, *keep})


def _layout_case(seed):
    rng = random.Random(seed)
    N = rng.choice([1, 2, 3, 4, 8, 64, 96, 128])
    dts = [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16"), ("f32", "f32"), ("f16", "f32")]
    params = []
    for j in range(rng.randint(1, 12)):
        pd, gd = rng.choice(dts[: rng.randint(1, 5)])
        numel = rng.randint(1, 3000) if rng.random() < 0.8 else rng.randint(3000, 60_000)
        params.append(ParamSpec(f"p{j}", numel, pd, gd, int(rng.random() < 0.15), rng.randint(0, 2)))
    return rng, params, N, rng.randrange(N), rng.choice([0, 500, 5000, 40_000]), int(rng.random() < 0.2)


@pytest.mark.parametrize("seed", range(30))
def test_range_stats_against_enumerated_ownership_and_splits(seed):
    rng, params, N, r, bucket, busbw = _layout_case(seed)
    L = oracle.Layout(params, N, r, bucket, busbw)
    inv = rng.choice([1.0, 2.0 ** -16, 0.5])
    grads = []
    for k in range(L.num_buffers):
        dt = DT_NAME[L.buffer(k)["grad_dtype"]]
        n = _arena_n(L, k)
        owned = _owned_arena_slots(L, params, k, r, N)
        assert owned.size == L.buffer(k)["shard_numel"]
        g = _fill(rng, dt, n, owned, plant_inf_owned=(seed % 5 == 0 and k == 0))
        grads.append(g)
        ref_sq, ref_z, ref_inf, cnt = _reference(_as_f32(g, dt), owned, inv)
        # the whole arena (and a range running past it: clamped to the window)
        for lo, hi in [(0, n), (0, n + 4096)]:
            sq, z, fi = _range_stats(L, k, g, inv, lo, hi)
            assert (z, fi) == (ref_z, ref_inf), (seed, k, lo, hi)
            if not ref_inf:
                assert abs(sq - ref_sq) <= max(cnt, 1) * U * ref_sq, (seed, k, sq, ref_sq)
        # disjoint ranges cut anywhere, added in range order
        cuts = _cuts(rng, L, k, n)
        psq, pz, pfi = 0.0, 0, 0
        for lo, hi in zip(cuts[:-1], cuts[1:]):
            sq, z, fi = _range_stats(L, k, g, inv, lo, hi)
            sel = owned[(owned >= lo) & (owned < hi)]
            rsq, rz, rfi, rc = _reference(_as_f32(g, dt), sel, inv)
            assert (z, fi) == (rz, rfi), (seed, k, lo, hi)
            if not rfi:
                assert abs(sq - rsq) <= max(rc, 1) * U * rsq, (seed, k, lo, hi)
            psq, pz, pfi = psq + sq, pz + z, pfi | fi
        assert (pz, pfi) == (ref_z, ref_inf)
        if not ref_inf:
            assert abs(psq - ref_sq) <= max(cnt, 1) * U * ref_sq
        # empty and reversed ranges add nothing
        assert _range_stats(L, k, g, inv, 5, 5) == (0.0, 0, 0)
        assert _range_stats(L, k, g, inv, 9, 3) == (0.0, 0, 0)
    # the whole-layout pass agrees with the sum of the per-buffer ranges
    run = OracleRun(params, N, r, bucket, busbw, arena_numel=[g.size for g in grads])
    for k, g in enumerate(grads):
        run.bufs[k]["grad"][:] = g
    st = oracle.Stats()
    oracle.lib().or_grad_stats(run.L.handle, run.arrays(), inv, ctypes.byref(st))
    parts = [_range_stats(L, k, g, inv, 0, g.size) for k, g in enumerate(grads)]
    assert st.zeros == sum(p[1] for p in parts) and st.found_inf == max(p[2] for p in parts)
    if not st.found_inf:
        tot = sum(p[0] for p in parts)
        n_el = sum(L.buffer(k)["shard_numel"] for k in range(L.num_buffers))
        assert abs(st.sumsq - tot) <= max(n_el, 1) * U * tot


def test_tiny_rank_ranges_by_hand():
    # Rank 1 of the Tiny layout owns arena slots [0, 672) (w0's elements
    # 32..703); grads 1.0 everywhere give sumsq = count and no zeros.
    L = oracle.Layout(tiny(), 4, 1, 0)
    g = np.full(2048, 0x3F80, np.uint16)  # bf16 1.0
    g[672:] = 0x7FC0  # NaN in the arena tail, outside the window
    assert _range_stats(L, 0, g, 1.0, 0, 2048) == (672.0, 0, 0)
    assert _range_stats(L, 0, g, 1.0, 100, 300) == (200.0, 0, 0)
    assert _range_stats(L, 0, g, 1.0, 600, 2048) == (72.0, 0, 0)
    # Rank 0 owns b1 [0,16), w1 [64,576), b0 [576,608), w0 [640,672) of its
    # window; the 64-alignment gaps [16,64) and [608,640) are not shard slots.
    L0 = oracle.Layout(tiny(), 4, 0, 0)
    g0 = np.full(2048, 0x3F80, np.uint16)
    g0[16:64] = 0x7F80  # +inf in a gap
    g0[608:640] = 0x7FC0  # NaN in a gap
    g0[672:] = 0x7F80
    assert _range_stats(L0, 0, g0, 1.0, 0, 2048) == (592.0, 0, 0)
    assert _range_stats(L0, 0, g0, 1.0, 10, 70) == (12.0, 0, 0)  # 6 of b1, 6 of w1
    assert _range_stats(L0, 0, g0, 1.0, 600, 650) == (18.0, 0, 0)  # 8 of b0, 10 of w0
    g0[700] = 0x0000
    g0[5] = 0x8000  # -0 counts as a zero
    assert _range_stats(L0, 0, g0, 1.0, 0, 2048) == (591.0, 1, 0)
    g0[3] = 0xFF80  # -inf in a shard slot
    assert _range_stats(L0, 0, g0, 1.0, 0, 2048)[2] == 1
    assert _range_stats(L0, 0, g0, 1.0, 4, 2048)[2] == 0
