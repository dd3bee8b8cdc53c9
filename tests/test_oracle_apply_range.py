"""Pin for the oracle's update restricted to a range of arena slots
(or_apply_range), which the full-size parity runs split over host threads.

The update of "Megatron-LM distrib_optimizer.py 源码精读" section "三层继承体系"
(second layer: the inner AdamW step on the shard groups and the copy of the
masters back to the 16-bit params) acts on each shard element on its own,
given the step's scalars.  So the union of the range updates over any split
of the arena into disjoint ranges, run in any order, must equal the
whole-window update (or_apply, itself pinned by the closed forms of
test_oracle_adamw.py) bit for bit, and slots that hold no shard element must
stay untouched.
"""
import ctypes
import random

import numpy as np
import pytest

import oracle
from tests.oracle_harness import OracleRun
from tests.test_oracle_stats_range import _cuts, _layout_case


def _state(run, rng):
    nr = np.random.default_rng(rng.randrange(1 << 30))
    for b in run.bufs:
        n = b["n"]
        g = (nr.standard_normal(n) * 1e-2).astype(np.float32)
        w = (nr.standard_normal(n) * 2e-2).astype(np.float32)
        if b["gd"] == "f32":
            b["grad"][:] = g
        else:
            f = oracle.lib().or_f32_to_bf16_n if b["gd"] == "bf16" else oracle.lib().or_f32_to_f16_n
            f(g.ctypes.data, b["grad"].ctypes.data, n)
        if b["pd"] == "f32":
            b["param"][:] = w
        else:
            f = oracle.lib().or_f32_to_bf16_n if b["pd"] == "bf16" else oracle.lib().or_f32_to_f16_n
            f(w.ctypes.data, b["param"].ctypes.data, n)
            b["master"][:] = w
        b["m"][:] = (nr.standard_normal(n) * 1e-3).astype(np.float32)
        b["v"][:] = (nr.random(n) * 1e-6).astype(np.float32)


def _copy(run):
    return [{k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in b.items()} for b in run.bufs]


@pytest.mark.parametrize("seed", range(20))
def test_range_updates_equal_the_whole_window_update(seed):
    rng, params, N, r, bucket, busbw = _layout_case(seed)
    base = OracleRun(params, N, r, bucket, busbw)
    arena = [-(-max(base.L.buffer(k)["window_numel"], 1) // 2048) * 2048 for k in range(base.nb)]
    a = OracleRun(params, N, r, bucket, busbw, arena_numel=arena)
    _state(a, rng)
    b = OracleRun(params, N, r, bucket, busbw, arena_numel=arena)
    b.bufs = _copy(a)
    st = oracle.Stats()
    oracle.lib().or_grad_stats(a.L.handle, a.arrays(), 1.0, ctypes.byref(st))
    sc = oracle.Scalars()
    t = ctypes.c_int64(seed % 4)
    hps = oracle.make_hparams([(1e-3, 0.9, 0.999, 1e-8, 0.01), (3e-4, 0.8, 0.99, 1e-6, 0.0),
                               (2e-3, 0.95, 0.9999, 1e-8, 0.1)])
    scaler = oracle.make_scaler(False, 1.0)
    assert oracle.lib().or_decide(ctypes.byref(st), ctypes.byref(scaler), ctypes.byref(t), hps, 3, 0.5,
                                  ctypes.byref(sc)) == 0
    before = _copy(a)
    oracle.lib().or_apply(a.L.handle, a.arrays(), ctypes.byref(sc))
    arr_b = b.arrays()
    for k in range(b.nb):
        ranges = list(zip(*(lambda c: (c[:-1], c[1:]))(_cuts(rng, b.L, k, b.bufs[k]["n"]))))
        rng.shuffle(ranges)
        for lo, hi in ranges:
            oracle.lib().or_apply_range(b.L.handle, k, arr_b, ctypes.byref(sc), lo, hi)
    changed = False
    for k in range(a.nb):
        for key in ("param", "master", "m", "v"):
            x, y = a.bufs[k][key], b.bufs[k][key]
            if x is None:
                continue
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (seed, k, key)
            changed |= not np.array_equal(x.view(np.uint8), before[k][key].view(np.uint8))
        mask = a.L.valid_mask(k, a.bufs[k]["n"])
        for key in ("param", "m", "v"):
            assert np.array_equal(b.bufs[k][key][~mask].view(np.uint8), before[k][key][~mask].view(np.uint8))
    assert changed or all(a.L.buffer(k)["shard_numel"] == 0 for k in range(a.nb))
    # a skipped step changes nothing, whatever the range
    sc.skip = 1
    snap = _copy(b)
    oracle.lib().or_apply_range(b.L.handle, 0, arr_b, ctypes.byref(sc), 0, b.bufs[0]["n"])
    for k in range(b.nb):
        for key in ("param", "master", "m", "v"):
            if snap[k][key] is not None:
                assert np.array_equal(snap[k][key].view(np.uint8), b.bufs[k][key].view(np.uint8))
