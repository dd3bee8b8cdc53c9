"""Closed-form pins for the oracle's step: unscale, inf/NaN, norm, clip,
zero count, loss scaling, step skipping and AdamW.

The step order (grads to fp32 main grads + unscale + inf/NaN check, then
clip by global norm, then the inner Adam step and the master-to-model copy)
is "Megatron-LM distrib_optimizer.py 源码精读", section 三层继承体系 (second
layer); the same order appears in the DeepSpeed stage-2 step of "Megatron-LM与
DeepSpeed的分布式训练源码里…" §2.  The Adam/AdamW update itself is only named on
the pages; the checks below use facts of that published algorithm (Kingma &
Ba; Loshchilov & Hutter) that hold whatever the fp32 operation order:
first-step update = lr * g / (|g| + eps), constant-gradient moments are
geometric series, lr = 0 freezes the weight, zero grads only decay it.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.models import ParamSpec, tiny
from tests.oracle_harness import OracleRun, as_f32, to_bits

LR, B1, B2, EPS, WD = 1e-3, 0.9, 0.999, 1e-8, 0.01
HP = [(LR, B1, B2, EPS, WD)]


def _single(n, pd="bf16", gd="bf16", N=1, r=0):
    run = OracleRun([ParamSpec("w", n, pd, gd)], N, r, 0)
    return run


def _set_params_normal(run, k, sigma=0.02, seed=0):
    b = run.bufs[k]
    t = synth.fill_normal(b["pd"], b["n"], seed, synth.STREAM_WEIGHT, 0, sigma)
    b["param"][:] = to_bits(t)


def _set_grads(run, k, x_f32: np.ndarray):
    b = run.bufs[k]
    x = np.zeros(b["n"], np.float32)
    x[:len(x_f32)] = x_f32  # arena slots past the params stay zero
    t = torch.from_numpy(x).to(synth.torch_dtype(b["gd"]))
    b["grad"][:] = to_bits(t)


def _ulp(x):
    return np.spacing(np.abs(x).astype(np.float32)).astype(np.float64)


def test_first_step_closed_form():
    n = 4096
    run = _single(n)
    _set_params_normal(run, 0)
    rng = np.random.default_rng(0)
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 0, n)).astype(np.float32)
    _set_grads(run, 0, g)
    run.init_state()
    p0 = as_f32(run.bufs[0]["param"], "bf16").astype(np.float64)
    graw = as_f32(run.bufs[0]["grad"], "bf16").astype(np.float64)
    st = run.step(HP, 0.0)
    assert st.skipped == 0 and st.t == 1
    p1 = run.bufs[0]["master"].astype(np.float64)
    # m1 = (1-b1) g, v1 = (1-b2) g^2 -> m_hat = g, sqrt(v_hat) = |g|
    want = p0 * (1 - LR * WD) - LR * graw / (np.abs(graw) + EPS)
    tol = 6 * _ulp(p1) + 8 * np.spacing(np.float32(LR))
    assert np.all(np.abs(p1 - want) <= tol)
    # hence lr * sign(g) up to eps/|g|
    assert np.all(np.abs((p0 * (1 - LR * WD) - p1) - LR * np.sign(graw)) <= LR * EPS / np.abs(graw) + tol)
    m = run.bufs[0]["m"].astype(np.float64)
    v = run.bufs[0]["v"].astype(np.float64)
    assert np.allclose(m, (1 - B1) * graw, rtol=2e-7, atol=0)
    assert np.allclose(v, (1 - B2) * graw * graw, rtol=4e-7, atol=0)
    # written-back param is the RNE bf16 of the master
    assert np.array_equal(run.bufs[0]["param"], to_bits(torch.from_numpy(run.bufs[0]["master"]).to(torch.bfloat16)))


def test_decay_multiplies_the_weight_before_the_adam_term():
    """Decoupled weight decay scales the pre-step weight: p1 = p0 (1 - lr wd)
    - lr g / (|g| + eps).  With lr = 0.1 and wd = 0.5 the other placement,
    (p0 - lr g / (|g| + eps)) (1 - lr wd), differs by lr^2 wd ~ 5e-3 per
    element, far above rounding."""
    n = 2048
    lr, wd = 0.1, 0.5
    run = _single(n, "f32", "f32")
    rng = np.random.default_rng(3)
    run.bufs[0]["param"][:] = rng.standard_normal(n).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    g[g == 0] = 1e-3
    _set_grads(run, 0, g)
    run.init_state()
    p0 = run.bufs[0]["param"].astype(np.float64).copy()
    run.step([(lr, B1, B2, EPS, wd)], 0.0)
    p1 = run.bufs[0]["param"].astype(np.float64)
    gd = g.astype(np.float64)
    u = gd / (np.abs(gd) + EPS)
    want = p0 * (1 - lr * wd) - lr * u
    other = (p0 - lr * u) * (1 - lr * wd)
    # fp32 rounding of each term (the weight, the decayed weight, the Adam term)
    tol = 4 * (_ulp(p0) + _ulp(lr * u) + _ulp(p1))
    assert np.all(np.abs(p1 - want) <= tol)
    assert np.all(np.abs(p1 - other) > 100 * tol)


def test_constant_gradient_geometric_series():
    n, T = 512, 25
    run = _single(n, "f32", "f32")
    rng = np.random.default_rng(1)
    run.bufs[0]["param"][:] = rng.standard_normal(n).astype(np.float32) * 0.02
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    _set_grads(run, 0, g)
    run.init_state()
    p_prev = run.bufs[0]["param"].astype(np.float64).copy()
    gd = g.astype(np.float64)
    for t in range(1, T + 1):
        run.step(HP, 0.0)
        m = run.bufs[0]["m"].astype(np.float64)
        v = run.bufs[0]["v"].astype(np.float64)
        assert np.allclose(m, (1 - B1 ** t) * gd, rtol=2e-7 * t + 1e-7, atol=0)
        assert np.allclose(v, (1 - B2 ** t) * gd * gd, rtol=2e-7 * t + 1e-7, atol=0)
        p = run.bufs[0]["param"].astype(np.float64)
        # bias-corrected moments are g and |g|: the same update every step
        upd = p_prev * (1 - LR * WD) - p
        assert np.allclose(upd, LR * gd / (np.abs(gd) + EPS), rtol=5e-6 * t, atol=6 * _ulp(p).max())
        p_prev = p.copy()
    assert run.t == T


def test_lr_zero_and_zero_grad_and_beta1_zero():
    n = 1024
    run = _single(n, "f32", "f32")
    run.bufs[0]["param"][:] = np.linspace(-1, 1, n, dtype=np.float32)
    g = np.linspace(-1e-3, 1e-3, n, dtype=np.float32)
    g[::7] = 0.0
    _set_grads(run, 0, g)
    run.init_state()
    p0 = run.bufs[0]["param"].copy()
    run.step([(0.0, B1, B2, EPS, WD)], 0.0)  # lr = 0: weight frozen, moments still move
    assert np.array_equal(run.bufs[0]["param"], p0)
    assert np.array_equal(run.bufs[0]["m"] != 0, g != 0)
    # zero grad elements: moments stay 0, the weight only decays
    run2 = _single(n, "f32", "f32")
    run2.bufs[0]["param"][:] = p0
    _set_grads(run2, 0, g)
    run2.init_state()
    run2.step(HP, 0.0)
    z = g == 0
    assert np.all(run2.bufs[0]["m"][z] == 0) and np.all(run2.bufs[0]["v"][z] == 0)
    assert np.array_equal(run2.bufs[0]["param"][z], p0[z] * np.float32(1 - LR * WD))
    # beta1 = 0: m is the (unscaled, unclipped) grad itself
    run3 = _single(n, "f32", "f32")
    run3.bufs[0]["param"][:] = p0
    _set_grads(run3, 0, g)
    run3.init_state()
    run3.step([(LR, 0.0, B2, EPS, WD)], 0.0)
    assert np.array_equal(run3.bufs[0]["m"], g)


def test_unscale_is_exact_for_power_of_two_scale():
    n = 2048
    run = _single(n, "f16", "f16")
    _set_params_normal(run, 0)
    x = (np.random.default_rng(2).standard_normal(n) * 1e-3).astype(np.float32)
    S = 2.0 ** 16
    _set_grads(run, 0, x * np.float32(S))
    run.init_state()
    run.scaler = oracle.make_scaler(True, S)
    run.step([(LR, 0.0, B2, EPS, WD)], 0.0)
    raw = as_f32(run.bufs[0]["grad"], "f16")
    assert np.array_equal(run.bufs[0]["m"], raw * np.float32(1 / S))
    assert np.array_equal(run.bufs[0]["m"] * np.float32(S), raw)


def test_norm_closed_form_and_textbook():
    # constant grads a over k^2 elements: norm = |a| * k exactly
    k = 64
    run = _single(k * k, "bf16", "bf16")
    _set_grads(run, 0, np.full(k * k, -0.5, np.float32))
    run.init_state()
    st = run.step(HP, 0.0)
    assert st.norm == 0.5 * k and st.sumsq == 0.25 * k * k
    # random grads: the library two-norm on the same fp32 values
    run = OracleRun(tiny(), 4, 0, 0)
    x = synth.normal_f32(0, synth.STREAM_GRAD, 1, 0, run.bufs[0]["n"], 1e-2)
    _set_grads(run, 0, x)
    run.init_state()
    st = run.step(HP, 1.0)
    mask = run.valid(0)
    gv = as_f32(run.bufs[0]["grad"], "bf16")[mask].astype(np.float64)
    assert math.isclose(st.norm, float(np.linalg.norm(gv)), rel_tol=1e-13)
    assert st.zeros == int(np.count_nonzero(gv == 0))


def test_clip_closed_form():
    n = 3072
    run = _single(n, "bf16", "bf16")
    _set_params_normal(run, 0)
    x = (np.random.default_rng(3).standard_normal(n) * 0.1).astype(np.float32)  # norm ~ 5.5 > 1
    _set_grads(run, 0, x)
    run.init_state()
    st = run.step([(LR, 0.0, B2, EPS, WD)], 1.0)  # beta1 = 0 exposes the clipped grad as m
    assert st.clip_applied == 1
    assert st.clip_coef == 1.0 / (st.norm + 1e-6)
    post = float(np.linalg.norm(run.bufs[0]["m"].astype(np.float64)))
    assert math.isclose(post, st.norm / (st.norm + 1e-6), rel_tol=1e-6)
    # a norm below max_norm is not clipped
    run2 = _single(n, "bf16", "bf16")
    _set_grads(run2, 0, x * np.float32(1e-3))
    run2.init_state()
    st2 = run2.step(HP, 1.0)
    assert st2.clip_applied == 0 and st2.clip_coef > 1.0


def test_skip_on_overflow_is_bit_identical_and_scale_backs_off():
    run = OracleRun(tiny(), 4, 0, 0)
    _set_params_normal(run, 0)
    run.init_state()
    run.scaler = oracle.make_scaler(True, 2.0 ** 16)
    x = synth.normal_f32(0, synth.STREAM_GRAD, 1, 0, run.bufs[0]["n"], 1e-2)
    _set_grads(run, 0, x)
    run.step(HP, 1.0)
    snap = {key: run.bufs[0][key].copy() for key in ("param", "master", "m", "v")}
    for bad in (np.inf, -np.inf, np.nan):
        y = x.copy()
        s, ln, _ = run.L.segments(0)
        y[s[-1] + ln[-1] - 1] = bad
        _set_grads(run, 0, y)
        scale_before = run.scaler.scale
        st = run.step(HP, 1.0)
        assert st.found_inf == 1 and st.skipped == 1 and st.t == 1 and run.t == 1
        assert st.scale_used == scale_before and st.scale_next == scale_before / 2
        for key, val in snap.items():
            assert np.array_equal(run.bufs[0][key], val, equal_nan=False)
    assert run.scaler.scale == 2.0 ** 13  # three backoffs: 2^(16-3)


def test_scaler_growth_and_floor():
    run = _single(256, "f16", "f16")
    run.init_state()
    run.scaler = oracle.make_scaler(True, 4.0, growth_interval=3, hysteresis=2, min_scale=1.0)
    _set_grads(run, 0, np.full(256, 1e-3, np.float32))
    for _ in range(6):
        run.step(HP, 0.0)
    assert run.scaler.scale == 16.0 and run.t == 6  # grew twice
    _set_grads(run, 0, np.full(256, np.inf, np.float32))
    scales = [run.step(HP, 0.0).scale_next for _ in range(6)]
    # hysteresis 2: the first overflow only uses up the hysteresis count
    assert scales == [16.0, 8.0, 4.0, 2.0, 1.0, 1.0]
    assert run.t == 6


def test_zero_count_matches_mask():
    n = 100_000
    run = _single(n, "bf16", "bf16")
    x = synth.normal_f32(7, synth.STREAM_GRAD, 1, 0, n, 1e-3, zero_frac=0.01)
    _set_grads(run, 0, x)
    run.init_state()
    st = run.step(HP, 1.0)
    raw = as_f32(run.bufs[0]["grad"], "bf16")[:n]
    assert st.zeros == int(np.count_nonzero(raw == 0))
    assert 800 < st.zeros < 1200


def test_sumsq_over_ranks_equals_whole_buffer():
    # values keyed by buffer element index, so every rank sees the same buffer
    params = tiny()
    L0 = oracle.Layout(params, 4, 0, 0)
    numel = L0.buffer(0)["numel"]
    full = synth.normal_f32(0, synth.STREAM_GRAD, 1, 0, numel, 1e-2)
    full_bits = to_bits(torch.from_numpy(full).to(torch.bfloat16))
    owned = np.zeros(numel, bool)
    for i in range(len(params)):
        p = L0.param(i)
        owned[p["start"]:p["end"]] = True
    whole = float(np.sum(as_f32(full_bits, "bf16")[owned].astype(np.float64) ** 2))
    tot, zeros = 0.0, 0
    for r in range(4):
        run = OracleRun(params, 4, r, 0)
        b = run.L.bucket(0, 0)
        run.bufs[0]["grad"][:] = full_bits[b["window_start"]:b["window_start"] + b["shard"]]
        run.init_state()
        st = run.step(HP, 1.0)
        tot += st.sumsq
        zeros += st.zeros
    assert math.isclose(tot, whole, rel_tol=1e-13)
    assert zeros == int(np.count_nonzero(as_f32(full_bits, "bf16")[owned] == 0))


def test_dp1_equals_plain_elementwise_update():
    # N = 1: every param is wholly on the one rank, so the layout-driven step
    # must equal the element-wise update applied param by param
    params = [ParamSpec("a", 700, "bf16", "bf16", 0, 0), ParamSpec("b", 130, "bf16", "bf16", 0, 1)]
    hps = [HP[0], (2e-3, 0.8, 0.99, 1e-6, 0.1)]
    run = OracleRun(params, 1, 0, 0)
    _set_params_normal(run, 0)
    x = synth.normal_f32(0, synth.STREAM_GRAD, 1, 0, run.bufs[0]["n"], 1e-2)
    _set_grads(run, 0, x)
    run.init_state()
    before = {key: run.bufs[0][key].copy() for key in ("param", "master", "m", "v", "grad")}
    st = oracle.Stats()
    t = ctypes.c_int64(0)
    sc = oracle.make_scaler(False, 1.0)
    lib = oracle.lib()
    arr = run.arrays()
    lib.or_grad_stats(run.L.handle, arr, 1.0, ctypes.byref(st))
    s = oracle.Scalars()
    lib.or_decide(ctypes.byref(st), ctypes.byref(sc), ctypes.byref(t), oracle.make_hparams(hps), 2, 1.0,
                  ctypes.byref(s))
    run.step(hps, 1.0)
    for i in range(2):
        p = run.L.param(i)
        a, e = p["arena_offset"], p["arena_offset"] + (p["param"][1] - p["param"][0])
        mas, m, v = (before[k][a:e].copy() for k in ("master", "m", "v"))
        out = np.zeros(e - a, np.uint16)
        hg = np.full(e - a, i, np.int32)
        g = before["grad"][a:e].copy()
        lib.or_apply_elems(1, 1, e - a, hg.ctypes.data, g.ctypes.data, mas.ctypes.data, m.ctypes.data,
                           v.ctypes.data, out.ctypes.data, ctypes.byref(s))
        assert np.array_equal(mas, run.bufs[0]["master"][a:e])
        assert np.array_equal(m, run.bufs[0]["m"][a:e]) and np.array_equal(v, run.bufs[0]["v"][a:e])
        assert np.array_equal(out, run.bufs[0]["param"][a:e])


def test_hyper_groups_use_their_own_lr():
    params = [ParamSpec("a", 640, "f32", "f32", 0, 0), ParamSpec("b", 640, "f32", "f32", 0, 1)]
    hps = [(1e-3, B1, B2, EPS, 0.0), (1e-2, B1, B2, EPS, 0.0)]
    run = OracleRun(params, 1, 0, 0)
    run.bufs[0]["param"][:] = 0.5
    _set_grads(run, 0, np.full(run.bufs[0]["n"], 1e-2, np.float32))
    run.init_state()
    run.step(hps, 0.0)
    for i, lr in enumerate((1e-3, 1e-2)):
        p = run.L.param(i)
        a = p["arena_offset"]
        upd = 0.5 - run.bufs[0]["param"][a:a + 640].astype(np.float64)
        assert np.allclose(upd, lr, rtol=1e-5)


@pytest.mark.parametrize("max_norm", [0.0, 0.05])
def test_steps_track_fp64_adamw(max_norm):
    """Six steps of the oracle on generic inputs (fresh normal grads each
    step, two hyper-groups, weight decay, clipping off or active on every
    step) against the textbook AdamW recurrences evaluated in fp64 from the
    same fp32 start and the same fp32 grads: m, v, m_hat = m / (1 - b1^t),
    v_hat = v / (1 - b2^t), p <- p (1 - lr wd) - lr m_hat / (sqrt(v_hat) + eps),
    after clipping g by max_norm / (norm + 1e-6) when that is below 1.  The
    fp32 oracle may differ only by its roundings: a few ulps of p per step,
    and 1e-6 of the size of the terms in m and v."""
    params = [ParamSpec("a", 3000, "bf16", "bf16", 0, 0), ParamSpec("b", 1500, "bf16", "bf16", 0, 1)]
    hps = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (3e-3, 0.8, 0.99, 1e-6, 0.1)]
    run = OracleRun(params, 1, 0, 0)
    _set_params_normal(run, 0)
    run.init_state()
    b = run.bufs[0]
    ok = run.valid(0)
    hg = np.zeros(b["n"], np.int64)
    for i in range(2):
        p = run.L.param(i)
        hg[p["arena_offset"]:p["arena_offset"] + (p["param"][1] - p["param"][0])] = i
    lr, b1, b2, eps, wd = (np.array([h[j] for h in hps])[hg] for j in range(5))
    p64 = b["master"].astype(np.float64)
    m64 = np.zeros(b["n"])
    v64 = np.zeros(b["n"])
    sm = np.zeros(b["n"])  # running size of the terms summed into m
    for t in range(1, 7):
        x = synth.normal_f32(0, synth.STREAM_GRAD, t, 0, b["n"], 1e-3)
        t16 = torch.from_numpy(x).to(torch.bfloat16)
        b["grad"][:] = to_bits(t16)
        g = t16.float().numpy().astype(np.float64)
        g[~ok] = 0.0
        norm = math.sqrt(float(np.sum(g * g)))
        if max_norm > 0 and max_norm / (norm + 1e-6) < 1.0:
            g = g * (max_norm / (norm + 1e-6))
        stats = run.step(hps, max_norm)
        assert stats.found_inf == 0
        assert abs(stats.norm - norm) <= 1e-12 * norm
        p64 = p64 * (1.0 - lr * wd)
        m64 = b1 * m64 + (1.0 - b1) * g
        v64 = b2 * v64 + (1.0 - b2) * g * g
        sm = b1 * sm + (1.0 - b1) * np.abs(g)
        mhat = m64 / (1.0 - b1 ** t)
        vhat = v64 / (1.0 - b2 ** t)
        p64 = p64 - lr * mhat / (np.sqrt(vhat) + eps)
        dm = np.abs(b["m"].astype(np.float64) - m64)[ok]
        dv = np.abs(b["v"].astype(np.float64) - v64)[ok]
        dp = np.abs(b["master"].astype(np.float64) - p64)[ok]
        assert np.all(dm <= 1e-6 * sm[ok]), f"step {t}: m off by {np.max(dm / sm[ok]):.3g} of its terms"
        assert np.all(dv <= 1e-6 * v64[ok]), f"step {t}: v off by {np.max(dv / v64[ok]):.3g}"
        tol_p = t * (4 * _ulp(p64[ok]) + lr[ok] * 1e-5)
        assert np.all(dp <= tol_p), f"step {t}: master off by {np.max(dp / tol_p):.3g} of the bound"
