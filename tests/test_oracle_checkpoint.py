"""Pins of the oracle's model-space optimizer-state checkpoint.

[DO] "三层继承体系" (third layer) lists fully reshardable checkpoint formats,
formats that do not depend on the optimizer's buffer structure.  What fixes
the oracle's export / import here:
  * coverage: over all ranks of any layout, the exported shards tile every
    element of every param exactly once;
  * placement: importing model-space values puts each value at the arena slot
    the (separately pinned) layout gives it, and the 16-bit param becomes the
    value rounded to nearest even (checked against PyTorch's cast);
  * round trip: export(import(x)) == x bit for bit;
  * reshard continuation: a job that runs k steps on N=8 ranks, is saved,
    reloaded on N=4 ranks with another bucket size and runs k more steps ends
    bit-identical to one rank running 2k steps (clipping off, so no
    cross-rank rounding enters), and it does not when the step count is
    dropped on reload.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.models import ParamSpec
from tests.oracle_harness import (OracleRanks, OracleRun, export_to_model, model_to_export,
                                  oracle_export, oracle_import, shard_pieces, to_bits)

PARAMS = [ParamSpec("emb", 20000, "bf16", "f32", 1, 0), ParamSpec("w1", 7001, "bf16", "bf16", 0, 0),
          ParamSpec("n1", 256, "f32", "f32", 0, 1), ParamSpec("h1", 3333, "f16", "f16", 0, 0),
          ParamSpec("w2", 12345, "bf16", "bf16", 0, 1), ParamSpec("n2", 100, "f32", "f32", 0, 0),
          ParamSpec("w3", 999, "bf16", "f32", 0, 0)]
HPS = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (3e-4, 0.8, 0.99, 1e-6, 0.0)]


def model_values(seed=1):
    rng = np.random.default_rng(seed)
    return {key: [rng.standard_normal(p.numel).astype(np.float32) * s for p in PARAMS]
            for key, s in (("master", 0.05), ("m", 1e-3), ("v", 1e-6))}


def weights():
    return [synth.fill_normal(p.param_dtype, p.numel, 7, synth.weight_stream(i), 0, 0.02)
            for i, p in enumerate(PARAMS)]


def grads(step, sigma=1e-2, inf_at=None):
    out = [synth.fill_normal(p.grad_dtype, p.numel, 7, synth.grad_stream(i), step, sigma)
           for i, p in enumerate(PARAMS)]
    if inf_at is not None:
        p, i = inf_at
        out[p][i] = math.inf
    return out


@pytest.mark.parametrize("dp,bucket", [(1, 0), (3, 9000), (8, 4000), (8, 0)])
def test_exports_tile_the_model_once(dp, bucket):
    count = [np.zeros(p.numel, np.int64) for p in PARAMS]
    total = 0
    for r in range(dp):
        L = oracle.Layout(PARAMS, dp, r, bucket)
        for p, _, _, lo, hi, _ in shard_pieces(L, len(PARAMS)):
            count[p][lo:hi] += 1
        total += sum(L.buffer(k)["shard_numel"] for k in range(L.num_buffers))
    assert all(np.all(c == 1) for c in count)
    assert total == sum(p.numel for p in PARAMS)


@pytest.mark.parametrize("dp,rank,bucket", [(1, 0, 0), (3, 2, 9000), (8, 5, 4000)])
def test_import_places_values_and_rounds_params(dp, rank, bucket):
    full = model_values()
    run = OracleRun(PARAMS, dp, rank, bucket)
    ex = model_to_export(run.L, len(PARAMS), full)
    oracle_import(run, ex)
    for p, k, a, lo, hi, _ in shard_pieces(run.L, len(PARAMS)):
        b = run.bufs[k]
        want = full["master"][p][lo:hi]
        if b["pd"] == "f32":
            assert np.array_equal(b["param"][a:a + hi - lo].view(np.uint32), want.view(np.uint32))
        else:
            assert np.array_equal(b["master"][a:a + hi - lo].view(np.uint32), want.view(np.uint32))
            ref = to_bits(torch.from_numpy(want).to(synth.torch_dtype(b["pd"])))
            assert np.array_equal(b["param"][a:a + hi - lo], ref)
        assert np.array_equal(b["m"][a:a + hi - lo], full["m"][p][lo:hi])
        assert np.array_equal(b["v"][a:a + hi - lo], full["v"][p][lo:hi])
    back = oracle_export(run)
    for e, x in zip(back, ex):
        assert np.array_equal(e.view(np.uint32), x.view(np.uint32))
    # and the assembled model space holds exactly the rank's pieces
    got = {key: [np.full(p.numel, np.nan, np.float32) for p in PARAMS] for key in full}
    export_to_model(run.L, len(PARAMS), back, got)
    for p, _, _, lo, hi, _ in shard_pieces(run.L, len(PARAMS)):
        for key in full:
            assert np.array_equal(got[key][p][lo:hi], full[key][p][lo:hi])


def _model_equal(a, b):
    for key in a:
        for x, y in zip(a[key], b[key]):
            if not np.array_equal(x.view(np.uint32), y.view(np.uint32)):
                return False
    return True


def _params_equal(a, b):
    return all(np.array_equal(x, y) for x, y in zip(a, b))


def _run_resharded(k, n1, b1, n2, b2, scaler=(False, 1.0), inf_at=None, max_norm=0.0, keep_t=True):
    A = OracleRanks(PARAMS, n1, b1)
    A.init(weights(), scaler)
    for s in range(1, k + 1):
        A.step(grads(s, inf_at=inf_at if s == 2 else None), HPS, max_norm)
    state, sc = A.model_state(), A.scalars()
    for key in state:
        assert not any(np.isnan(x).any() for x in state[key]), "export left a model element unset"
    B = OracleRanks(PARAMS, n2, b2)
    zero_w = [torch.zeros(p.numel, dtype=synth.torch_dtype(p.param_dtype)) for p in PARAMS]
    B.init(zero_w, scaler)  # everything the continuation reads must come from the checkpoint
    if not keep_t:
        sc = dict(sc, t=0)
    B.load(state, sc)
    for s in range(k + 1, 2 * k + 1):
        B.step(grads(s), HPS, max_norm)
    return B


def test_reshard_continuation_matches_single_rank():
    k = 3
    one = OracleRanks(PARAMS, 1, 0)
    one.init(weights())
    for s in range(1, 2 * k + 1):
        one.step(grads(s), HPS, 0.0)
    B = _run_resharded(k, 8, 4000, 4, 15000)
    assert _model_equal(B.model_state(), one.model_state())
    assert _params_equal(B.model_params(), one.model_params())
    assert B.scalars() == one.scalars()
    # dropping the step count on reload changes Adam's bias correction
    bad = _run_resharded(k, 8, 4000, 4, 15000, keep_t=False)
    assert not _model_equal(bad.model_state(), one.model_state())


def test_reshard_carries_loss_scale_state_over_a_skipped_step():
    k = 3
    sc = (True, 1024.0)
    inf_at = (4, 777)  # w2 element 777, overflow at step 2
    one = OracleRanks(PARAMS, 1, 0)
    one.init(weights(), sc)
    for s in range(1, 2 * k + 1):
        one.step(grads(s, inf_at=inf_at if s == 2 else None), HPS, 0.0)
    assert one.scalars()["t"] == 2 * k - 1 and one.scalars()["scale"] == 512.0
    B = _run_resharded(k, 8, 4000, 2, 0, scaler=sc, inf_at=inf_at)
    assert _model_equal(B.model_state(), one.model_state())
    assert _params_equal(B.model_params(), one.model_params())
    assert B.scalars() == one.scalars()


def test_multi_rank_seam_on_one_rank_is_the_plain_step():
    """OracleRanks at N=1 is or_step: the seam adds nothing on one rank."""
    ranks = OracleRanks(PARAMS, 1, 5000)
    ranks.init(weights())
    plain = OracleRun(PARAMS, 1, 0, 5000)
    for p, k, a, lo, hi, _ in shard_pieces(plain.L, len(PARAMS)):
        plain.bufs[k]["param"][a:a + hi - lo] = to_bits(weights()[p])[lo:hi]
    plain.init_state()
    for s in (1, 2):
        g = grads(s)
        st = ranks.step(g, HPS, 1.0)
        for p, k, a, lo, hi, _ in shard_pieces(plain.L, len(PARAMS)):
            plain.bufs[k]["grad"][a:a + hi - lo] = to_bits(g[p])[lo:hi]
        ref = plain.step(HPS, 1.0)
        assert st.sumsq == ref.sumsq and st.clip_applied == ref.clip_applied == 1
    for x, y in zip(ranks.runs[0].bufs, plain.bufs):
        for key in ("param", "m", "v"):
            assert np.array_equal(x[key].view(np.uint8), y[key].view(np.uint8))
