"""GPU parity of the model-space optimizer-state checkpoint.

* export / import against the oracle's export / import of the same arenas,
  bit for bit (both are copies, plus round-to-nearest-even of the 16-bit
  params on import), including the slots no param owns;
* scalar state read / write, and the written loss scale taking effect;
* a job run on the device at N=8 through the cross-rank seam, saved,
  reloaded at N=4 with another bucket size, saved again and reloaded at N=3,
  against one oracle rank running all steps, within the step's tolerances,
  with clipping active, and once with an overflow-skipped step whose
  loss-scale state has to survive the reload.
"""
import math

import numpy as np
import pytest
import torch

import synth
from synth.models import ParamSpec
from tests import gpu_harness as H
from tests.oracle_harness import (OracleRanks, OracleRun, model_to_export, oracle_export, oracle_import,
                                  shard_pieces, to_bits)

pytestmark = pytest.mark.gpu

PARAMS = [ParamSpec("emb", 1_000_003, "bf16", "f32", 1, 0), ParamSpec("w1", 700_001, "bf16", "bf16", 0, 0),
          ParamSpec("n1", 4096, "f32", "f32", 0, 1), ParamSpec("h1", 333_333, "f16", "f16", 0, 0),
          ParamSpec("w2", 1_234_567, "bf16", "bf16", 0, 1), ParamSpec("n2", 100, "f32", "f32", 0, 0),
          ParamSpec("w3", 99_999, "bf16", "f32", 0, 0)]
HPS = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (3e-4, 0.8, 0.99, 1e-6, 0.0)]


@pytest.fixture(autouse=True)
def _announce(request):
    H.log(f"[gpu-test] start {request.node.name}")
    yield
    torch.cuda.synchronize()


def weights():
    return [synth.fill_normal(p.param_dtype, p.numel, 11, synth.weight_stream(i), 0, 0.02)
            for i, p in enumerate(PARAMS)]


def grads(step, inf_at=None):
    out = [synth.fill_normal(p.grad_dtype, p.numel, 11, synth.grad_stream(i), step, 1e-2)
           for i, p in enumerate(PARAMS)]
    if inf_at is not None:
        out[inf_at[0]][inf_at[1]] = math.inf
    return out


def _oracle_view(run: OracleRun, ranks: H.DeviceRanks, r: int):
    """Copy rank r's device arenas into the oracle run's host arrays."""
    A = ranks.arenas[r]
    for k, b in enumerate(run.bufs):
        for key, dkey in (("param", "param"), ("master", "master"), ("m", "exp_avg"), ("v", "exp_avg_sq")):
            if b[key] is not None:
                b[key][:] = to_bits(A.bufs[k][dkey].cpu())


@pytest.mark.parametrize("rank", [0, 5])
def test_export_import_match_oracle(rank):
    ranks = H.DeviceRanks(PARAMS, 8, 400_000)
    ranks.init(weights())
    for s in (1, 2):
        ranks.step(grads(s), HPS, 1.0)
    L, A = ranks.layouts[rank], ranks.arenas[rank]
    arena = [A.info[k]["n"] for k in range(L.num_buffers)]
    run = OracleRun(PARAMS, 8, rank, 400_000, arena_numel=arena)
    _oracle_view(run, ranks, rank)
    n = L.state_numel
    ex = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    ranks.D.dopt_state_export(L, A.bufs, *ex, A.workspace, ranks.stream)
    ref = oracle_export(run)
    for e, x in zip(ex, ref):
        assert np.array_equal(e.cpu().numpy().view(np.uint32), x.view(np.uint32))
    # import fresh model-space values over the trained state
    rng = np.random.default_rng(3)
    full = {key: [(rng.standard_normal(p.numel) * s).astype(np.float32) for p in PARAMS]
            for key, s in (("master", 0.05), ("m", 1e-3), ("v", 1e-6))}
    new = model_to_export(L, len(PARAMS), full)
    ranks.D.dopt_state_import(L, A.bufs, *[torch.from_numpy(e).cuda() for e in new], A.workspace, ranks.stream)
    oracle_import(run, new)
    for k, b in enumerate(run.bufs):
        for key, dkey in (("param", "param"), ("master", "master"), ("m", "exp_avg"), ("v", "exp_avg_sq")):
            if b[key] is not None:
                got = to_bits(A.bufs[k][dkey].cpu())
                assert np.array_equal(got.view(np.uint8), b[key].view(np.uint8)), (k, key)
    H.log(f"[ckpt] rank {rank}: {n} elements exported and imported bit-exact")


def test_scalar_state_get_set():
    ranks = H.DeviceRanks(PARAMS[:3], 2, 0, scaler=(True, 1024.0))
    ranks.init(weights()[:3])
    st = ranks.step(grads(1)[:3], HPS, 1.0)
    L, A, D = ranks.layouts[0], ranks.arenas[0], ranks.D
    got = D.dopt_state_scalars_get(L, A.workspace, ranks.stream)
    assert got == {"step_count": 1, "loss_scale": 1024.0, "growth_tracker": 1, "hysteresis_tracker": 1}
    assert st["step_count"] == 1
    new = {"step_count": 41, "loss_scale": 65536.0, "growth_tracker": 7, "hysteresis_tracker": 2}
    for L_, A_ in zip(ranks.layouts, ranks.arenas):
        D.dopt_state_scalars_set(L_, A_.workspace, new, ranks.stream)
    assert D.dopt_state_scalars_get(L, A.workspace, ranks.stream) == new
    st = ranks.step(grads(2)[:3], HPS, 1.0)
    assert st["loss_scale_used"] == 65536.0 and st["step_count"] == 42
    with pytest.raises(D.DoptError):
        D.dopt_state_scalars_set(L, A.workspace, dict(new, loss_scale=0.0), ranks.stream)


@pytest.mark.parametrize("scaler,max_norm,inf_at", [((False, 1.0), 1.0, None), ((True, 1024.0), 1e-3, (4, 777))],
                         ids=["clip", "overflow"])
def test_reshard_8_to_4_to_3_matches_one_rank(scaler, max_norm, inf_at):
    phases = [(8, 400_000), (4, 1_000_000), (3, 0)]
    steps_per_phase = 2
    ref = OracleRanks(PARAMS, 1, 0)
    ref.init(weights(), scaler)
    dev, state, sc, s = None, None, None, 0
    zero_w = [torch.zeros(p.numel, dtype=synth.torch_dtype(p.param_dtype)) for p in PARAMS]
    for n, bucket in phases:
        dev = H.DeviceRanks(PARAMS, n, bucket, scaler)
        if state is None:
            dev.init(weights())
        else:
            dev.init(zero_w)  # everything the continuation reads comes from the checkpoint
            dev.load(state, sc)
        for _ in range(steps_per_phase):
            s += 1
            g = grads(s, inf_at if s == 2 else None)
            got = dev.step(g, HPS, max_norm)
            want = ref.step(g, HPS, max_norm)
            H.check_stats(got, want, s)
        state, sc = dev.model_state(), dev.scalars()
        assert sc == ref.scalars(), (sc, ref.scalars())
        rep = H.check_model_state(f"N={n} step {s}", state, ref.model_state())
        ulps = H.check_model_params(f"N={n} step {s}", PARAMS, dev.model_params(), ref.model_params())
        H.log(f"[reshard] N={n} after step {s}: {rep} param ulps {ulps}")
    if inf_at is not None:
        assert sc["scale"] == 512.0 and sc["t"] == s - 1


def test_export_import_large_window_matches_oracle():
    """A window of more than 32768 tiles: the fixed-grid, grid-stride path,
    launched over more than one range of tiles."""
    params = [ParamSpec("big", 70_000_003, "bf16", "bf16"), ParamSpec("n", 5000, "f32", "f32", 0, 1),
              ParamSpec("h", 777, "bf16", "bf16", 1, 0)]
    w = [synth.fill_normal(p.param_dtype, p.numel, 5, synth.weight_stream(i), 0, 0.02) for i, p in enumerate(params)]
    g = [synth.fill_normal(p.grad_dtype, p.numel, 5, synth.grad_stream(i), 1, 1e-2) for i, p in enumerate(params)]
    ranks = H.DeviceRanks(params, 1, 0)
    ranks.init(w)
    ranks.step(g, HPS, 1.0)
    L, A = ranks.layouts[0], ranks.arenas[0]
    assert L.buffer(0)["arena_numel"] // 2048 > 32768
    run = OracleRun(params, 1, 0, 0, arena_numel=[A.info[k]["n"] for k in range(L.num_buffers)])
    _oracle_view(run, ranks, 0)
    n = L.state_numel
    ex = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    ranks.D.dopt_state_export(L, A.bufs, *ex, A.workspace, ranks.stream)
    for e, x in zip(ex, oracle_export(run)):
        assert np.array_equal(e.cpu().numpy().view(np.uint32), x.view(np.uint32))
    rng = np.random.default_rng(9)
    new = tuple((rng.standard_normal(n) * s).astype(np.float32) for s in (0.05, 1e-3, 1e-6))
    ranks.D.dopt_state_import(L, A.bufs, *[torch.from_numpy(e).cuda() for e in new], A.workspace, ranks.stream)
    oracle_import(run, new)
    for k, b in enumerate(run.bufs):
        for key, dkey in (("param", "param"), ("master", "master"), ("m", "exp_avg"), ("v", "exp_avg_sq")):
            if b[key] is not None:
                assert np.array_equal(to_bits(A.bufs[k][dkey].cpu()).view(np.uint8), b[key].view(np.uint8)), (k, key)
