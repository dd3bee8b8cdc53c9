"""GPU parity: the HIP path (called through the C ABI) against the oracle.

Tiny and GPT-2-small are compared element by element after every step; the
three multi-billion-byte workloads run at full size on the device, with the
oracle computing the exact per-step statistics over every shard element and
the trajectories of about a million sampled elements per buffer (plus every
segment's first and last element).  Edge cases: windows that start at odd
offsets, empty windows, mixed dtypes and hyper-groups, lone-param buckets,
bus-bandwidth padding, all-zero grads, NaN / -inf overflow, the dynamic loss
scaler's growth, hysteresis, backoff and floor, clipping on and off, the
three-call split API, and run-to-run determinism.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.models import ParamSpec
from tests import gpu_harness as H
from tests.oracle_harness import OracleRun, to_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    H.log(f"[gpu-test] start {request.node.name}")
    yield
    torch.cuda.synchronize()


def test_tiny_workload_full():
    H.run_full(H.case_from_workload(synth.WORKLOADS["tiny"]))


def test_gpt2_small_workload_full():
    rep = H.run_full(H.case_from_workload(synth.WORKLOADS["gpt2-small"]))
    assert rep[-1]["param0"]["n"] == 15_554_976


def test_chunked_full_compare_on_gpt2_small_and_a_gapped_layout():
    # the threaded full-size harness (used on request for the largest
    # workloads) on small windows split into many ranges, one with
    # alignment gaps, bucket padding and an overflow-skipped step
    case = H.case_from_workload(synth.WORKLOADS["gpt2-small"])
    case.steps = 3
    rep = H.run_full_chunked(case, chunk=1 << 20)
    assert rep[-1]["master"]["n"] == 15_554_976 and rep[-1]["param"]["bit_exact"] == 1.0
    params = [ParamSpec(f"p{i}", n, "bf16", "bf16") for i, n in enumerate([1000, 77, 4097, 3, 20000, 9, 131])]
    case = H.Case("odd-chunked", params, 8, 5, bucket_size=2000, steps=4, dynamic=True, initial_scale=1024.0,
                  inf_step=2)
    rep = H.run_full_chunked(case, chunk=4096)
    assert [r["skipped"] for r in rep] == [0, 1, 0, 0]


@pytest.mark.timeout(600)
def test_llama3_8b_workload_sampled():
    H.run_sampled(H.case_from_workload(synth.WORKLOADS["llama3-8b"]))


@pytest.mark.timeout(900)
def test_dense_7b_workload_sampled():
    # on arenas placed region by region, as the bench runs this workload
    case = H.case_from_workload(synth.WORKLOADS["dense-7b"])
    case.placement, case.placement_tries = "regions", 2
    rep = H.run_sampled(case)
    assert [r["skipped"] for r in rep] == [0, 0, 1, 0, 0]


@pytest.mark.timeout(600)
def test_llama3_70b_workload_sampled():
    H.run_sampled(H.case_from_workload(synth.WORKLOADS["llama3-70b"]))


@pytest.mark.parametrize("rank", [0, 5, 37, 63])
def test_unaligned_windows(rank):
    params = [ParamSpec("a", 384, "bf16", "bf16"), ParamSpec("b", 321, "bf16", "bf16")]
    H.run_full(H.Case(f"unaligned-r{rank}", params, 64, rank, steps=3))


@pytest.mark.parametrize("rank", [0, 77, 127])
def test_odd_shards_many_buckets(rank):
    params = [ParamSpec(f"p{i}", n, "bf16", "bf16") for i, n in enumerate([1000, 77, 4097, 3, 20000, 9, 131])]
    H.run_full(H.Case(f"odd-r{rank}", params, 128, rank, bucket_size=2000, steps=3))


def test_mixed_dtypes_hgroups_lone_buckets():
    params = [ParamSpec("emb", 50000, "bf16", "f32", 1, 0), ParamSpec("w1", 7000, "bf16", "f32", 0, 0),
              ParamSpec("n1", 256, "f32", "f32", 0, 1), ParamSpec("h1", 3333, "f16", "f16", 0, 2),
              ParamSpec("w2", 12345, "bf16", "f32", 0, 1), ParamSpec("h2", 999, "f16", "f32", 0, 0),
              ParamSpec("n2", 100, "f32", "f32", 0, 0)]
    hps = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (3e-4, 0.8, 0.99, 1e-6, 0.0), (2e-3, 0.95, 0.9999, 1e-8, 0.1)]
    H.run_full(H.Case("mixed", params, 3, 1, bucket_size=5000, steps=4, hparams=hps))


def test_every_dtype_pair():
    """All nine (param dtype, grad dtype) pairs, one flat buffer each of two
    params in two buckets, with window ends that cut params and
    tiles."""
    dts = ["f32", "bf16", "f16"]
    pairs = [(pd, gd) for pd in dts for gd in dts]
    params = []
    for i, (pd, gd) in enumerate(pairs):
        params += [ParamSpec(f"{pd}-{gd}-a", 9_001 + 2_048 * i, pd, gd, 0, i % 3),
                   ParamSpec(f"{pd}-{gd}-b", 3_001 + 517 * i, pd, gd, 0, (i + 1) % 3)]
    hps = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (3e-4, 0.8, 0.99, 1e-6, 0.0), (2e-3, 0.95, 0.9999, 1e-8, 0.1)]
    for r in (0, 2):
        rep = H.run_full(H.Case(f"dtype-pairs-r{r}", params, 3, r, bucket_size=2_500, steps=3, hparams=hps))
        assert sum(1 for k in rep[-1] if k.startswith("param")) == 9


def test_one_nonzero_hgroup_full_tiles():
    """Every shard of the buffer in hyper-group 2, with tiles wholly inside one
    shard: pass 2 takes such tiles' AdamW scalars from the group it loaded
    up front, which must be group 2's (the three groups differ)."""
    params = [ParamSpec("a", 50_000, "bf16", "bf16", 0, 2), ParamSpec("b", 30_011, "bf16", "bf16", 0, 2)]
    hps = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (3e-4, 0.8, 0.99, 1e-6, 0.0), (2e-3, 0.95, 0.9999, 1e-8, 0.1)]
    H.run_full(H.Case("hgroup2", params, 2, 1, steps=3, hparams=hps))


def test_high_busbw_padding():
    params = [ParamSpec("a", 100_000, "bf16", "bf16"), ParamSpec("b", 3000, "bf16", "bf16")]
    H.run_full(H.Case("busbw", params, 8, 6, busbw=1, steps=2))


def test_empty_window():
    # one 64-element param at N=4: numel pads to 128, ranks 2 and 3 own only padding
    params = [ParamSpec("a", 64, "bf16", "bf16")]
    for r in (2, 3):
        rep = H.run_full(H.Case(f"empty-r{r}", params, 4, r, steps=2))
        assert rep[-1]["param0"]["n"] == 0 and rep[-1]["norm_dev"] == 0.0


def test_all_zero_grads():
    params = [ParamSpec("a", 70000, "bf16", "bf16"), ParamSpec("b", 500, "bf16", "bf16")]
    rep = H.run_full(H.Case("zeros", params, 2, 1, steps=2, const_grad=0.0))
    assert rep[-1]["norm_dev"] == 0.0


@pytest.mark.parametrize("bad", [math.nan, -math.inf, math.inf])
def test_overflow_skips_step(bad):
    params = [ParamSpec("a", 40000, "f16", "f16"), ParamSpec("b", 1000, "f16", "f16")]
    H.run_full(H.Case("overflow", params, 2, 0, steps=4, dynamic=True, initial_scale=1024.0, inf_step=2,
                      inf_value=bad, grad_sigma=1e-3))


def test_dynamic_scaler_growth_hysteresis_backoff_and_floor():
    """The dynamic loss scaler through each of its rules, with a growth
    interval of 2 and a hysteresis of 2: growth after clean steps, the first
    overflow of a run kept at the same scale, backoff from the second on, the
    minimum scale as a floor, and the hysteresis restored by a growth.  13
    steps, overflows planted at steps 3, 4 and 7 to 11, each step's grads
    drawn at the scale the step carries.  Every step: the stats, the scalar
    state (scale, growth and hysteresis trackers, step count) and every shard
    element against the oracle."""
    params = [ParamSpec("a", 5000, "bf16", "bf16"), ParamSpec("h", 3000, "f16", "f16")]
    rules = dict(growth_factor=2.0, backoff_factor=0.5, growth_interval=2, hysteresis=2, min_scale=4.0)
    case = H.Case("scaler-rules", params, 2, 1, 0, steps=13, dynamic=True, initial_scale=16.0)
    dev = H.DeviceRun(case)
    D = dev.D
    arena = [dev.L.buffer(k)["arena_numel"] for k in range(dev.L.num_buffers)]
    orc = OracleRun(params, 2, 1, 0, arena_numel=arena)
    orc.scaler = oracle.make_scaler(True, 16.0, **rules)
    for k, b in enumerate(orc.bufs):
        t = H.host_weights(case, k, b["pd"], b["n"])
        b["param"][:] = to_bits(t)
        dev.A.bufs[k]["param"].copy_(t)
    D.dopt_init_state(dev.L, dev.A.bufs, D.scaler_cfg(True, 16.0, **rules), dev.A.workspace, dev.stream)
    orc.init_state()
    masks = [orc.valid(k) for k in range(orc.nb)]
    scales = []
    for s in range(1, case.steps + 1):
        carried = orc.scaler.scale
        grads = []
        for k, b in enumerate(orc.bufs):
            g = synth.fill_normal(b["gd"], b["n"], 0, synth.grad_stream(k), s, 1e-2, scale=carried)
            if s in (3, 4, 7, 8, 9, 10, 11) and k == s % 2:
                owned = np.flatnonzero(masks[k])
                g[int(owned[(37 * s) % owned.size])] = math.inf
            b["grad"][:] = to_bits(g)
            grads.append(g)
        ref = orc.step(case.hparams, case.max_norm)
        got = dev.step(grads)
        H.check_stats(got, ref, s)
        sc = D.dopt_state_scalars_get(dev.L, dev.A.workspace, dev.stream)
        assert sc == {"step_count": orc.t, "loss_scale": orc.scaler.scale,
                      "growth_tracker": orc.scaler.growth_tracker,
                      "hysteresis_tracker": orc.scaler.hysteresis_tracker}, (s, sc)
        for k, b in enumerate(orc.bufs):
            m = masks[k]
            H.check_f32(f"step {s} master[{k}]", dev.host(k, "master")[m], b["master"][m])
            H.check_f32(f"step {s} m[{k}]", dev.host(k, "exp_avg")[m], b["m"][m])
            H.check_f32(f"step {s} v[{k}]", dev.host(k, "exp_avg_sq")[m], b["v"][m])
            H.check_param(f"step {s} param[{k}]", dev.host(k, "param")[m], b["param"][m], b["pd"])
        scales.append((carried, bool(ref.skipped), orc.scaler.scale))
    # every rule was taken: a growth, an overflow kept at its scale, a backoff, and the floor
    assert any(not sk and after > before for before, sk, after in scales), scales
    assert any(sk and after == before for before, sk, after in scales), scales
    assert any(sk and after < before for before, sk, after in scales), scales
    assert any(sk and before == rules["min_scale"] and after == before for before, sk, after in scales), scales


def test_clip_off_and_clip_active():
    params = [ParamSpec("a", 30000, "bf16", "bf16")]
    H.run_full(H.Case("noclip", params, 1, 0, steps=2, max_norm=0.0, grad_sigma=1.0))
    H.run_full(H.Case("bigclip", params, 1, 0, steps=2, max_norm=1.0, grad_sigma=1.0))
    H.run_full(H.Case("noclip-small", params, 1, 0, steps=2, max_norm=1.0, grad_sigma=1e-5))


def test_split_api_matches_one_call():
    params = [ParamSpec("a", 9000, "bf16", "bf16"), ParamSpec("n", 64, "f32", "f32")]
    H.run_full(H.Case("split", params, 4, 2, steps=4), split_steps=(1, 3), half_steps=(2,))


def test_split_api_large_window():
    """A window of more than 8192 tiles: pass 1 runs on its large-window grid
    (more than 2048 partials), so the reduction of the split API (no
    finalize) and of the fused step both take the 1024-thread finish."""
    import sharded_mixed_precision_amd as D
    params = [ParamSpec("a", 25_000_003, "bf16", "bf16"), ParamSpec("b", 24_999_999, "bf16", "bf16"),
              ParamSpec("n", 4096, "f32", "f32")]
    L = D.dopt_build_ranges(params, 2, 1)
    b0 = L.buffer(0)
    assert b0["arena_numel"] // D.DOPT_ARENA_ALIGN > 8192
    H.run_full(H.Case("split-large", params, 2, 1, steps=3), split_steps=(1, 3), half_steps=(2,))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dt,n,r", [(("bf16", "bf16"), 1, 0), (("f16", "f32"), 2, 1), (("f32", "f32"), 1, 0)],
                         ids=["bf16-n1", "f16-f32-n2", "f32-n1"])
def test_large_window_with_boundary_tiles(dt, n, r):
    """A window of more than 16384 tiles (pass 2 grid-strides over it) whose
    params meet inside tiles: tiles shared by two params of one hyper-group
    (updated from registers and stored element by element) and by params of
    two hyper-groups (updated element by element with each one's scalars);
    every element compared for 3 steps."""
    import sharded_mixed_precision_amd as D
    pd, gd = dt
    sizes = [(20_000_003, 0), (3_000_001, 0), (9_999_999, 1), (7_000_001, 2), (333, 2)]
    params = [ParamSpec(f"p{i}", k * n, pd, gd, 0, hg) for i, (k, hg) in enumerate(sizes)]
    hps = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (3e-4, 0.8, 0.99, 1e-6, 0.0), (2e-3, 0.95, 0.9999, 1e-8, 0.1)]
    L = D.dopt_build_ranges(params, n, r)
    assert L.buffer(0)["arena_numel"] // D.DOPT_ARENA_ALIGN > 16384 and L.buffer(0)["apply_bnd"] == 1
    H.run_full(H.Case(f"bnd-{pd}-{gd}-n{n}", params, n, r, steps=3, hparams=hps))


def test_many_tiny_params():
    """About 3000 params of 1 to 100 elements (64-element aligned starts): nearly
    every tile is a boundary tile holding up to 32 shards, the worst case of
    the per-element ownership walk in both passes; three hyper-groups."""
    rng = np.random.default_rng(7)
    sizes = rng.integers(1, 101, size=3000)
    params = [ParamSpec(f"t{i}", int(n), "bf16", "bf16", 0, i % 3) for i, n in enumerate(sizes)]
    hps = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (3e-4, 0.8, 0.99, 1e-6, 0.0), (2e-3, 0.95, 0.9999, 1e-8, 0.1)]
    H.run_full(H.Case("tiny-params", params, 3, 1, bucket_size=40_000, steps=3, hparams=hps))


def test_extreme_magnitudes():
    """Grads at both ends of the fp32 range, fp32 and bf16 grad buffers.
    Subnormal grads (sigma 1e-38) must be kept, not flushed to zero, in both
    passes.  Grads near 1e37 are finite, their double sum of squares too, but
    g*g overflows fp32 in the moment update when nothing clips them, so v and
    its square root become +inf and the Adam term 0; with clipping the grads
    are scaled to tiny values first."""
    params = [ParamSpec("a", 20_000, "bf16", "f32"), ParamSpec("b", 3_000, "bf16", "bf16")]
    H.run_full(H.Case("subnormal", params, 2, 1, steps=3, grad_sigma=1e-38))
    H.run_full(H.Case("huge-noclip", params, 2, 1, steps=2, grad_sigma=1e37, max_norm=0.0))
    H.run_full(H.Case("huge-clip", params, 2, 1, steps=2, grad_sigma=1e37))


def test_placement_search_arenas():
    """Arenas chosen by the placement search (the kept candidate set refined
    array by array and zeroed, the others freed) carry the step exactly like a
    plain allocation."""
    case = H.case_from_workload(synth.WORKLOADS["gpt2-small"])
    case.name, case.steps, case.placement_tries = "gpt2-placement", 3, 3
    dev = H.DeviceRun(case)
    assert dev.A.placement["candidates"] == 3 and len(dev.A.placement["pass2_ms"]) == 3
    assert [r[1] for r in dev.A.placement["refined"]] == ["grad", "param", "master", "exp_avg", "exp_avg_sq"]
    del dev
    H.run_full(case)


def test_region_placed_arenas():
    """Arenas whose large arrays are reserved address ranges backed region by
    region (dopt_vmm.h), each region's backing chosen by timing pass 2 on it:
    the step over them equals the oracle element by element, and the arena
    tensors are views of the reserved ranges.  Regions of 2^20 elements give
    the GPT-2-small rank's arrays 15 regions each (the last one partly used)."""
    case = H.case_from_workload(synth.WORKLOADS["gpt2-small"])
    case.name, case.steps, case.placement_tries = "gpt2-regions", 3, 3
    case.placement, case.region_elems = "regions", 1 << 20
    dev = H.DeviceRun(case)
    p = dev.A.placement
    assert p["kind"] == "regions" and p["buffers"][0]["regions"] == 15
    assert len(p["buffers"][0]["last_sweep"]) == 15
    back = dev.A._backings[0]
    assert dev.A.bufs[0]["master"].data_ptr() == back["master"].va
    assert dev.A.bufs[0]["param"].dtype == torch.bfloat16 and dev.A.bufs[0]["param"].data_ptr() == back["param"].va
    del dev, back
    H.run_full(case)


def test_deterministic():
    case = H.case_from_workload(synth.WORKLOADS["gpt2-small"])
    case.steps = 2
    outs = []
    for _ in range(2):
        dev = H.DeviceRun(case)
        nb = dev.L.num_buffers
        params0 = [H.host_weights(case, k, "bf16", dev.L.buffer(k)["arena_numel"]) for k in range(nb)]
        dev.init(params0)
        stats = []
        for s in (1, 2):
            g = [H.host_grads(case, k, "bf16", dev.L.buffer(k)["arena_numel"], s) for k in range(nb)]
            stats.append(dev.step(g))
        outs.append((stats, [dev.host(0, key) for key in ("master", "exp_avg", "exp_avg_sq", "param")]))
    assert outs[0][0] == outs[1][0]
    for a, b in zip(outs[0][1], outs[1][1]):
        assert np.array_equal(a, b)


def test_argument_errors_are_reported():
    import sharded_mixed_precision_amd as D
    from sharded_mixed_precision_amd.arena import DeviceArenas
    params = [ParamSpec("a", 5000, "bf16", "bf16", 0, 1)]
    L = D.dopt_build_ranges(params, 2, 0)
    A = DeviceArenas(L)
    stream = torch.cuda.current_stream()
    D.dopt_init_state(L, A.bufs, D.scaler_cfg(), A.workspace, stream)
    with pytest.raises(D.DoptError) as e:  # hgroup 1 needs two hparam sets
        D.dopt_step(L, A.bufs, [(1e-3, 0.9, 0.999, 1e-8, 0.0)], 1.0, A.workspace, stream)
    assert e.value.code == -1
    bad = dict(A.bufs[0])
    bad["grad"] = A.bufs[0]["grad"].data_ptr() + 2  # a raw address 2 bytes off: not 256-byte aligned (the library)
    with pytest.raises(D.DoptError, match="aligned"):
        D.dopt_step(L, [bad], [(1e-3, 0.9, 0.999, 1e-8, 0.0)] * 2, 1.0, A.workspace, stream)
    bad["grad"] = A.bufs[0]["grad"][1:]  # one element short (the binding)
    with pytest.raises(D.DoptError, match="at least"):
        D.dopt_step(L, [bad], [(1e-3, 0.9, 0.999, 1e-8, 0.0)] * 2, 1.0, A.workspace, stream)
    with pytest.raises(D.DoptError):
        D.dopt_init_state(L, A.bufs, D.scaler_cfg(True, 0.0), A.workspace, stream)


def test_instances_gpt2_small():
    # N=16 split into 2 optimizer instances of 8: rank 11 owns shard 3 of its instance
    case = H.case_from_workload(synth.WORKLOADS["gpt2-small"])
    case.name, case.dp_size, case.dp_rank, case.instances, case.steps = "gpt2-inst", 16, 11, 2, 3
    rep = H.run_full(case)
    assert rep[-1]["param0"]["n"] == 15_554_976
