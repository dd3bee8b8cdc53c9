"""The memory ledger the pages print, recomputed from the oracle's layout.

Per-rank optimizer state is 4 B of fp32 master per 16-bit shard element plus
8 B of Adam moments per shard element; summed over all ranks it must count
every param element exactly once (12 B/param), and the per-card totals must
reproduce the pages' figures (tests/golden/ledger.json, each with its page).
"""
import json
import os

import pytest

import oracle
from synth.models import ParamSpec

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ledger.json")))
GB = 1e9


def _state_bytes(L):
    tot = 0
    for k in range(L.num_buffers):
        b = L.buffer(k)
        per = 12 if b["param_dtype"] != 0 else 8  # fp32 params are their own master
        tot += per * b["shard_numel"]
    return tot


def _window_elems(L):
    return sum(L.buffer(k)["window_numel"] for k in range(L.num_buffers))


def _params(total, pieces, dt="bf16"):
    assert total % pieces == 0
    return [ParamSpec(f"p{i}", total // pieces, dt, dt) for i in range(pieces)]


def test_7b_dp8():
    g = GOLDEN
    P = g["p_7b"]
    params = _params(P, 7)
    per_rank = [_state_bytes(oracle.Layout(params, 8, r, 40_000_000)) for r in range(8)]
    assert sum(per_rank) == g["state_bytes_per_param"] * P
    assert sum(per_rank) / GB == pytest.approx(g["adam_state_7b_gb"], rel=1e-12)
    for s in per_rank:
        assert s / GB == pytest.approx(g["dp8_state_per_card_gb"], rel=1e-12)
    saving = g["adam_state_7b_gb"] - per_rank[0] / GB
    assert saving == pytest.approx(g["dp8_saving_gb"], rel=1e-12)
    assert saving / g["adam_state_7b_gb"] == pytest.approx(g["dp8_saving_frac"], rel=1e-12)


@pytest.mark.parametrize("N", [1, 2, 8, 64])
def test_ledger_formula(N):
    # per card: full 16-bit params + full 16-bit grads + this rank's state (ZeRO-1),
    # or the rank's grad window (ZeRO-2), or both windows (ZeRO-3)
    P = 64 * 128 * 1000 * 7
    params = _params(P, 7)
    c = GOLDEN["ledger_coeffs"]
    for r in (0, N - 1):
        L = oracle.Layout(params, N, r, 0)
        st = _state_bytes(L)
        win = _window_elems(L)
        assert st == 12 * P // N
        zero1 = 2 * P + 2 * P + st
        zero2 = 2 * P + 2 * win + st
        zero3 = 2 * win + 2 * win + st
        assert zero1 == c["zero1"][0] * P + c["zero1"][1] * P // N
        assert zero2 == c["zero2"][0] * P + c["zero2"][1] * P // N
        assert zero3 == c["zero3"][0] * P + c["zero3"][1] * P // N
        if N == 1:
            assert zero1 == c["ddp"][0] * P


def test_deepspeed_7p5b():
    g = GOLDEN
    P = g["p_7p5b"]
    params = _params(P, 75, "f16")
    L1 = oracle.Layout(params, 1, 0, 0)
    st = _state_bytes(L1)
    assert 2 * P / GB == pytest.approx(g["ds_params_gb"])
    assert 2 * _window_elems(L1) / GB == pytest.approx(g["ds_grads_gb"])
    assert st / GB == pytest.approx(3 * g["ds_each_fp32_gb"])
    assert (2 * P + 2 * _window_elems(L1) + st) / GB == pytest.approx(g["ds_total_gb"])
    z = g["ds_zero2_dp8"]
    for r in (0, 7):
        L = oracle.Layout(params, 8, r, 0)
        assert 2 * _window_elems(L) / GB == pytest.approx(z["grads_gb"])
        assert _state_bytes(L) / GB == pytest.approx(z["state_gb"])
        assert (2 * P + 2 * _window_elems(L) + _state_bytes(L)) / GB == pytest.approx(z["total_gb"])


def test_every_element_once_with_padding():
    # odd sizes: padding and gaps never enter the state; the union over ranks is P exactly
    params = [ParamSpec("a", 1001, "bf16", "bf16"), ParamSpec("b", 77, "bf16", "bf16"),
              ParamSpec("c", 4097, "bf16", "bf16"), ParamSpec("d", 3, "f32", "f32")]
    P = sum(p.numel for p in params)
    for N in (3, 8, 64):
        tot_state_elems = 0
        for r in range(N):
            L = oracle.Layout(params, N, r, 2000)
            tot_state_elems += sum(L.buffer(k)["shard_numel"] for k in range(L.num_buffers))
        assert tot_state_elems == P


@pytest.mark.parametrize("N,I", [(8, 2), (64, 8), (16, 16), (6, 3)])
def test_instances_ledger(N, I):
    # "02 · ZeRO 显存账本…" §5: with I optimizer instances the 12P of state is cut
    # to 1/(N/I) per rank, every instance holding one full copy of it.
    P = 64 * 128 * 48 * 5
    params = _params(P, 5)
    per = N // I
    states = [_state_bytes(oracle.Layout(params, N, r, 0, 0, I)) for r in range(N)]
    for r in range(N):
        assert states[r] == 12 * P // per
    for i in range(I):
        assert sum(states[i * per:(i + 1) * per]) == 12 * P
    assert sum(states) == I * 12 * P
