"""Pins for the oracle's shard layout (integer results, bit-exact).

What the layout must satisfy comes from "Megatron-LM distrib_optimizer.py
源码精读": sections "Bucket 划分算法：逆序遍历 + 尺寸触发", "两级 Padding 机制",
"最终内存大小断言", "Bucket 级别的均等切分", "Range 类：四种视角的统一抽象" and the
group-building section.  The checks below are written as properties of the
result (ownership enumerated element by element, a declarative statement of
the bucket rules), not as a second copy of the construction.
"""
import json
import math
import os
import random

import numpy as np
import pytest

import oracle
from synth.models import ParamSpec, tiny

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _divisor(n, busbw):
    d = n * 128 // math.gcd(n, 128)
    if busbw:
        d = d * 65536 // math.gcd(d, 65536)
    return d


def _round_up(x, d):
    return -(-x // d) * d


def test_tiny_hand_derivation():
    # Params in model order: w0 (64x32 = 2048), b0 (32), w1 (32x16 = 512), b1 (16).
    # Placement runs last-to-first with starts raised to multiples of 64:
    #   b1 at [0,16); w1 at round_up(16,64)=64 -> [64,576); b0 at 576 -> [576,608);
    #   w0 at round_up(608,64)=640 -> [640,2688).
    # No size trigger: one bucket, closed at 2688, padded to a multiple of
    # lcm(4,128)=128 -> 2688 (=21*128). Shard = 2688/4 = 672.
    # Rank 1's window is [672,1344): it cuts w0 on both sides; w0's elements
    # 32..703 are rank 1's.  Nothing else of rank 1's window is a param.
    L = oracle.Layout(tiny(), 4, 1, 0)
    assert L.num_buffers == 1
    b = L.buffer(0)
    assert (b["numel"], b["numel_unpadded"], b["n_buckets"], b["window_numel"], b["shard_numel"]) == \
        (2688, 2688, 1, 672, 672)
    assert [(L.param(i)["start"], L.param(i)["end"]) for i in range(4)] == \
        [(640, 2688), (576, 608), (64, 576), (0, 16)]
    w0 = L.param(0)
    assert w0["has_shard"] == 1
    assert w0["gbuf_world"] == (672, 1344)
    assert w0["gbuf_world_in_bucket"] == (672, 1344)
    assert w0["gbuf_local"] == (0, 672)
    assert w0["param"] == (32, 704)
    assert [L.param(i)["has_shard"] for i in (1, 2, 3)] == [0, 0, 0]
    # Rank 0 owns b1, w1, b0 and w0[0:32) (with the 64-alignment gaps between them).
    L0 = oracle.Layout(tiny(), 4, 0, 0)
    assert [L0.param(i)["param"] for i in range(4)] == [(0, 32), (0, 32), (0, 512), (0, 16)]
    assert L0.buffer(0)["shard_numel"] == 32 + 32 + 512 + 16


def test_pages_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    ps = [ParamSpec("w", g["bucket_numel"], g["dtype"], g["dtype"])]
    for r in range(g["dp_size"]):
        L = oracle.Layout(ps, g["dp_size"], r, 0)
        assert L.buffer(0)["numel"] == g["bucket_numel"]
        assert L.bucket(0, 0)["shard"] == g["per_rank_shard"]
        assert L.param(0)["param"] == (r * g["per_rank_shard"], (r + 1) * g["per_rank_shard"])
        assert L.buffer(0)["shard_numel"] == g["per_rank_shard"]


def _check_partition(params, L, bucket_size, busbw, N):
    """Declarative statement of the bucket rules, checked on the oracle's output."""
    div = _divisor(N, busbw)
    nb = L.num_buffers
    seen = set()
    for k in range(nb):
        info = L.buffer(k)
        idx = [i for i in range(len(params)) if L.param(i)["buffer"] == k]
        dts = {(params[i].param_dtype, params[i].grad_dtype) for i in idx}
        assert len(dts) == 1
        seen |= dts
        buckets = [L.bucket(k, b) for b in range(info["n_buckets"])]
        # buckets tile [0, numel) in order, each a multiple of the divisor
        off = 0
        for bk in buckets:
            assert bk["offset"] == off
            assert bk["numel"] % div == 0 and bk["numel"] > 0
            assert bk["numel"] == _round_up(bk["offset"] + bk["numel_unpadded"], div) - bk["offset"]
            off += bk["numel"]
        assert info["numel"] == off
        assert info["numel"] % N == 0
        assert info["numel_unpadded"] == sum(b["numel_unpadded"] for b in buckets) <= info["numel"]
        placed = list(reversed(idx))  # placement order is reverse model order
        prev = None
        for j, i in enumerate(placed):
            p = L.param(i)
            assert p["start"] % 64 == 0 and p["end"] - p["start"] == params[i].numel
            bk = buckets[p["bucket"]]
            assert bk["offset"] <= p["start"] and p["end"] <= bk["offset"] + bk["numel_unpadded"]
            newb = bool(params[i].requires_new_bucket)
            if prev is None:
                first = True
            else:
                pp = L.param(prev)
                pbk = buckets[pp["bucket"]]
                prev_closed = (bucket_size > 0 and pp["end"] - pbk["offset"] >= bucket_size) or \
                    bool(params[prev].requires_new_bucket)
                first = prev_closed or newb
                if first:
                    assert p["bucket"] == pp["bucket"] + 1 and p["start"] == bk["offset"]
                    # the bucket before closed at the previous end (size trigger or a lone
                    # param) or at the 64-aligned start of this lone param
                    end_unp = pbk["offset"] + pbk["numel_unpadded"]
                    assert end_unp == (pp["end"] if prev_closed else _round_up(pp["end"], 64))
                else:
                    assert p["bucket"] == pp["bucket"] and p["start"] == _round_up(pp["end"], 64)
            if first and prev is None:
                assert p["bucket"] == 0 and p["start"] == 0
            prev = i
        last = L.param(placed[-1])
        lbk = buckets[last["bucket"]]
        assert last["bucket"] == len(buckets) - 1
        assert lbk["offset"] + lbk["numel_unpadded"] == last["end"]
    assert seen == {(p.param_dtype, p.grad_dtype) for p in params}


def _check_ownership(params, layouts, N):
    """Enumerate, element by element, which rank owns each buffer element and
    compare every rank's four views with that enumeration."""
    L0 = layouts[0]
    for k in range(L0.num_buffers):
        numel = L0.buffer(k)["numel"]
        owner = np.full(numel, -1, np.int64)
        nbk = L0.buffer(k)["n_buckets"]
        for r, L in enumerate(layouts):
            for b in range(nbk):
                bk = L.bucket(k, b)
                ws = bk["window_start"]
                assert np.all(owner[ws:ws + bk["shard"]] == -1)
                owner[ws:ws + bk["shard"]] = r
        assert np.all(owner >= 0)  # windows tile every bucket
        for r, L in enumerate(layouts):
            arena_base = {}
            acc = 0
            for b in range(nbk):
                arena_base[b] = acc
                assert L.bucket(k, b)["arena_offset"] == acc
                acc += L.bucket(k, b)["shard"]
            assert L.buffer(k)["window_numel"] == acc
            tot = 0
            for i in range(len(params)):
                p = L.param(i)
                if p["buffer"] != k:
                    continue
                el = np.arange(p["start"], p["end"])
                mine = el[owner[p["start"]:p["end"]] == r]
                if mine.size == 0:
                    assert p["has_shard"] == 0
                    continue
                assert p["has_shard"] == 1
                assert mine[-1] - mine[0] + 1 == mine.size  # contiguous
                lo, hi = int(mine[0]), int(mine[-1]) + 1
                bk = L.bucket(k, p["bucket"])
                assert p["gbuf_world"] == (lo, hi)
                assert p["gbuf_world_in_bucket"] == (lo - bk["offset"], hi - bk["offset"])
                assert p["gbuf_local"] == (lo - bk["window_start"], hi - bk["window_start"])
                assert p["param"] == (lo - p["start"], hi - p["start"])
                assert p["arena_offset"] == arena_base[p["bucket"]] + lo - bk["window_start"]
                tot += hi - lo
            assert L.buffer(k)["shard_numel"] == tot
        # every param element is owned by exactly one rank (the union covers it once)
        for i in range(len(params)):
            p = L0.param(i)
            if p["buffer"] != k:
                continue
            assert sum((L.param(i)["param"][1] - L.param(i)["param"][0]) for L in layouts) == params[i].numel


def _random_params(rng, n, dtypes=(("bf16", "bf16"),), newb_p=0.0, max_numel=400):
    out = []
    for j in range(n):
        pd, gd = rng.choice(dtypes)
        out.append(ParamSpec(f"p{j}", rng.randint(1, max_numel), pd, gd,
                             int(rng.random() < newb_p), rng.randint(0, 2)))
    return out


@pytest.mark.parametrize("seed", range(40))
def test_random_layouts_brute_force(seed):
    rng = random.Random(seed)
    N = rng.choice([1, 2, 3, 4, 5, 8, 16, 64, 96, 128])
    dts = [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16"), ("f32", "f32")]
    params = _random_params(rng, rng.randint(1, 14), dtypes=dts[: rng.randint(1, 4)],
                            newb_p=rng.choice([0.0, 0.2]))
    bucket_size = rng.choice([0, 1, 100, 500, 2000])
    busbw = int(seed % 7 == 0)
    layouts = [oracle.Layout(params, N, r, bucket_size, busbw) for r in range(N)]
    _check_partition(params, layouts[0], bucket_size, busbw, N)
    _check_ownership(params, layouts, N)


def test_unaligned_windows():
    # 384 + 321 elements at N=64: numel 768 -> shard 12; windows start at 0/4 mod 8.
    params = [ParamSpec("a", 384, "bf16", "bf16"), ParamSpec("b", 321, "bf16", "bf16")]
    layouts = [oracle.Layout(params, 64, r, 0) for r in range(64)]
    assert layouts[0].buffer(0)["numel"] == 768
    assert {L.bucket(0, 0)["window_start"] % 8 for L in layouts} == {0, 4}
    _check_ownership(params, layouts, 64)


def test_groups():
    params = [ParamSpec("a", 100, "bf16", "f32", 0, 0), ParamSpec("n", 64, "f32", "f32", 0, 1),
              ParamSpec("b", 300, "bf16", "f32", 0, 1), ParamSpec("c", 5, "f32", "f32", 0, 0)]
    L = oracle.Layout(params, 1, 0, 0)
    # at N=1 every param has a shard; 16-bit params go to the float16 lists,
    # fp32 params to the fp32 lists, split per hyper-group, in model order
    assert L.group("model_float16", 0) == [0] and L.group("model_float16", 1) == [2]
    assert L.group("shard_float16", 1) == [2] and L.group("shard_fp32_from_float16", 1) == [2]
    assert L.group("model_fp32", 0) == [3] and L.group("shard_fp32", 1) == [1]
    assert L.group("shard_fp32", 0) == [3]


def test_errors():
    ps = tiny()
    for args in [(0, 0), (4, 4), (4, -1)]:
        with pytest.raises(oracle.OracleError):
            oracle.Layout(ps, *args)
    with pytest.raises(oracle.OracleError):
        oracle.Layout([ParamSpec("z", 0, "bf16", "bf16")], 1, 0)


@pytest.mark.parametrize("N,I", [(8, 2), (12, 3), (64, 4)])
def test_instances_own_every_element_once_per_instance(N, I):
    rng = random.Random(N * 100 + I)
    params = _random_params(rng, 9, newb_p=0.1)
    per = N // I
    for i in range(I):
        layouts = [oracle.Layout(params, N, r, 700, 0, I) for r in range(i * per, (i + 1) * per)]
        # within an instance the windows are those of a plain N/I-rank layout
        _check_partition(params, layouts[0], 700, 0, per)
        _check_ownership(params, layouts, per)
    with pytest.raises(oracle.OracleError):
        oracle.Layout(params, N, 0, 0, 0, N + 1)
