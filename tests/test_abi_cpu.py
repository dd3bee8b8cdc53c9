"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, and its host range mapper is bit-exact against the oracle on the
five workloads and on random layouts.  No device call is made here."""
import ctypes
import glob
import os
import random
import re

import pytest

import oracle
from synth import PARAM_LISTS, WORKLOADS
from synth.models import ParamSpec
from tests.oracle_harness import shard_pieces

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _dopt():
    import sharded_mixed_precision_amd as d
    return d


def test_library_exports_every_declared_symbol():
    d = _dopt()
    declared = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        header = open(h).read()
        declared |= set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(dopt_\w+)\s*\(", header, re.M))
    assert len(declared) >= 25 and "dopt_vmm_map" in declared and "dopt_check_grads_noalloc" in declared
    lib = ctypes.CDLL(d.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} not exported"
    assert declared == set(d.EXPORTED)


def _compare(params, N, r, bucket_size, busbw=0):
    d = _dopt()
    A = d.dopt_build_ranges(params, N, r, bucket_size, busbw)
    B = oracle.Layout(params, N, r, bucket_size, busbw)
    assert A.num_buffers == B.num_buffers
    state = 0
    for k in range(A.num_buffers):
        a, b = A.buffer(k), B.buffer(k)
        for key in ("param_dtype", "grad_dtype", "n_buckets", "n_params", "numel", "numel_unpadded",
                    "window_numel", "shard_numel"):
            assert a[key] == b[key], (k, key)
        assert a["arena_numel"] % d.DOPT_ARENA_ALIGN == 0 and a["arena_numel"] >= a["window_numel"]
        state += a["shard_numel"]
        for bi in range(a["n_buckets"]):
            x, y = A.bucket(k, bi), B.bucket(k, bi)
            assert (x["offset"], x["numel"], x["numel_unpadded"], x["shard_size"], x["window_start"],
                    x["arena_offset"], x["n_params"]) == \
                   (y["offset"], y["numel"], y["numel_unpadded"], y["shard"], y["window_start"],
                    y["arena_offset"], y["n_params"])
            for rr in {0, r, N - 1}:
                assert A.rank_window(k, bi, rr) == (y["offset"] + rr * y["shard"],
                                                    y["offset"] + (rr + 1) * y["shard"])
    assert A.state_numel == state
    for p in range(len(params)):
        x, y = A.param(p), B.param(p)
        for key in ("buffer", "bucket", "start", "end", "has_shard", "hgroup", "arena_offset"):
            assert x[key] == y[key], (p, key)
        if x["has_shard"]:
            for key in ("gbuf_world", "gbuf_world_in_bucket", "gbuf_local", "param"):
                assert x[key] == y[key], (p, key)
        else:
            assert x["export_offset"] == -1
    # model-space export offsets: the oracle's shards in model order, back to back
    for p, _, _, _, _, xoff in shard_pieces(B, len(params)):
        assert A.param(p)["export_offset"] == xoff, p
    for kind in oracle.GROUP_KINDS:
        for h in range(3):
            assert A.group(kind, h) == B.group(kind, h)
    return A


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_mapper_matches_oracle_on_workloads(name):
    w = WORKLOADS[name]
    params = PARAM_LISTS[w.model]()
    A = _compare(params, w.dp_size, w.dp_rank, w.bucket_size, w.pad_for_high_busbw)
    assert A.workspace_bytes > 0


@pytest.mark.parametrize("seed", range(30))
def test_mapper_matches_oracle_random(seed):
    rng = random.Random(1000 + seed)
    N = rng.choice([1, 2, 3, 4, 8, 64, 96, 128, 256])
    dts = [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16"), ("f32", "f32"), ("f16", "f32")]
    params = [ParamSpec(f"p{i}", rng.randint(1, 5000), *rng.choice(dts[: rng.randint(1, 5)]),
                        int(rng.random() < 0.1), rng.randint(0, 2)) for i in range(rng.randint(1, 40))]
    bucket_size = rng.choice([0, 1, 700, 5000, 20000])
    for r in sorted({0, rng.randrange(N), N - 1}):
        _compare(params, N, r, bucket_size, int(seed % 5 == 0))


def test_mapper_errors():
    d = _dopt()
    ok = [ParamSpec("a", 10, "bf16", "bf16")]
    with pytest.raises(d.DoptError) as e:
        d.dopt_build_ranges(ok, 4, 4)
    assert e.value.code == -1
    with pytest.raises(d.DoptError):
        d.dopt_build_ranges(ok, 0, 0)
    with pytest.raises(d.DoptError):
        d.dopt_build_ranges([ParamSpec("z", 0, "bf16", "bf16")], 1, 0)
    with pytest.raises(d.DoptError):
        d.dopt_build_ranges([ParamSpec("z", 5, "bf16", "bf16", 0, 16)], 1, 0)
    # element counts that would overflow the padded 64-bit offsets
    for big in ([ParamSpec("h", 1 << 62, "bf16", "bf16")],
                [ParamSpec("h", 3 << 50, "bf16", "bf16"), ParamSpec("i", 3 << 50, "f32", "f32")]):
        with pytest.raises(d.DoptError) as e:
            d.dopt_build_ranges(big, 8, 0)
        assert e.value.code == -1
    L = d.dopt_build_ranges(ok, 2, 1)
    with pytest.raises(d.DoptError) as e:
        L.buffer(3)
    assert e.value.code == -5
    with pytest.raises(d.DoptError):
        L.param(1)


def test_workload_sizes_are_one_gpu_shares():
    # state + windows of every workload fit one MI355X (288 GB HBM)
    d = _dopt()
    for name, w in WORKLOADS.items():
        A = d.dopt_build_ranges(PARAM_LISTS[w.model](), w.dp_size, w.dp_rank, w.bucket_size)
        tot = 0
        for k in range(A.num_buffers):
            b = A.buffer(k)
            es = {0: 4, 1: 2, 2: 2}
            n = b["arena_numel"]
            tot += n * (es[b["grad_dtype"]] + es[b["param_dtype"]] + 8 + (4 if b["param_dtype"] else 0))
        assert tot < 200e9, name


@pytest.mark.parametrize("N,I,r", [(16, 2, 11), (64, 8, 37), (8, 8, 5), (12, 3, 7)])
def test_mapper_matches_oracle_with_instances(N, I, r):
    d = _dopt()
    params = PARAM_LISTS["gpt2-small"]()
    A = d.dopt_build_ranges(params, N, r, 40_000_000, 0, I)
    B = oracle.Layout(params, N, r, 40_000_000, 0, I)
    per = N // I
    assert A.sharding() == {"dp_size": N, "dp_rank": r, "num_instances": I, "instance_size": per,
                            "instance_index": r // per, "instance_rank": r % per}
    for k in range(A.num_buffers):
        a, b = A.buffer(k), B.buffer(k)
        for key in ("numel", "numel_unpadded", "window_numel", "shard_numel", "n_buckets"):
            assert a[key] == b[key]
        for bi in range(a["n_buckets"]):
            x, y = A.bucket(k, bi), B.bucket(k, bi)
            assert (x["window_start"], x["shard_size"], x["arena_offset"]) == \
                   (y["window_start"], y["shard"], y["arena_offset"])
    for p in range(len(params)):
        x, y = A.param(p), B.param(p)
        assert (x["has_shard"], x["arena_offset"], x["param"]) == (y["has_shard"], y["arena_offset"], y["param"])
    with pytest.raises(d.DoptError):
        d.dopt_build_ranges(params, 10, 0, 0, 0, 3)
