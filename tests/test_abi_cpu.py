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


def _expected_apply_bnd(B, k) -> int:
    """From the oracle's segments: a window of more than 16384 2048-element
    tiles (pass 2 grid-strides over it) in which some tile is not covered by
    one segment (params meeting inside it, a gap, the ragged tail)."""
    s, ln, _ = B.segments(k)
    tiles = -(-B.buffer(k)["window_numel"] // 2048)
    full = sum(max(0, (e // 2048) - (-(-a // 2048))) for a, e in zip(s.tolist(), (s + ln).tolist()))
    return int(tiles > 16384 and full < tiles)


@pytest.mark.parametrize("case", ["workloads", "boundary-layouts"])
def test_pass2_kernel_choice_follows_the_tiles(case):
    """dopt_buffer_info.apply_bnd (pass 2 in k_apply_bnd) is set exactly for
    grid-stride windows that hold a boundary tile: the Llama-3-70B rank, whose
    windows all cut params, and not dense-7B or Llama-3-8B (whose shards fill
    their tiles) or the small windows."""
    d = _dopt()
    if case == "workloads":
        layouts = [(PARAM_LISTS[w.model](), w.dp_size, w.dp_rank, w.bucket_size, w.pad_for_high_busbw)
                   for w in WORKLOADS.values()]
    else:
        sizes = [(20_000_003, 0), (3_000_001, 0), (9_999_999, 1), (7_000_001, 2), (333, 2)]
        layouts = []
        for n, r, scale in ((1, 0, 1), (2, 1, 2), (1, 0, 0.5)):  # the last: 19.5M slots, one tile per workgroup
            params = [ParamSpec(f"p{i}", int(k * scale), "bf16", "bf16", 0, hg) for i, (k, hg) in enumerate(sizes)]
            layouts.append((params, n, r, 0, 0))
    got = []
    for params, N, r, bucket_size, busbw in layouts:
        A = d.dopt_build_ranges(params, N, r, bucket_size, busbw)
        B = oracle.Layout(params, N, r, bucket_size, busbw)
        for k in range(A.num_buffers):
            assert A.buffer(k)["apply_bnd"] == _expected_apply_bnd(B, k), (len(params), N, r, k)
            got.append(A.buffer(k)["apply_bnd"])
    if case == "workloads":
        # tiny, gpt2-small, llama3-8b (two buffers), dense-7b, llama3-70b
        assert got == [0, 0, 0, 0, 0, 1], got
    else:
        assert got == [1, 1, 0], got


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
    # padding alone past the 64-bit range: 9000 one-param buckets (bucket_size
    # 1), each padded to a multiple of (2^31 - 1) * 2^16 elements (an odd
    # dp_size with the high-busbw padding), is 1.27e18 > 2^60 padded elements
    many = [ParamSpec(f"p{i}", 128, "bf16", "bf16") for i in range(9000)]
    with pytest.raises(d.DoptError) as e:
        d.dopt_build_ranges(many, (1 << 31) - 1, 5, 1, 1)
    assert e.value.code == -1 and "2^60" in str(e.value)
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
