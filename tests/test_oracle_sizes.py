"""The oracle's layout of the five workloads at their real sizes.

The expected figures were derived on their own from the bucketing rules of
"Megatron-LM distrib_optimizer.py 源码精读" -- sections "Bucket 划分算法：逆序
遍历 + 尺寸触发" (last param first, 64-element starts, a bucket closes once it
holds at least bucket_size elements), "两级 Padding 机制" (bucket ends padded
to lcm(N, 128), or lcm(N, 128, 2^16) for bus bandwidth) and "Bucket 级别的均等
切分" (rank r owns the r-th of N equal parts of each bucket) -- applied to the
param lists by hand arithmetic, with the bucket size max(40M, 1M * N) of
"Megatron-LM distributed 包深度解析" §2.2 where a workload states none.  They
are not produced by the oracle; the test checks that the oracle reproduces
them.  The model totals are the public parameter counts of the architectures
the lists are shaped after (GPT-2 small 124,439,808; Llama-3-8B
8,030,261,248; the 32-layer 4096-wide 7B 6,738,415,616; Llama-3-70B
70,553,706,496).

Two of the sizes pin the order of params inside a transformer layer: with
the norms registered in forward order (input norm before attention,
post-attention norm before the MLP) the dense 7B list's largest bucket is
the embedding plus layer 0's query projection and input norm, 147,853,312
elements; with both norms after the MLP it would be 4,096 elements smaller.
"""
import pytest

import oracle
import synth

# name -> per buffer: (total params P, buffer numel (= unpadded here), buckets,
#                      smallest bucket, largest bucket, rank window E,
#                      rank segments, segments that cut a param)
TABLE = {
    "tiny": [(2_608, 2_688, 1, 2_688, 2_688, 672, 1, 1)],
    "gpt2-small": [(124_439_808, 124_439_808, 3, 40_163_328, 44_111_616, 15_554_976, 17, 5)],
    "llama3-8b": [(8_029_995_008, 8_029_995_008, 130, 41_943_040, 525_336_576, 1_003_749_376, 130, 130),
                  (266_240, 266_240, 1, 266_240, 266_240, 33_280, 9, 2)],
    "dense-7b": [(6_738_415_616, 6_738_415_616, 130, 45_088_768, 147_853_312, 6_738_415_616, 291, 0)],
    "llama3-70b": [(70_553_706_496, 70_553_706_496, 402, 67_117_056, 1_050_681_344, 1_102_401_664, 402, 402)],
}
PUBLIC_TOTALS = {"gpt2-small": 124_439_808, "llama3-8b": 8_030_261_248, "dense-7b": 6_738_415_616,
                 "llama3-70b": 70_553_706_496}


def _sizes(L, params, k):
    b = L.buffer(k)
    bk = [L.bucket(k, i) for i in range(b["n_buckets"])]
    s, ln, pr = L.segments(k)
    cuts = sum(1 for p in pr.tolist() if L.param(p)["param"] != (0, params[p].numel))
    P = sum(params[i].numel for i in range(len(params)) if L.param(i)["buffer"] == k)
    assert b["numel_unpadded"] == b["numel"]
    assert b["window_numel"] == b["shard_numel"]  # no gaps or padding inside these windows
    assert {x["window_start"] % 8 for x in bk} == {0}
    return (P, b["numel"], b["n_buckets"], min(x["numel"] for x in bk), max(x["numel"] for x in bk),
            b["window_numel"], len(s), cuts)


@pytest.mark.parametrize("name", list(TABLE))
def test_workload_sizes(name):
    w = synth.WORKLOADS[name]
    params = synth.PARAM_LISTS[w.model]()
    L = oracle.Layout(params, w.dp_size, w.dp_rank, w.bucket_size, w.pad_for_high_busbw)
    assert L.num_buffers == len(TABLE[name])
    for k, row in enumerate(TABLE[name]):
        assert _sizes(L, params, k) == row, (name, k)
    if name in PUBLIC_TOTALS:
        assert sum(p.numel for p in params) == PUBLIC_TOTALS[name]
    # the ledger: the rank's optimizer state covers its window's param elements
    assert sum(L.buffer(k)["shard_numel"] for k in range(L.num_buffers)) == sum(r[5] for r in TABLE[name])


def test_llama70b_with_bus_bandwidth_padding():
    # not a workload: the same rank with bucket ends padded to lcm(64, 128, 2^16)
    w = synth.WORKLOADS["llama3-70b"]
    params = synth.PARAM_LISTS[w.model]()
    L = oracle.Layout(params, w.dp_size, w.dp_rank, w.bucket_size, 1)
    b = L.buffer(0)
    assert (b["numel"], b["numel_unpadded"], b["n_buckets"], b["window_numel"]) == \
        (70_562_938_880, 70_553_706_496, 402, 1_102_545_920)
    assert all(L.bucket(0, i)["numel"] % 65536 == 0 for i in range(b["n_buckets"]))


def test_gpt2_bucket_membership():
    # bucket 0 = {ln_f ... layer-6 fc}, 1 = {layer-6 ln_2.b ... layer-0 mlp proj}, 2 = {layer-0 fc.b ... wte}
    w = synth.WORKLOADS["gpt2-small"]
    params = synth.PARAM_LISTS[w.model]()
    L = oracle.Layout(params, w.dp_size, w.dp_rank, w.bucket_size)
    ends = []
    for b in range(3):
        idx = [i for i in range(len(params)) if L.param(i)["bucket"] == b]
        ends.append((params[idx[-1]].name, params[idx[0]].name, len(idx)))
    assert ends == [("ln_f.b", "h6.mlp.c_fc.w", 66), ("h6.ln_2.b", "h0.mlp.c_proj.w", 70),
                    ("h0.mlp.c_fc.b", "wte", 12)]


def test_tiny_all_ranks():
    # r0 = b1[0,16) + w1[0,512) + b0[0,32) + w0[0,32); r1 = w0[32,704);
    # r2 = w0[704,1376); r3 = w0[1376,2048)
    params = synth.PARAM_LISTS["tiny"]()
    want = [{"w0": (0, 32), "b0": (0, 32), "w1": (0, 512), "b1": (0, 16)}, {"w0": (32, 704)},
            {"w0": (704, 1376)}, {"w0": (1376, 2048)}]
    for r in range(4):
        L = oracle.Layout(params, 4, r, 0)
        got = {params[i].name: L.param(i)["param"] for i in range(4) if L.param(i)["has_shard"]}
        assert got == want[r]
