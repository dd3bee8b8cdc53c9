"""GPU parity for the rows next to the step: the fused local fp32-accumulating
reduce + pass 1 ("Megatron-LM distributed 包深度解析…" §3.2,
reduce_scatter_with_fp32_accumulation) and hierarchical optimizer instances
("02 · ZeRO 显存账本…" §5) are covered here and in test_gpu_parity.py."""
import pytest
import torch

import synth
from synth.models import ParamSpec, gpt2_small
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    H.log(f"[gpu-test] start {request.node.name}")
    yield
    torch.cuda.synchronize()


def test_reduce_fp32_grads_gpt2_small_full():
    # bf16 on the wire, 8 chunks, fp32 grad buffer (grad_reduce_in_fp32): every
    # reduced slot and every state element compared after each step
    case = H.Case("reduce-gpt2", gpt2_small("bf16", "f32"), 8, 3, 40_000_000, steps=3, grad_sigma=1e-3,
                  chunks=8, wire="bf16")
    rep = H.run_full(case)
    assert rep[-1]["param0"]["n"] == 15_554_976


def test_reduce_bf16_grads_split_scaled():
    # fp16 on the wire, average by 1/N after the fp32 sum, bf16 grad buffer,
    # stats-only call followed by the separate finalize (the cross-rank seam)
    params = [ParamSpec(f"p{i}", n, "bf16", "bf16", 0, i % 2) for i, n in enumerate([70000, 333, 4097, 129, 20000])]
    hps = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (5e-4, 0.9, 0.99, 1e-8, 0.0)]
    case = H.Case("reduce-split", params, 4, 1, 6000, steps=3, grad_sigma=1e-2, hparams=hps, chunks=4, wire="f16",
                  reduce_scale=0.25, reduce_split=True)
    H.run_full(case)


def test_reduce_mixed_buffers_odd_windows():
    params = [ParamSpec("a", 50000, "bf16", "f32"), ParamSpec("n", 300, "f32", "f32"), ParamSpec("b", 777, "bf16", "f32")]
    H.run_full(H.Case("reduce-mixed", params, 128, 77, 0, steps=2, chunks=128, wire="bf16"))


@pytest.mark.parametrize("wire,pad", [("bf16", 384), ("f32", 2048 + 64)], ids=["bf16", "f32"])
def test_reduce_padded_chunk_stride(wire, pad):
    """Chunks received at a stride wider than the arena (a caller's receive
    buffer with room between chunks), the gaps filled with NaN: the reduced
    grads, the statistics and the step after them match the oracle reading
    the same buffer at the same stride, so no gap slot is read."""
    params = [ParamSpec("a", 50000, "bf16", "f32"), ParamSpec("n", 300, "f32", "f32"),
              ParamSpec("b", 7777, "f16", "f16", 0, 1)]
    hps = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (5e-4, 0.9, 0.99, 1e-8, 0.0)]
    H.run_full(H.Case(f"reduce-stride-{wire}", params, 4, 1, 0, steps=2, hparams=hps, chunks=4, wire=wire,
                      chunk_pad=pad))


@pytest.mark.timeout(600)
def test_reduce_padded_chunk_stride_large_window():
    """A 70M-slot window (several range launches of the reduce) with its 2
    chunks 2176 slots apart beyond the arena, every slot compared."""
    import sharded_mixed_precision_amd as D
    params = [ParamSpec("w", 139_999_991, "bf16", "f32"), ParamSpec("x", 777, "bf16", "f32")]
    L = D.dopt_build_ranges(params, 2, 1, 0)
    assert L.buffer(0)["arena_numel"] // D.DOPT_ARENA_ALIGN > 32768
    H.run_full(H.Case("reduce-stride-large", params, 2, 1, 0, steps=2, chunks=2, wire="bf16", chunk_pad=2176))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n,wire", [(1, "bf16"), (3, "bf16"), (3, "f32"), (3, "f16")],
                         ids=["1-bf16", "3-bf16", "3-f32", "3-f16"])
def test_reduce_large_window_odd_chunk_counts(n, wire):
    """A window past the one-tile-per-workgroup grid (the large-window reduce,
    which issues its chunk loads two at a time) reduced from an odd number of
    chunks, so that the last chunk is loaded alone (with one chunk, every
    one); every slot compared."""
    import sharded_mixed_precision_amd as D
    params = [ParamSpec("w", 59_999_989, "bf16", "f32"), ParamSpec("x", 4097, "bf16", "f32")]
    r = n // 2
    L = D.dopt_build_ranges(params, n, r, 0)
    assert L.buffer(0)["arena_numel"] // D.DOPT_ARENA_ALIGN > 8192
    H.run_full(H.Case(f"reduce-odd-{n}-{wire}", params, n, r, 0, steps=2, chunks=n, wire=wire))


@pytest.mark.timeout(600)
def test_reduce_llama3_8b_sampled():
    # the Llama-3-8B rank (N=8, r=5, ~1.0e9 fp32 grad slots): 8 bf16 chunks per slot
    case = H.case_from_workload(synth.WORKLOADS["llama3-8b"])
    case.name, case.steps, case.chunks, case.wire = "reduce-llama3-8b", 2, 8, "bf16"
    H.run_sampled(case)


def test_check_gpt2_small_buffer_with_injections():
    # the whole local bf16 grad buffer of the GPT-2-small rank (124,439,808
    # elements, 3 buckets): a NaN in bucket 1, an infinity in bucket 2, a large
    # value in bucket 0, NaN and infinity together in a second case
    case = H.case_from_workload(synth.WORKLOADS["gpt2-small"])
    case.grad_sigma = 1e-3
    from sharded_mixed_precision_amd import dopt_build_ranges
    L = dopt_build_ranges(case.params, case.dp_size, case.dp_rank, case.bucket_size)
    off = [L.bucket(0, b)["offset"] for b in range(3)]
    res = H.run_check(case, 0.5, [(0, off[0] + 12345, 3.0), (0, off[1] + 777, float("nan")),
                                  (0, off[2] + 5, float("-inf"))])[0]
    assert [(r["has_nan"], r["has_inf"], r["large"]) for r in res] == [(0, 0, 1), (1, 0, 0), (0, 1, 1)]
    res = H.run_check(case, 0.0, [(0, off[1] + 1, float("nan")), (0, off[1] + 2, float("inf"))])[0]
    assert [(r["has_nan"], r["has_inf"], r["large"]) for r in res] == [(0, 0, 0), (1, 1, 0), (0, 0, 0)]


def test_check_mixed_buffers_odd_sizes():
    params = [ParamSpec("a", 50000, "bf16", "f32"), ParamSpec("n", 300, "f32", "f32"),
              ParamSpec("h", 70001, "f16", "f16"), ParamSpec("b", 777, "bf16", "f32")]
    H.run_check(H.Case("check-mixed", params, 96, 5, 20000, grad_sigma=1.0), 3.0)


@pytest.mark.timeout(600)
def test_check_dense_7b_buffer():
    # the whole fp16 buffer of the dense 7B model (6,738,415,616 elements, 130 buckets)
    case = H.case_from_workload(synth.WORKLOADS["dense-7b"])
    res = H.run_check(case, 4.0e-3, [(0, 123_456_789, float("inf"))])[0]
    assert len(res) == 130 and sum(r["has_inf"] for r in res) == 1


def test_reduce_argument_errors():
    import sharded_mixed_precision_amd as D
    from sharded_mixed_precision_amd.arena import DeviceArenas
    params = [ParamSpec("a", 5000, "bf16", "f32")]
    hp = [(1e-3, 0.9, 0.999, 1e-8, 0.0)]
    stream = torch.cuda.current_stream()
    L = D.dopt_build_ranges(params, 4, 1)
    A = DeviceArenas(L)
    D.dopt_init_state(L, A.bufs, D.scaler_cfg(), A.workspace, stream)
    ch = [torch.zeros(4 * A.info[0]["n"], dtype=torch.bfloat16, device="cuda")]
    with pytest.raises(D.DoptError):  # one chunk per rank is required
        D.dopt_reduce_prepare(L, A.bufs, ch, "bf16", 3, 1.0, hp, 1.0, A.workspace, stream)
    L2 = D.dopt_build_ranges(params, 4, 1, 0, 0, 2)
    A2 = DeviceArenas(L2)
    D.dopt_init_state(L2, A2.bufs, D.scaler_cfg(), A2.workspace, stream)
    with pytest.raises(D.DoptError):  # not with more than one optimizer instance
        D.dopt_reduce_prepare(L2, A2.bufs, [torch.zeros(4 * A2.info[0]["n"], dtype=torch.bfloat16, device="cuda")],
                              "bf16", 4, 1.0, hp, 1.0, A2.workspace, stream)
