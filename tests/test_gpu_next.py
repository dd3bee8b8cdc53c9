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


@pytest.mark.timeout(600)
def test_reduce_llama3_8b_sampled():
    # the Llama-3-8B rank (N=8, r=5, ~1.0e9 fp32 grad slots): 8 bf16 chunks per slot
    case = H.case_from_workload(synth.WORKLOADS["llama3-8b"])
    case.name, case.steps, case.chunks, case.wire = "reduce-llama3-8b", 2, 8, "bf16"
    H.run_sampled(case)


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
        D.dopt_reduce_prepare(L2, A2.bufs, [torch.zeros(2 * A2.info[0]["n"], dtype=torch.bfloat16, device="cuda")],
                              "bf16", 4, 1.0, hp, 1.0, A2.workspace, stream)
