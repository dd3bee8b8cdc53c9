"""The allocation-free bucket check, dopt_check_grads_noalloc, called through
the C ABI and compared with the workspace entry point dopt_check_grads on the
same device buffers, on two calls in a row, the second with a smaller input
(fewer buckets and check tiles, so stale partials of the first call would
show), and both with the oracle.  The noalloc output starts filled with 0xff
bytes, so every record must be written."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.models import ParamSpec
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _check_layout(name, params, N, r, bucket, thr, injections=()):
    import sharded_mixed_precision_amd as D
    from sharded_mixed_precision_amd.arena import DeviceArenas

    H.log(f"[noalloc] {name}: N={N} r={r} bucket={bucket}")
    L = D.dopt_build_ranges(params, N, r, bucket)
    O = oracle.Layout(params, N, r, bucket)
    A = DeviceArenas(L)
    stream = torch.cuda.current_stream()
    D.dopt_init_state(L, A.bufs, D.scaler_cfg(), A.workspace, stream)
    sizes = []
    for k, info in enumerate(L.infos()):
        n, nb = info["numel"], info["n_buckets"]
        host = synth.fill_normal(info["gd"], n, 0, synth.local_grad_stream(k), 1, 1e-2,
                                 out=torch.empty(n, dtype=synth.torch_dtype(info["gd"]), pin_memory=True))
        for kk, i, val in injections:
            if kk == k:
                host[i] = val
        dev = host.to("cuda")
        out_ws = torch.zeros(nb * D.BUCKET_CHECK_BYTES, dtype=torch.uint8, device="cuda")
        out_na = torch.full((nb * D.BUCKET_CHECK_BYTES,), 0xFF, dtype=torch.uint8, device="cuda")
        D.dopt_check_grads(L, k, dev, thr, out_ws, A.workspace, stream)
        D.dopt_check_grads_noalloc(L, k, dev, thr, out_na, stream)
        a, b = out_ws.cpu().numpy(), out_na.cpu().numpy()
        assert np.array_equal(a, b), f"{name} buffer {k}: noalloc records differ from the workspace entry point"
        got = D.bucket_checks(b.tobytes(), nb)
        H.check_bucket_results(got, H.oracle_check_parallel(O, k, host, thr), f"{name} buffer {k}")
        sizes.append((nb, -(-n // 16384)))
    H.log(f"[noalloc] {name}: buckets and check tiles {sizes} equal to dopt_check_grads and the oracle")
    return sizes


def test_noalloc_check_equals_workspace_check_twice_second_smaller():
    w = synth.WORKLOADS["gpt2-small"]
    p = synth.PARAM_LISTS[w.model]()
    first = _check_layout("gpt2-small", p, w.dp_size, w.dp_rank, w.bucket_size, 0.1,
                          injections=[(0, 45_000_000, float("nan")), (0, 100_000_000, 0.5),
                                      (0, 3, float("-inf"))])
    params = [ParamSpec("a", 70001, "bf16", "f32"), ParamSpec("b", 129, "f32", "f32"),
              ParamSpec("c", 33333, "f16", "f16"), ParamSpec("d", 5, "bf16", "f32")]
    second = _check_layout("mixed-small", params, 3, 2, 20_000, 0.03, injections=[(2, 17, float("inf"))])
    assert sum(t for _, t in second) < sum(t for _, t in first)  # the second input is the smaller

