"""The Python binding refuses, before any library call, device arrays that do
not match the layout: a wrong element type, too few elements, a
non-contiguous view, a host tensor, a missing array, a workspace that is too
small, tensors marshalled for another layout.  The C library receives bare
pointers and cannot check sizes itself, so a short array would make its
kernels read or write past its end.  Runs on the CPU: every check fires
before anything touches a device."""
import pytest
import torch

import sharded_mixed_precision_amd as D
from synth.models import ParamSpec

PARAMS = [ParamSpec("w", 5000, "bf16", "f32"), ParamSpec("n", 300, "f32", "f32"), ParamSpec("h", 7000, "f16", "f16")]


@pytest.fixture(scope="module")
def L():
    return D.dopt_build_ranges(PARAMS, 4, 1, 0)


T = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _bufs(L, **override):
    """Raw device addresses (which pass: their size is the caller's to
    guarantee) for every array, with the given entries replaced."""
    out = []
    for inf in L.infos():
        out.append({"grad": 4096, "param": 4096, "master": 4096 if inf["pd"] != "f32" else None,
                    "exp_avg": 4096, "exp_avg_sq": 4096})
    for key, val in override.items():
        k, name = key.split("_", 1)
        out[int(k[1:])][name] = val
    return out


def _err(fn, *words):
    with pytest.raises(D.DoptError) as e:
        fn()
    for w in words:
        assert w in str(e.value), str(e.value)
    assert e.value.code == -1 or e.value.code == -5


def test_layout_infos(L):
    inf = L.infos()
    assert [(i["pd"], i["gd"]) for i in inf] == [("bf16", "f32"), ("f32", "f32"), ("f16", "f16")]
    assert all(i["arena_numel"] % D.DOPT_ARENA_ALIGN == 0 for i in inf)


def test_host_tensors_of_the_right_shape_are_refused_as_host_memory(L):
    inf = L.infos()[2]
    n = inf["arena_numel"]
    _err(lambda: D.tensors(L, _bufs(L, b2_grad=torch.zeros(n, dtype=torch.float16))), "buffer 2 grad",
         "not a device tensor")
    _err(lambda: D.tensors(L, _bufs(L, b2_master=torch.zeros(n))), "buffer 2 master", "not a device tensor")
    D.tensors(L, _bufs(L))


def test_wrong_dtype(L):
    n = L.infos()[0]["arena_numel"]
    _err(lambda: D.tensors(L, _bufs(L, b0_grad=torch.zeros(n, dtype=torch.bfloat16))), "buffer 0 grad", "dtype")
    _err(lambda: D.tensors(L, _bufs(L, b2_param=torch.zeros(n, dtype=torch.bfloat16))), "buffer 2 param", "dtype")
    _err(lambda: D.tensors(L, _bufs(L, b0_exp_avg=torch.zeros(n, dtype=torch.float64))), "exp_avg", "dtype")


def test_too_short(L):
    n = L.infos()[1]["arena_numel"]
    _err(lambda: D.tensors(L, _bufs(L, b1_exp_avg_sq=torch.zeros(n - 1))), "buffer 1 exp_avg_sq", "at least")
    _err(lambda: D.tensors(L, _bufs(L, b0_master=torch.zeros(10))), "buffer 0 master", "at least")


def test_non_contiguous(L):
    n = L.infos()[0]["arena_numel"]
    strided = torch.zeros(2 * n)[::2]
    _err(lambda: D.tensors(L, _bufs(L, b0_exp_avg=strided)), "not contiguous")


def test_missing_arrays_and_buffer_count(L):
    _err(lambda: D.tensors(L, _bufs(L, b0_master=None)), "buffer 0 master", "missing")
    _err(lambda: D.tensors(L, _bufs(L, b2_grad=None)), "buffer 2 grad", "missing")
    _err(lambda: D.tensors(L, _bufs(L)[:2]), "2 buffer entries")
    # fp32 params are their own master: none is needed there
    D.tensors(L, _bufs(L, b1_master=None))


def test_workspace_and_marshalled_tensors(L):
    raw = _bufs(L)
    t = D.tensors(L, raw)
    small_ws = torch.zeros(L.workspace_bytes - 1, dtype=torch.uint8)
    _err(lambda: D.dopt_step_apply(L, t, small_ws), "workspace", "bytes")
    other = D.dopt_build_ranges(PARAMS, 4, 2, 0)
    _err(lambda: D.dopt_step_apply(other, t, 0), "another layout")
    t_nograd = D.tensors(L, [{**b, "grad": None} for b in raw], need_grad=False)
    _err(lambda: D.dopt_step(L, t_nograd, [(1e-3, 0.9, 0.999, 1e-8, 0.0)], 1.0, 0), "without grads")


def test_bucket_check_needs_the_whole_buffer(L):
    inf = L.infos()[0]
    out = torch.zeros(inf["n_buckets"] * D.BUCKET_CHECK_BYTES, dtype=torch.uint8)
    arena_grad = torch.zeros(inf["arena_numel"], dtype=torch.float32)  # the rank's window, not the buffer
    assert inf["arena_numel"] < inf["numel"]
    _err(lambda: D.dopt_check_grads(L, 0, arena_grad, 1.0, out, 0), "grad buffer", "at least")
    full = torch.zeros(inf["numel"], dtype=torch.float32)
    _err(lambda: D.dopt_check_grads(L, 0, 4096, 1.0, out[:-1], 0), "bucket check output", "bytes")
    _err(lambda: D.dopt_check_grads(L, 3, full, 1.0, out, 0), "out of range")


def test_reduce_chunks_and_exports(L):
    t = D.tensors(L, _bufs(L))
    infos = L.infos()
    ch = [torch.zeros(4 * inf["arena_numel"], dtype=torch.bfloat16) for inf in infos]
    ch[0] = 4096  # a raw address passes
    ch[1] = torch.zeros(3 * infos[1]["arena_numel"], dtype=torch.bfloat16)
    _err(lambda: D.dopt_reduce_prepare(L, t, ch, "bf16", 4, 1.0, None, 1.0, 0), "buffer 1 chunks", "at least")
    _err(lambda: D.dopt_reduce_prepare(L, t, ch[:2], "bf16", 4, 1.0, None, 1.0, 0), "2 chunk buffers")
    n = L.state_numel
    ok, short = torch.zeros(n), torch.zeros(n - 1)
    _err(lambda: D.dopt_state_export(L, t, 4096, short, ok, 0), "export exp_avg", "at least")
    _err(lambda: D.dopt_state_import(L, t, ok.double(), ok, ok, 0), "import master", "dtype")


def test_reduce_chunk_strides(L):
    """A stride below the arena, a chunk buffer too short for its stride, a
    stride list of the wrong length (binding), and a stride whose bytes are
    not a multiple of 256 (the library's own check, reached here with raw
    addresses before anything touches a device)."""
    t = D.tensors(L, _bufs(L))
    infos = L.infos()
    ar = [inf["arena_numel"] for inf in infos]
    raw = [4096] * len(infos)
    _err(lambda: D.dopt_reduce_prepare(L, t, raw, "bf16", 4, 1.0, None, 1.0, 4096, chunk_strides=ar[:2]),
         "2 chunk strides")
    _err(lambda: D.dopt_reduce_prepare(L, t, raw, "bf16", 4, 1.0, None, 1.0, 4096,
                                       chunk_strides=[ar[0], ar[1] - 128, ar[2]]), "buffer 1", "below the arena")
    ch = [torch.zeros(4 * a, dtype=torch.bfloat16) for a in ar]  # back to back: too short for a wider stride
    _err(lambda: D.dopt_reduce_prepare(L, t, ch, "bf16", 4, 1.0, None, 1.0, 4096,
                                       chunk_strides=[ar[0] + 128, ar[1], ar[2]]), "buffer 0 chunks", "at least")
    _err(lambda: D.dopt_reduce_prepare(L, t, raw, "bf16", 4, 1.0, None, 1.0, 4096,
                                       chunk_strides=[ar[0], ar[1], ar[2] + 8]), "buffer 2", "chunk stride",
         "multiple of 256 bytes")
    _err(lambda: D.dopt_reduce_prepare(L, t, raw, "f32", 4, 1.0, None, 1.0, 4096,
                                       chunk_strides=[ar[0] + 32, ar[1], ar[2]]), "buffer 0", "chunk stride")
    _err(lambda: D.dopt_reduce_prepare(L, t, raw, "bf16", 4, 1.0, None, 1.0, 4096,
                                       chunk_strides=[ar[0], (1 << 41), ar[2]]), "buffer 1", "above 2^40")


def test_reduce_chunk_span_beyond_64_bit_offsets():
    """2^22 chunks (one per rank) at a stride of 2^40 bf16 elements would span
    2^63 bytes: the library refuses before forming any chunk offset (raw
    addresses, nothing touches a device)."""
    n = 1 << 22
    Lb = D.dopt_build_ranges([ParamSpec("a", 5000, "bf16", "bf16")], n, 7, 0)
    t = D.tensors(Lb, [{"grad": 4096, "param": 4096, "master": 4096, "exp_avg": 4096, "exp_avg_sq": 4096}])
    _err(lambda: D.dopt_reduce_prepare(Lb, t, [4096], "bf16", n, 1.0, None, 1.0, 4096, chunk_strides=[1 << 40]),
         "buffer 0", f"{n} chunks", "2^62 bytes")


def test_noalloc_check_refuses_buffers_beyond_its_static_scratch():
    # 2^34 elements: 2^20 check tiles of 16 B = 16 MiB of partials plus the
    # bucket table, more than the library's static scratch holds.  The library
    # refuses before any device work (the addresses are never used).
    L = D.dopt_build_ranges([ParamSpec("huge", 1 << 34, "bf16", "bf16")], 1024, 0, 0)
    _err(lambda: D.dopt_check_grads_noalloc(L, 0, 1 << 20, 1.0, 1 << 21), "scratch", "16777216")
    assert D.NOALLOC_SCRATCH_BYTES == 16 << 20
    _err(lambda: D.dopt_check_grads_noalloc(L, 1, 1 << 20, 1.0, 1 << 21), "out of range")


def test_vmm_wrappers_report_hip_errors_as_dopt_errors():
    # the placement helpers of dopt_vmm.h return the library's error codes; a
    # bad handle or an empty size is refused before HIP is reached, and on a
    # machine without a GPU the HIP calls themselves fail cleanly
    with pytest.raises(D.DoptError) as e:
        D.dopt_vmm_reserve(0)
    assert e.value.code == -1 and "zero size" in str(e.value)
    with pytest.raises(D.DoptError) as e:
        D.dopt_vmm_create(0)
    assert e.value.code == -1
    if not torch.cuda.is_available():
        with pytest.raises(D.DoptError) as e:
            D.dopt_vmm_granularity(0)
        assert e.value.code == -4 and "hipMemGetAllocationGranularity" in str(e.value)


@pytest.mark.parametrize("cfg", [
    dict(initial_scale=float("inf")), dict(initial_scale=float("nan")), dict(initial_scale=1e-320),
    dict(initial_scale=1e50), dict(dynamic=True, growth_factor=float("inf")), dict(dynamic=True, min_scale=1e-320),
], ids=["inf", "nan", "reciprocal-inf", "reciprocal-zero", "growth-inf", "min-scale-reciprocal-inf"])
def test_init_state_refuses_scales_without_a_usable_reciprocal(L, cfg):
    """Every grad is unscaled by 1/scale in fp32: a scale that is not finite,
    or whose fp32 reciprocal is infinite or zero, is refused before anything
    touches a device (raw addresses)."""
    _err(lambda: D.dopt_init_state(L, D.tensors(L, _bufs(L)), D.scaler_cfg(**cfg), 4096), "scale")


@pytest.mark.parametrize("scale", [float("inf"), 0.0, 1e50, 1e-320])
def test_scalar_set_refuses_scales_without_a_usable_reciprocal(L, scale):
    _err(lambda: D.dopt_state_scalars_set(L, 4096, {"step_count": 3, "loss_scale": scale, "growth_tracker": 0,
                                                    "hysteresis_tracker": 1}), "loss_scale", "finite")
