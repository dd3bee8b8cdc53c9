"""Python binding of libdopt.so, the shard-local mixed-precision AdamW step
of a ZeRO-1 distributed optimizer for AMD Instinct MI355X (gfx950).

Argument marshalling only: every computation happens in the library (host
range mapper in C++, the step in HIP kernels).  Function names match the C
ABI in include/dopt.h.  Device buffers may be given as PyTorch CUDA tensors
or raw integer addresses; PyTorch is used only to own device memory and
streams.  There is no fallback: if the library is not built, import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdopt.so")

DOPT_F32, DOPT_BF16, DOPT_F16 = 0, 1, 2
DTYPES = {"f32": DOPT_F32, "bf16": DOPT_BF16, "f16": DOPT_F16}
DTYPE_NAMES = {v: k for k, v in DTYPES.items()}
DOPT_SCALER_CONSTANT, DOPT_SCALER_DYNAMIC = 0, 1
GROUP_KINDS = {"model_float16": 0, "model_fp32": 1, "shard_float16": 2, "shard_fp32_from_float16": 3,
               "shard_fp32": 4}
DOPT_MAX_HGROUPS = 16
DOPT_ARENA_ALIGN = 2048
DOPT_PTR_ALIGN = 256


class DoptError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dopt error {code}: {msg}")
        self.code = code


class dopt_param_desc(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("param_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
                ("requires_new_bucket", ctypes.c_int32), ("hgroup", ctypes.c_int32)]


class dopt_shard_cfg(ctypes.Structure):
    _fields_ = [("dp_size", ctypes.c_int32), ("dp_rank", ctypes.c_int32), ("bucket_size", ctypes.c_int64),
                ("pad_for_high_busbw", ctypes.c_int32), ("num_instances", ctypes.c_int32)]


class dopt_sharding_info(ctypes.Structure):
    _fields_ = [("dp_size", ctypes.c_int32), ("dp_rank", ctypes.c_int32), ("num_instances", ctypes.c_int32),
                ("instance_size", ctypes.c_int32), ("instance_index", ctypes.c_int32),
                ("instance_rank", ctypes.c_int32)]


class dopt_range(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("end", ctypes.c_int64)]

    def tuple(self):
        return (self.start, self.end)


class dopt_buffer_info(ctypes.Structure):
    _fields_ = [("param_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32), ("n_buckets", ctypes.c_int32),
                ("n_params", ctypes.c_int32), ("numel", ctypes.c_int64), ("numel_unpadded", ctypes.c_int64),
                ("window_numel", ctypes.c_int64), ("arena_numel", ctypes.c_int64), ("shard_numel", ctypes.c_int64),
                ("apply_bnd", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class dopt_bucket_info(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("numel", ctypes.c_int64), ("numel_unpadded", ctypes.c_int64),
                ("shard_size", ctypes.c_int64), ("window_start", ctypes.c_int64), ("arena_offset", ctypes.c_int64),
                ("n_params", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class dopt_param_info(ctypes.Structure):
    _fields_ = [("buffer", ctypes.c_int32), ("bucket", ctypes.c_int32), ("has_shard", ctypes.c_int32),
                ("hgroup", ctypes.c_int32), ("start", ctypes.c_int64), ("end", ctypes.c_int64),
                ("gbuf_world", dopt_range), ("gbuf_world_in_bucket", dopt_range), ("gbuf_local", dopt_range),
                ("param", dopt_range), ("arena_offset", ctypes.c_int64), ("export_offset", ctypes.c_int64)]


class dopt_buffer_tensors(ctypes.Structure):
    _fields_ = [("grad", ctypes.c_void_p), ("param", ctypes.c_void_p), ("master", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p)]


class dopt_scaler_cfg(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("hysteresis", ctypes.c_int32), ("growth_interval", ctypes.c_int64),
                ("initial_scale", ctypes.c_double), ("growth_factor", ctypes.c_double),
                ("backoff_factor", ctypes.c_double), ("min_scale", ctypes.c_double)]


class dopt_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


class dopt_state_scalars(ctypes.Structure):
    _fields_ = [("step_count", ctypes.c_int64), ("loss_scale", ctypes.c_double),
                ("growth_tracker", ctypes.c_int64), ("hysteresis_tracker", ctypes.c_int64)]


class dopt_stats(ctypes.Structure):
    _fields_ = [("found_inf", ctypes.c_int32), ("skipped", ctypes.c_int32), ("clip_applied", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("sumsq", ctypes.c_double), ("grad_norm", ctypes.c_double),
                ("clip_coef", ctypes.c_double), ("num_zeros", ctypes.c_uint64), ("loss_scale_used", ctypes.c_double),
                ("loss_scale_next", ctypes.c_double), ("step_count", ctypes.c_int64)]

    def as_dict(self) -> Dict:
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "reserved"}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python sharded_mixed_precision_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, VP, D = ctypes.POINTER, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
    sig = {
        "dopt_build_ranges": ([P(dopt_param_desc), I64, P(dopt_shard_cfg), P(VP)], ctypes.c_int),
        "dopt_layout_free": ([VP], None),
        "dopt_layout_num_buffers": ([VP], I32),
        "dopt_layout_sharding": ([VP, P(dopt_sharding_info)], ctypes.c_int),
        "dopt_layout_buffer": ([VP, I32, P(dopt_buffer_info)], ctypes.c_int),
        "dopt_layout_bucket": ([VP, I32, I32, P(dopt_bucket_info)], ctypes.c_int),
        "dopt_layout_rank_window": ([VP, I32, I32, I32, P(dopt_range)], ctypes.c_int),
        "dopt_layout_param": ([VP, I64, P(dopt_param_info)], ctypes.c_int),
        "dopt_layout_group": ([VP, I32, I32, VP, I64], I64),
        "dopt_layout_state_numel": ([VP], I64),
        "dopt_workspace_bytes": ([VP], I64),
        "dopt_init_state": ([VP, P(dopt_buffer_tensors), P(dopt_scaler_cfg), VP, VP], ctypes.c_int),
        "dopt_step": ([VP, P(dopt_buffer_tensors), P(dopt_hparams), I32, D, VP, VP, P(dopt_stats)], ctypes.c_int),
        "dopt_step_prepare": ([VP, P(dopt_buffer_tensors), P(dopt_hparams), I32, D, VP, VP], ctypes.c_int),
        "dopt_step_stats": ([VP, P(dopt_buffer_tensors), VP, VP], ctypes.c_int),
        "dopt_reduce_prepare": ([VP, P(dopt_buffer_tensors), P(VP), P(I64), I32, I32, ctypes.c_float, P(dopt_hparams),
                                 I32, D, VP, VP], ctypes.c_int),
        "dopt_check_grads": ([VP, I32, VP, D, VP, VP, VP], ctypes.c_int),
        "dopt_check_grads_noalloc": ([VP, I32, VP, D, VP, VP], ctypes.c_int),
        "dopt_step_finalize": ([VP, P(dopt_hparams), I32, D, VP, VP], ctypes.c_int),
        "dopt_step_apply": ([VP, P(dopt_buffer_tensors), VP, VP], ctypes.c_int),
        "dopt_state_export": ([VP, P(dopt_buffer_tensors), VP, VP, VP, VP, VP], ctypes.c_int),
        "dopt_state_import": ([VP, P(dopt_buffer_tensors), VP, VP, VP, VP, VP], ctypes.c_int),
        "dopt_state_scalars_get": ([VP, VP, VP, P(dopt_state_scalars)], ctypes.c_int),
        "dopt_state_scalars_set": ([VP, VP, VP, P(dopt_state_scalars)], ctypes.c_int),
        "dopt_stats_record_offset": ([VP], I64),
        "dopt_read_stats": ([VP, VP, VP, P(dopt_stats)], ctypes.c_int),
        "dopt_last_error": ([], ctypes.c_char_p),
        "dopt_vmm_granularity": ([I32, P(ctypes.c_size_t)], ctypes.c_int),
        "dopt_vmm_reserve": ([ctypes.c_size_t, ctypes.c_size_t, P(ctypes.c_uint64)], ctypes.c_int),
        "dopt_vmm_free": ([ctypes.c_uint64, ctypes.c_size_t], ctypes.c_int),
        "dopt_vmm_create": ([I32, ctypes.c_size_t, P(ctypes.c_uint64)], ctypes.c_int),
        "dopt_vmm_map": ([ctypes.c_uint64, ctypes.c_size_t, ctypes.c_uint64], ctypes.c_int),
        "dopt_vmm_set_access": ([ctypes.c_uint64, ctypes.c_size_t, I32], ctypes.c_int),
        "dopt_vmm_unmap": ([ctypes.c_uint64, ctypes.c_size_t], ctypes.c_int),
        "dopt_vmm_release": ([ctypes.c_uint64], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


_lib = _load()
EXPORTED = ("dopt_build_ranges", "dopt_layout_free", "dopt_layout_num_buffers", "dopt_layout_sharding",
            "dopt_layout_buffer",
            "dopt_layout_bucket", "dopt_layout_rank_window", "dopt_layout_param", "dopt_layout_group",
            "dopt_layout_state_numel", "dopt_workspace_bytes", "dopt_init_state", "dopt_step", "dopt_step_prepare", "dopt_step_stats",
            "dopt_step_finalize", "dopt_step_apply", "dopt_reduce_prepare", "dopt_check_grads",
            "dopt_check_grads_noalloc",
            "dopt_state_export", "dopt_state_import", "dopt_state_scalars_get", "dopt_state_scalars_set",
            "dopt_stats_record_offset",
            "dopt_read_stats",
            "dopt_last_error",
            "dopt_vmm_granularity", "dopt_vmm_reserve", "dopt_vmm_free", "dopt_vmm_create", "dopt_vmm_map",
            "dopt_vmm_set_access", "dopt_vmm_unmap", "dopt_vmm_release")


def lib():
    return _lib


def _check(rc: int):
    if rc != 0:
        raise DoptError(rc, _lib.dopt_last_error().decode())


def _addr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


DOPT_ERR_INVALID = -1
_TORCH_DTYPE_NAMES = {"f32": "torch.float32", "bf16": "torch.bfloat16", "f16": "torch.float16"}


def _dev(x, what: str, dtype: Optional[str] = None, min_numel: int = 0, min_bytes: int = 0) -> int:
    """Device address of ``x`` after checking it against what the library
    will touch: a contiguous device tensor of the given element type holding
    at least ``min_numel`` elements / ``min_bytes`` bytes.  The library cannot
    check sizes itself (it receives bare pointers), and a short buffer would
    make its kernels read or write past the end.  A raw integer address is
    passed through: its size and type are then the caller's to guarantee."""
    if x is None:
        raise DoptError(DOPT_ERR_INVALID, f"{what}: missing")
    if isinstance(x, int):
        return x
    if dtype is not None and str(x.dtype) != _TORCH_DTYPE_NAMES[dtype]:
        raise DoptError(DOPT_ERR_INVALID, f"{what}: dtype {x.dtype}, the layout needs {_TORCH_DTYPE_NAMES[dtype]}")
    if x.numel() < min_numel:
        raise DoptError(DOPT_ERR_INVALID, f"{what}: {x.numel()} elements, the layout needs at least {min_numel}")
    if x.numel() * x.element_size() < min_bytes:
        raise DoptError(DOPT_ERR_INVALID,
                        f"{what}: {x.numel() * x.element_size()} bytes, the layout needs at least {min_bytes}")
    if not x.is_contiguous():
        raise DoptError(DOPT_ERR_INVALID, f"{what}: not contiguous")
    if not getattr(x, "is_cuda", False):
        raise DoptError(DOPT_ERR_INVALID, f"{what}: not a device tensor")
    return x.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


class Layout:
    """Owns a dopt_layout handle (freed with the object)."""

    def __init__(self, handle: ctypes.c_void_p, dp_size: int, dp_rank: int, n_params: int):
        self._h = handle
        self._free = _lib.dopt_layout_free  # kept so that freeing works during interpreter shutdown
        self.dp_size, self.dp_rank, self.n_params = dp_size, dp_rank, n_params

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None:
            self._free(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    @property
    def num_buffers(self) -> int:
        return int(_lib.dopt_layout_num_buffers(self._h))

    def infos(self) -> List[Dict]:
        """dopt_layout_buffer of every buffer, with the dtype names (cached;
        the layout is immutable)."""
        if getattr(self, "_infos", None) is None:
            out = []
            for k in range(self.num_buffers):
                b = self.buffer(k)
                out.append({**b, "pd": DTYPE_NAMES[b["param_dtype"]], "gd": DTYPE_NAMES[b["grad_dtype"]]})
            self._infos = out
        return self._infos

    def sharding(self) -> Dict:
        o = dopt_sharding_info()
        _check(_lib.dopt_layout_sharding(self._h, ctypes.byref(o)))
        return {name: getattr(o, name) for name, _ in o._fields_}

    def buffer(self, k: int) -> Dict:
        o = dopt_buffer_info()
        _check(_lib.dopt_layout_buffer(self._h, k, ctypes.byref(o)))
        return {name: getattr(o, name) for name, _ in o._fields_ if name != "reserved"}

    def bucket(self, k: int, b: int) -> Dict:
        o = dopt_bucket_info()
        _check(_lib.dopt_layout_bucket(self._h, k, b, ctypes.byref(o)))
        return {name: getattr(o, name) for name, _ in o._fields_ if name != "reserved"}

    def rank_window(self, k: int, b: int, rank: int):
        o = dopt_range()
        _check(_lib.dopt_layout_rank_window(self._h, k, b, rank, ctypes.byref(o)))
        return o.tuple()

    def param(self, p: int) -> Dict:
        o = dopt_param_info()
        _check(_lib.dopt_layout_param(self._h, p, ctypes.byref(o)))
        d = {name: getattr(o, name) for name, _ in o._fields_}
        for key in ("gbuf_world", "gbuf_world_in_bucket", "gbuf_local", "param"):
            d[key] = d[key].tuple()
        return d

    def group(self, kind: str, hgroup: int = 0) -> List[int]:
        k = GROUP_KINDS[kind]
        n = _lib.dopt_layout_group(self._h, k, hgroup, None, 0)
        if n < 0:
            _check(int(n))
        arr = (ctypes.c_int64 * max(n, 1))()
        _lib.dopt_layout_group(self._h, k, hgroup, arr, n)
        return list(arr[:n])

    @property
    def state_numel(self) -> int:
        return int(_lib.dopt_layout_state_numel(self._h))

    @property
    def workspace_bytes(self) -> int:
        return int(_lib.dopt_workspace_bytes(self._h))

    @property
    def stats_record_offset(self) -> int:
        return int(_lib.dopt_stats_record_offset(self._h))


def dopt_build_ranges(params: Sequence, dp_size: int, dp_rank: int, bucket_size: int = 0,
                      pad_for_high_busbw: int = 0, num_instances: int = 1) -> Layout:
    """params: objects with numel, param_dtype, grad_dtype ('f32'|'bf16'|'f16'),
    optional requires_new_bucket and hgroup, in model order."""
    n = len(params)
    arr = (dopt_param_desc * n)()
    for i, p in enumerate(params):
        arr[i].numel = p.numel
        arr[i].param_dtype = DTYPES[p.param_dtype] if isinstance(p.param_dtype, str) else p.param_dtype
        arr[i].grad_dtype = DTYPES[p.grad_dtype] if isinstance(p.grad_dtype, str) else p.grad_dtype
        arr[i].requires_new_bucket = int(getattr(p, "requires_new_bucket", 0))
        arr[i].hgroup = int(getattr(p, "hgroup", 0))
    cfg = dopt_shard_cfg(dp_size, dp_rank, bucket_size, pad_for_high_busbw, num_instances)
    h = ctypes.c_void_p()
    _check(_lib.dopt_build_ranges(arr, n, ctypes.byref(cfg), ctypes.byref(h)))
    return Layout(h, dp_size, dp_rank, n)


class Tensors:
    """The device arrays of every flat buffer, checked against one layout and
    marshalled into the C array of dopt_buffer_tensors (make it once with
    tensors() and pass it to every step)."""

    def __init__(self, layout: "Layout", arr: ctypes.Array, need_grad: bool):
        self.handle, self.arr, self.need_grad = layout.handle.value, arr, need_grad


def tensors(layout: "Layout", bufs: Sequence[Dict], need_grad: bool = True) -> Tensors:
    """bufs: per flat buffer a dict with grad, param, master (None for fp32
    params), exp_avg and exp_avg_sq, each of the buffer's arena_numel
    elements: device tensors (checked here) or raw device addresses."""
    infos = layout.infos()
    if len(bufs) != len(infos):
        raise DoptError(DOPT_ERR_INVALID, f"{len(bufs)} buffer entries, the layout has {len(infos)}")
    arr = (dopt_buffer_tensors * len(bufs))()
    for k, (b, inf) in enumerate(zip(bufs, infos)):
        n, pre = inf["arena_numel"], f"buffer {k} "
        if need_grad or b.get("grad") is not None:
            arr[k].grad = _dev(b.get("grad"), pre + "grad", inf["gd"], n)
        arr[k].param = _dev(b.get("param"), pre + "param", inf["pd"], n)
        if inf["pd"] != "f32":
            arr[k].master = _dev(b.get("master"), pre + "master", "f32", n)
        arr[k].exp_avg = _dev(b.get("exp_avg"), pre + "exp_avg", "f32", n)
        arr[k].exp_avg_sq = _dev(b.get("exp_avg_sq"), pre + "exp_avg_sq", "f32", n)
    return Tensors(layout, arr, need_grad)


def _marshal(layout: "Layout", bufs, need_grad: bool = True) -> ctypes.Array:
    if isinstance(bufs, Tensors):
        if bufs.handle != layout.handle.value:
            raise DoptError(DOPT_ERR_INVALID, "tensors were marshalled for another layout")
        if need_grad and not bufs.need_grad:
            raise DoptError(DOPT_ERR_INVALID, "tensors were marshalled without grads")
        return bufs.arr
    return tensors(layout, bufs, need_grad).arr


def _ws(layout: "Layout", workspace) -> int:
    return _dev(workspace, "workspace", None, 0, layout.workspace_bytes)


def scaler_cfg(dynamic: bool = False, initial_scale: float = 1.0, growth_factor: float = 2.0,
               backoff_factor: float = 0.5, growth_interval: int = 1000, hysteresis: int = 1,
               min_scale: float = 1.0) -> dopt_scaler_cfg:
    return dopt_scaler_cfg(DOPT_SCALER_DYNAMIC if dynamic else DOPT_SCALER_CONSTANT, hysteresis, growth_interval,
                           initial_scale, growth_factor, backoff_factor, min_scale)


def _hparams(hps: Sequence) -> ctypes.Array:
    arr = (dopt_hparams * len(hps))()
    for i, h in enumerate(hps):
        arr[i] = dopt_hparams(*h) if not isinstance(h, dopt_hparams) else h
    return arr


def dopt_init_state(layout: Layout, bufs: Sequence[Dict], scaler: dopt_scaler_cfg, workspace, stream=None):
    _check(_lib.dopt_init_state(layout.handle, _marshal(layout, bufs, False), ctypes.byref(scaler),
                                _ws(layout, workspace), _stream(stream)))


def dopt_step(layout: Layout, bufs, hparams: Sequence, max_grad_norm: float, workspace, stream=None,
              want_stats: bool = True):
    st = dopt_stats() if want_stats else None
    t = _marshal(layout, bufs)
    hp = hparams if isinstance(hparams, ctypes.Array) else _hparams(hparams)
    _check(_lib.dopt_step(layout.handle, t, hp, len(hparams), max_grad_norm, _ws(layout, workspace),
                          _stream(stream), ctypes.byref(st) if st is not None else None))
    return st.as_dict() if st is not None else None


def dopt_step_prepare(layout: Layout, bufs, hparams, max_grad_norm: float, workspace, stream=None):
    t = _marshal(layout, bufs)
    hp = hparams if isinstance(hparams, ctypes.Array) else _hparams(hparams)
    _check(_lib.dopt_step_prepare(layout.handle, t, hp, len(hp), max_grad_norm, _ws(layout, workspace),
                                  _stream(stream)))


def dopt_reduce_prepare(layout: Layout, bufs, chunks: Sequence, wire_dtype: str, n_chunks: int, scale: float,
                        hparams, max_grad_norm: float, workspace, stream=None, chunk_strides: Optional[Sequence] = None):
    """chunks: one device buffer per flat buffer holding n_chunks arenas,
    chunk j at element j * stride (stride = chunk_strides[k], default
    arena_numel: back to back).  hparams None: stats only (finalize later with
    dopt_step_finalize)."""
    t = _marshal(layout, bufs)
    infos = layout.infos()
    if len(chunks) != len(infos):
        raise DoptError(DOPT_ERR_INVALID, f"{len(chunks)} chunk buffers, the layout has {len(infos)}")
    if chunk_strides is not None and len(chunk_strides) != len(infos):
        raise DoptError(DOPT_ERR_INVALID, f"{len(chunk_strides)} chunk strides, the layout has {len(infos)} buffers")
    strides = [int(chunk_strides[k]) if chunk_strides is not None else inf["arena_numel"]
               for k, inf in enumerate(infos)]
    for k, (st, inf) in enumerate(zip(strides, infos)):
        if st < inf["arena_numel"]:
            raise DoptError(DOPT_ERR_INVALID, f"buffer {k}: chunk stride {st} below the arena ({inf['arena_numel']})")
    ch = (ctypes.c_void_p * len(chunks))(*[_dev(c, f"buffer {k} chunks", wire_dtype,
                                                max(n_chunks - 1, 0) * st + inf["arena_numel"])
                                            for k, (c, st, inf) in enumerate(zip(chunks, strides, infos))])
    cs = None if chunk_strides is None else (ctypes.c_int64 * len(strides))(*strides)
    if hparams is None:
        hp, nh = None, 0
    else:
        hp = hparams if isinstance(hparams, ctypes.Array) else _hparams(hparams)
        nh = len(hp)
    _check(_lib.dopt_reduce_prepare(layout.handle, t, ch, cs, DTYPES[wire_dtype], n_chunks, scale, hp, nh,
                                    max_grad_norm, _ws(layout, workspace), _stream(stream)))


class dopt_bucket_check(ctypes.Structure):
    _fields_ = [("sumsq", ctypes.c_double), ("max_abs", ctypes.c_float), ("has_nan", ctypes.c_int32),
                ("has_inf", ctypes.c_int32), ("large", ctypes.c_int32)]


BUCKET_CHECK_BYTES = ctypes.sizeof(dopt_bucket_check)


def dopt_check_grads(layout: Layout, k: int, grad_buffer, large_threshold: float, out, workspace, stream=None):
    """out: device buffer of n_buckets * BUCKET_CHECK_BYTES bytes (e.g. a uint8 CUDA tensor)."""
    infos = layout.infos()
    if not 0 <= k < len(infos):
        raise DoptError(-5, f"buffer index {k} out of range")
    g = _dev(grad_buffer, f"buffer {k} grad buffer", infos[k]["gd"], infos[k]["numel"])
    o = _dev(out, "bucket check output", None, 0, infos[k]["n_buckets"] * BUCKET_CHECK_BYTES)
    _check(_lib.dopt_check_grads(layout.handle, k, g, large_threshold, o, _ws(layout, workspace), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20


def dopt_check_grads_noalloc(layout: Layout, k: int, grad_buffer, large_threshold: float, out, stream=None):
    """dopt_check_grads without a workspace: the library's static device
    scratch holds the tables and partials (no allocation in the call)."""
    infos = layout.infos()
    if not 0 <= k < len(infos):
        raise DoptError(-5, f"buffer index {k} out of range")
    g = _dev(grad_buffer, f"buffer {k} grad buffer", infos[k]["gd"], infos[k]["numel"])
    o = _dev(out, "bucket check output", None, 0, infos[k]["n_buckets"] * BUCKET_CHECK_BYTES)
    _check(_lib.dopt_check_grads_noalloc(layout.handle, k, g, large_threshold, o, _stream(stream)))


def bucket_checks(raw: bytes, n: int) -> List[Dict]:
    """Decode n dopt_bucket_check records copied to the host."""
    arr = (dopt_bucket_check * n).from_buffer_copy(raw)
    return [{name: getattr(r, name) for name, _ in r._fields_} for r in arr]


def dopt_step_stats(layout: Layout, bufs, workspace, stream=None):
    t = _marshal(layout, bufs)
    _check(_lib.dopt_step_stats(layout.handle, t, _ws(layout, workspace), _stream(stream)))


def dopt_step_finalize(layout: Layout, hparams, max_grad_norm: float, workspace, stream=None):
    hp = hparams if isinstance(hparams, ctypes.Array) else _hparams(hparams)
    _check(_lib.dopt_step_finalize(layout.handle, hp, len(hp), max_grad_norm, _ws(layout, workspace),
                                   _stream(stream)))


def dopt_step_apply(layout: Layout, bufs, workspace, stream=None):
    t = _marshal(layout, bufs)
    _check(_lib.dopt_step_apply(layout.handle, t, _ws(layout, workspace), _stream(stream)))


def dopt_read_stats(layout: Layout, workspace, stream=None) -> Dict:
    st = dopt_stats()
    _check(_lib.dopt_read_stats(layout.handle, _ws(layout, workspace), _stream(stream), ctypes.byref(st)))
    return st.as_dict()


def dopt_state_export(layout: Layout, bufs, master, exp_avg, exp_avg_sq, workspace, stream=None):
    """Write the rank's (master, m, v) shards in model order into three fp32
    device arrays of layout.state_numel() elements."""
    t = _marshal(layout, bufs, False)
    x = [_dev(a, f"export {name}", "f32", layout.state_numel)
         for a, name in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"))]
    _check(_lib.dopt_state_export(layout.handle, t, *x, _ws(layout, workspace), _stream(stream)))


def dopt_state_import(layout: Layout, bufs, master, exp_avg, exp_avg_sq, workspace, stream=None):
    """Inverse of dopt_state_export; also rewrites the param window from the master."""
    t = _marshal(layout, bufs, False)
    x = [_dev(a, f"import {name}", "f32", layout.state_numel)
         for a, name in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"))]
    _check(_lib.dopt_state_import(layout.handle, t, *x, _ws(layout, workspace), _stream(stream)))


def dopt_state_scalars_get(layout: Layout, workspace, stream=None) -> Dict:
    st = dopt_state_scalars()
    _check(_lib.dopt_state_scalars_get(layout.handle, _ws(layout, workspace), _stream(stream), ctypes.byref(st)))
    return {name: getattr(st, name) for name, _ in st._fields_}


def dopt_state_scalars_set(layout: Layout, workspace, scalars: Dict, stream=None):
    st = dopt_state_scalars(**scalars)
    _check(_lib.dopt_state_scalars_set(layout.handle, _ws(layout, workspace), _stream(stream), ctypes.byref(st)))


def dopt_last_error() -> str:
    return _lib.dopt_last_error().decode()


# ---- device-memory placement helpers (include/dopt_vmm.h) ----

def dopt_vmm_granularity(device: int = 0) -> int:
    out = ctypes.c_size_t()
    _check(_lib.dopt_vmm_granularity(device, ctypes.byref(out)))
    return out.value


def dopt_vmm_reserve(nbytes: int, align: int = 0) -> int:
    out = ctypes.c_uint64()
    _check(_lib.dopt_vmm_reserve(nbytes, align, ctypes.byref(out)))
    return out.value


def dopt_vmm_free(va: int, nbytes: int):
    _check(_lib.dopt_vmm_free(va, nbytes))


def dopt_vmm_create(nbytes: int, device: int = 0) -> int:
    out = ctypes.c_uint64()
    _check(_lib.dopt_vmm_create(device, nbytes, ctypes.byref(out)))
    return out.value


def dopt_vmm_map(va: int, nbytes: int, handle: int):
    _check(_lib.dopt_vmm_map(va, nbytes, handle))


def dopt_vmm_set_access(va: int, nbytes: int, device: int = 0):
    _check(_lib.dopt_vmm_set_access(va, nbytes, device))


def dopt_vmm_unmap(va: int, nbytes: int):
    _check(_lib.dopt_vmm_unmap(va, nbytes))


def dopt_vmm_release(handle: int):
    _check(_lib.dopt_vmm_release(handle))


hparams_array = _hparams
