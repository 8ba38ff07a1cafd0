"""Python binding of ``libzs.so``, the MI355X shard-local step (ZeRO / FSDP).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. Functions carry the C ABI's names (``include/zs.h``). Device buffers
are PyTorch CUDA tensors (or raw integer device addresses); the stream is
``torch.cuda.current_stream()`` unless one is given. Before each call the
binding checks that every tensor is a contiguous CUDA tensor of the right
dtype and at least as long as the kernels will touch, so a wrong shape is a
Python exception instead of an out-of-bounds access on the device.

If the library has not been built this module raises on import: there is no
fallback path.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzs.so")

ZS_OK, ZS_EINVAL, ZS_EALIGN, ZS_ERANGE, ZS_EHIP, ZS_ENOMEM = 0, -1, -2, -3, -4, -5
ZS_LAYOUT_FLAT, ZS_LAYOUT_PER_TENSOR = 0, 1
ZS_MAX_CONTRIBS = 256
ZS_MAX_GROUPS = 8
GRAD_STATS_NOALLOC_MAX_ELEMS = 1431568384
FUSED_TWO_PASS_MIN_CONTRIBS = 52  # zs_fused_shard_step runs two passes from here when grad is given

_STATUS_NAMES = {0: "ZS_OK", -1: "ZS_EINVAL", -2: "ZS_EALIGN", -3: "ZS_ERANGE", -4: "ZS_EHIP",
                 -5: "ZS_ENOMEM"}


class ZsError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class AdamWHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("step", ctypes.c_int64)]

    def __init__(self, lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1):
        super().__init__(lr, beta1, beta2, eps, weight_decay, step)

    def at(self, step):
        return AdamWHParams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay, step)


class AdamWCoefs(ctypes.Structure):
    """The fp32 scalars of one AdamW step (zs_adamw_coefs)."""
    _fields_ = [(name, ctypes.c_float) for name in
                ("beta1", "one_minus_beta1", "beta2", "one_minus_beta2", "lr", "eps", "decay", "bias_correction1",
                 "bias_correction2")]

    def values(self):
        return [getattr(self, name) for name, _ in self._fields_]


class TensorInfo(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("flat_off", ctypes.c_int64),
                ("padded_numel", ctypes.c_int64), ("own_lo", ctypes.c_int64),
                ("own_hi", ctypes.c_int64), ("shard_off", ctypes.c_int64)]


class PlanOptions(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("tensor_align_elems", ctypes.c_int32),
                ("persist_below_elems", ctypes.c_int64), ("groups", ctypes.POINTER(ctypes.c_int32))]


class ReshardSlice(ctypes.Structure):
    _fields_ = [("group_size", ctypes.c_int32), ("slice_index", ctypes.c_int32), ("slice_off", ctypes.c_int64),
                ("slice_len", ctypes.c_int64), ("first_source", ctypes.c_int32), ("n_sources", ctypes.c_int32),
                ("owner_slice", ctypes.c_int32), ("reserved", ctypes.c_int32), ("own_off", ctypes.c_int64),
                ("retained_bytes", ctypes.c_int64)]


class PiecePtrs(ctypes.Structure):
    _fields_ = [("grad", ctypes.c_void_p), ("master", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("param", ctypes.c_void_p), ("full", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build() or "
                          f"python {os.path.join(_HERE, 'build.py')})")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    st = ctypes.c_int
    sigs = {
        "zs_shard_plan": (st, [ctypes.POINTER(i64), i32, i32, i32, i32, i32, ctypes.POINTER(vp)]),
        "zs_shard_plan_ex": (st, [ctypes.POINTER(i64), i32, i32, i32, ctypes.POINTER(PlanOptions),
                                  ctypes.POINTER(vp)]),
        "zs_plan_tensor_group": (i32, [vp, i32]),
        "zs_plan_tensor_replicated": (i32, [vp, i32]),
        "zs_plan_destroy": (None, [vp]),
        "zs_plan_padded_numel": (i64, [vp]),
        "zs_plan_shard_numel": (i64, [vp]),
        "zs_plan_persistent_bytes": (i64, [vp]),
        "zs_plan_num_tensors": (i32, [vp]),
        "zs_plan_world_size": (i32, [vp]),
        "zs_plan_rank": (i32, [vp]),
        "zs_plan_layout": (i32, [vp]),
        "zs_plan_tensor": (st, [vp, i32, ctypes.POINTER(TensorInfo)]),
        "zs_reduce_shard": (st, [vp, ctypes.POINTER(vp), i32, vp, i64, i64, vp]),
        "zs_adamw_shard_step": (st, [vp, ctypes.POINTER(AdamWHParams), vp, vp, vp, vp, vp, vp]),
        "zs_gather_params": (st, [vp, vp, vp, vp]),
        "zs_plan_reshard_slice": (st, [vp, i32, ctypes.POINTER(ReshardSlice)]),
        "zs_gather_params_to_slice": (st, [vp, i32, vp, vp, vp]),
        "zs_gather_slice": (st, [vp, i32, ctypes.POINTER(vp), i32, vp, vp]),
        "zs_fused_shard_step": (st, [vp, ctypes.POINTER(AdamWHParams), ctypes.POINTER(vp), i32, vp, vp,
                                     vp, vp, vp, vp, vp]),
        "zs_fused_shard_step_bucket": (st, [vp, ctypes.POINTER(AdamWHParams), ctypes.POINTER(vp), i32, vp, vp,
                                            vp, vp, vp, vp, i64, i64, vp]),
        "zs_multi_workspace_bytes": (i64, [vp, i32]),
        "zs_plan_workspace_bytes": (i64, [vp]),
        "zs_multi_bind": (st, [vp, ctypes.POINTER(PiecePtrs), ctypes.POINTER(vp), i32, vp, i64, vp]),
        "zs_multi_unbind": (st, [vp, vp]),
        "zs_reduce_shard_multi": (st, [vp, vp, vp]),
        "zs_adamw_shard_step_multi": (st, [vp, ctypes.POINTER(AdamWHParams), vp, vp]),
        "zs_gather_params_multi": (st, [vp, vp, vp]),
        "zs_fused_shard_step_multi": (st, [vp, ctypes.POINTER(AdamWHParams), vp, vp]),
        "zs_adamw_shard_step_multi_groups": (st, [vp, ctypes.POINTER(AdamWHParams), i32, vp, vp]),
        "zs_fused_shard_step_multi_groups": (st, [vp, ctypes.POINTER(AdamWHParams), i32, vp, vp]),
        "zs_quant_code_bytes": (i64, [vp, i32]),
        "zs_quant_num_scales": (i64, [vp, i32]),
        "zs_quantize_shard": (st, [vp, i32, i32, vp, vp, vp, vp]),
        "zs_fused_shard_step_quant": (st, [vp, ctypes.POINTER(AdamWHParams), ctypes.POINTER(vp), i32, vp, vp, vp,
                                           vp, vp, i32, i32, vp, vp, vp]),
        "zs_dequant_gather": (st, [vp, i32, i32, vp, vp, vp, vp]),
        "zs_host_adamw_step": (st, [ctypes.POINTER(AdamWHParams), vp, vp, vp, vp, vp, i64, i32]),
        "zs_offload_adamw_step": (st, [vp, ctypes.POINTER(AdamWHParams), vp, vp, vp, vp, vp, vp, vp, vp, i64, i32,
                                       vp]),
        "zs_accumulate_shard": (st, [vp, ctypes.POINTER(vp), i32, vp, i64, i64, i32, vp]),
        "zs_grad_stats_workspace_bytes": (i64, [vp]),
        "zs_grad_stats": (st, [vp, vp, ctypes.c_float, vp, vp, vp, i64, vp]),
        "zs_grad_stats_noalloc": (st, [vp, vp, ctypes.c_float, vp, vp, vp]),
        "zs_clip_scale": (st, [vp, vp, i32, ctypes.c_double, vp, vp, vp]),
        "zs_adamw_shard_step_accum": (st, [vp, ctypes.POINTER(AdamWHParams), vp, ctypes.c_float, vp, vp, vp, vp,
                                           vp, vp, vp, vp]),
        "zs_adamw_coefs_compute": (st, [ctypes.POINTER(AdamWHParams), ctypes.POINTER(AdamWCoefs)]),
        "zs_fused_shard_step_dc": (st, [vp, vp, ctypes.POINTER(vp), i32, vp, vp, vp, vp, vp, vp, vp]),
        "zs_adamw_shard_step_dc": (st, [vp, vp, vp, vp, vp, vp, vp, vp]),
        "zs_adamw_shard_step_accum_dc": (st, [vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp]),
        "zs_fused_shard_step_multi_dc": (st, [vp, vp, i32, vp, vp]),
        "zs_last_error": (ctypes.c_char_p, []),
        "zs_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


_lib = _load()
EXPORTED = ("zs_shard_plan", "zs_shard_plan_ex", "zs_plan_tensor_group", "zs_plan_tensor_replicated",
            "zs_plan_destroy", "zs_plan_padded_numel", "zs_plan_shard_numel",
            "zs_plan_persistent_bytes", "zs_plan_num_tensors", "zs_plan_world_size", "zs_plan_rank",
            "zs_plan_layout", "zs_plan_tensor", "zs_reduce_shard", "zs_adamw_shard_step",
            "zs_gather_params", "zs_plan_reshard_slice", "zs_gather_params_to_slice", "zs_gather_slice",
            "zs_fused_shard_step", "zs_fused_shard_step_bucket", "zs_multi_workspace_bytes",
            "zs_plan_workspace_bytes",
            "zs_multi_bind", "zs_multi_unbind",
            "zs_reduce_shard_multi", "zs_adamw_shard_step_multi", "zs_gather_params_multi",
            "zs_fused_shard_step_multi", "zs_adamw_shard_step_multi_groups",
            "zs_fused_shard_step_multi_groups", "zs_quant_code_bytes", "zs_quant_num_scales", "zs_quantize_shard",
            "zs_fused_shard_step_quant", "zs_dequant_gather", "zs_host_adamw_step", "zs_offload_adamw_step",
            "zs_accumulate_shard", "zs_grad_stats_workspace_bytes",
            "zs_grad_stats", "zs_grad_stats_noalloc", "zs_clip_scale", "zs_adamw_shard_step_accum",
            "zs_adamw_coefs_compute",
            "zs_fused_shard_step_dc", "zs_adamw_shard_step_dc", "zs_adamw_shard_step_accum_dc",
            "zs_fused_shard_step_multi_dc", "zs_last_error", "zs_version")


def lib():
    return _lib


def _check(status):
    if status != ZS_OK:
        raise ZsError(status, _lib.zs_last_error().decode())


# ---------------------------------------------------------------- marshalling helpers


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


_BF16_NAMES = ("bfloat16", "int16", "uint16")


def _ptr(t, kind, need, what):
    """Device address of ``t`` after checking dtype, device, contiguity and length."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    import torch
    if not t.is_cuda:
        raise ValueError(f"{what} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if kind == "bytes":
        if t.dtype not in (torch.uint8, torch.int8):
            raise ValueError(f"{what} must be a uint8 or int8 byte buffer, got {t.dtype}")
    elif kind == "bf16":
        if str(t.dtype).split(".")[-1] not in _BF16_NAMES:
            raise ValueError(f"{what} must hold bf16 (bfloat16 or 16-bit integer storage), got {t.dtype}")
    elif t.dtype != torch.float32:
        raise ValueError(f"{what} must be float32, got {t.dtype}")
    if t.numel() < need:
        raise ValueError(f"{what} holds {t.numel()} elements, the call touches {need}")
    return t.data_ptr()


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(len(ptrs), 1))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


# ---------------------------------------------------------------- plan


class Plan:
    """Owns a ``zs_plan*``; destroyed with the object (or by ``close``)."""

    def __init__(self, handle):
        self._h = ctypes.c_void_p(handle)

    @property
    def handle(self):
        if not self._h:
            raise ValueError("plan is closed")
        return self._h

    def close(self):
        if self._h:
            _lib.zs_plan_destroy(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def padded_numel(self):
        return _lib.zs_plan_padded_numel(self.handle)

    @property
    def shard_numel(self):
        return _lib.zs_plan_shard_numel(self.handle)

    @property
    def persistent_bytes(self):
        return _lib.zs_plan_persistent_bytes(self.handle)

    @property
    def num_tensors(self):
        return _lib.zs_plan_num_tensors(self.handle)

    @property
    def world_size(self):
        return _lib.zs_plan_world_size(self.handle)

    @property
    def rank(self):
        return _lib.zs_plan_rank(self.handle)

    @property
    def layout(self):
        return _lib.zs_plan_layout(self.handle)

    @property
    def workspace_bytes(self):
        return _lib.zs_plan_workspace_bytes(self.handle)

    def tensor(self, i):
        info = TensorInfo()
        _check(_lib.zs_plan_tensor(self.handle, i, ctypes.byref(info)))
        return info

    def tensor_group(self, i):
        g = _lib.zs_plan_tensor_group(self.handle, i)
        if g < 0:
            raise IndexError(f"tensor {i} is not in the plan")
        return g

    def tensor_replicated(self, i):
        r = _lib.zs_plan_tensor_replicated(self.handle, i)
        if r < 0:
            raise IndexError(f"tensor {i} is not in the plan")
        return bool(r)


def zs_shard_plan(numels, world_size, rank, tensor_align_elems=1, layout=ZS_LAYOUT_FLAT):
    arr = (ctypes.c_int64 * max(len(numels), 1))(*numels)
    out = ctypes.c_void_p()
    _check(_lib.zs_shard_plan(arr, len(numels), world_size, rank, tensor_align_elems, layout,
                              ctypes.byref(out)))
    return Plan(out.value)


def zs_shard_plan_ex(numels, world_size, rank, layout=ZS_LAYOUT_PER_TENSOR, tensor_align_elems=1,
                     persist_below_elems=0, groups=None):
    arr = (ctypes.c_int64 * max(len(numels), 1))(*numels)
    opt = PlanOptions(layout, tensor_align_elems, persist_below_elems, None)
    if groups is not None:
        if len(groups) != len(numels):
            raise ValueError(f"groups has {len(groups)} entries for {len(numels)} tensors")
        garr = (ctypes.c_int32 * max(len(groups), 1))(*groups)
        opt.groups = ctypes.cast(garr, ctypes.POINTER(ctypes.c_int32))
    out = ctypes.c_void_p()
    _check(_lib.zs_shard_plan_ex(arr, len(numels), world_size, rank, ctypes.byref(opt), ctypes.byref(out)))
    return Plan(out.value)


# ---------------------------------------------------------------- flat step


def zs_reduce_shard(plan, contribs, grad, off=0, length=None, stream=None):
    S = plan.shard_numel
    length = S - off if length is None else length
    end = min(max(off + length, 0), S)  # a bucket outside the shard is the library's ZS_ERANGE
    ptrs = [_ptr(c, "bf16", end, f"contribs[{q}]") for q, c in enumerate(contribs)]
    g = _ptr(grad, "bf16", end, "grad")
    _check(_lib.zs_reduce_shard(plan.handle, _ptr_array(ptrs), len(ptrs), g, off, length,
                                _stream(stream)))


def zs_adamw_shard_step(plan, hp, grad, master, m, v, param, stream=None):
    S = plan.shard_numel
    _check(_lib.zs_adamw_shard_step(plan.handle, ctypes.byref(hp), _ptr(grad, "bf16", S, "grad"),
                                    _ptr(master, "f32", S, "master"), _ptr(m, "f32", S, "m"),
                                    _ptr(v, "f32", S, "v"), _ptr(param, "bf16", S, "param"),
                                    _stream(stream)))


def zs_gather_params(plan, param, full, stream=None):
    S, r = plan.shard_numel, plan.rank
    _check(_lib.zs_gather_params(plan.handle, _ptr(param, "bf16", S, "param"),
                                 _ptr(full, "bf16", (r + 1) * S, "full"), _stream(stream)))


def zs_plan_reshard_slice(plan, group_size):
    out = ReshardSlice()
    _check(_lib.zs_plan_reshard_slice(plan.handle, group_size, ctypes.byref(out)))
    return out


def zs_gather_params_to_slice(plan, group_size, param, slice_buf, stream=None):
    """param: the own updated bf16 shard (S); slice_buf: the buffer holding the
    k-way slice that contains it (T/k elements)."""
    sl = zs_plan_reshard_slice(plan, group_size)
    _check(_lib.zs_gather_params_to_slice(plan.handle, group_size, _ptr(param, "bf16", plan.shard_numel, "param"),
                                          _ptr(slice_buf, "bf16", sl.slice_len, "slice"), _stream(stream)))


def zs_gather_slice(plan, group_size, shards, slice_buf, stream=None):
    """shards[i]: the updated bf16 shard (S) of rank first_source + i;
    slice_buf: this rank's kept slice (T/k elements)."""
    sl = zs_plan_reshard_slice(plan, group_size)
    ptrs = [_ptr(t, "bf16", plan.shard_numel, f"shards[{i}]") for i, t in enumerate(shards)]
    _check(_lib.zs_gather_slice(plan.handle, group_size, _ptr_array(ptrs), len(ptrs),
                                _ptr(slice_buf, "bf16", sl.slice_len, "slice"), _stream(stream)))


def zs_fused_shard_step(plan, hp, contribs, master, m, v, grad=None, param=None, full=None,
                        stream=None):
    S, r = plan.shard_numel, plan.rank
    ptrs = [_ptr(c, "bf16", S, f"contribs[{q}]") for q, c in enumerate(contribs)]
    _check(_lib.zs_fused_shard_step(plan.handle, ctypes.byref(hp), _ptr_array(ptrs), len(ptrs),
                                    _ptr(master, "f32", S, "master"), _ptr(m, "f32", S, "m"),
                                    _ptr(v, "f32", S, "v"), _ptr(grad, "bf16", S, "grad"),
                                    _ptr(param, "bf16", S, "param"),
                                    _ptr(full, "bf16", (r + 1) * S, "full"), _stream(stream)))


def zs_fused_shard_step_bucket(plan, hp, contribs, master, m, v, off=0, length=None, grad=None, param=None,
                               full=None, stream=None):
    S, r = plan.shard_numel, plan.rank
    length = S - off if length is None else length
    end = min(max(off + length, 0), S)  # a bucket outside the shard is the library's ZS_ERANGE
    ptrs = [_ptr(c, "bf16", end, f"contribs[{q}]") for q, c in enumerate(contribs)]
    _check(_lib.zs_fused_shard_step_bucket(plan.handle, ctypes.byref(hp), _ptr_array(ptrs), len(ptrs),
                                           _ptr(master, "f32", end, "master"), _ptr(m, "f32", end, "m"),
                                           _ptr(v, "f32", end, "v"), _ptr(grad, "bf16", end, "grad"),
                                           _ptr(param, "bf16", end, "param"),
                                           _ptr(full, "bf16", r * S + end, "full"), off, length, _stream(stream)))


# ---------------------------------------------------------------- quantized parameter gather


def zs_quant_code_bytes(plan, bits):
    n = _lib.zs_quant_code_bytes(plan.handle, bits)
    if n < 0:
        raise ValueError(f"bits = {bits} must be 4 or 8")
    return n


def zs_quant_num_scales(plan, block):
    n = _lib.zs_quant_num_scales(plan.handle, block)
    if n < 0:
        raise ValueError(f"block = {block} must be a power of two in [8, 256]")
    return n


def zs_quantize_shard(plan, bits, block, param, codes, scales, stream=None):
    S = plan.shard_numel
    _check(_lib.zs_quantize_shard(plan.handle, bits, block, _ptr(param, "bf16", S, "param"),
                                  _ptr(codes, "bytes", S * bits // 8, "codes"),
                                  _ptr(scales, "f32", -(-S // max(block, 1)), "scales"), _stream(stream)))


def zs_fused_shard_step_quant(plan, hp, contribs, master, m, v, bits, block, codes, scales, grad=None, param=None,
                              stream=None):
    S = plan.shard_numel
    ptrs = [_ptr(c, "bf16", S, f"contribs[{q}]") for q, c in enumerate(contribs)]
    _check(_lib.zs_fused_shard_step_quant(plan.handle, ctypes.byref(hp), _ptr_array(ptrs), len(ptrs),
                                          _ptr(master, "f32", S, "master"), _ptr(m, "f32", S, "m"),
                                          _ptr(v, "f32", S, "v"), _ptr(grad, "bf16", S, "grad"),
                                          _ptr(param, "bf16", S, "param"), bits, block,
                                          _ptr(codes, "bytes", S * bits // 8, "codes"),
                                          _ptr(scales, "f32", -(-S // max(block, 1)), "scales"), _stream(stream)))


def zs_dequant_gather(plan, bits, block, codes_all, scales_all, full, stream=None):
    S, N = plan.shard_numel, plan.world_size
    _check(_lib.zs_dequant_gather(plan.handle, bits, block, _ptr(codes_all, "bytes", N * S * bits // 8, "codes_all"),
                                  _ptr(scales_all, "f32", N * -(-S // max(block, 1)), "scales_all"),
                                  _ptr(full, "bf16", N * S, "full"), _stream(stream)))


# ---------------------------------------------------------------- CPU-offloaded optimizer step

_HOST_KINDS = {"bf16": ("uint16", "int16", "bfloat16"), "f32": ("float32",)}


def _host_ptr(a, kind, need, what):
    """Host address of a numpy array or CPU tensor after checking dtype, contiguity and length."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if hasattr(a, "is_cuda"):  # torch tensor
        if a.is_cuda:
            raise ValueError(f"{what} must be host memory")
        if not a.is_contiguous():
            raise ValueError(f"{what} must be contiguous")
        dt, n, addr = str(a.dtype).split(".")[-1], a.numel(), a.data_ptr()
    else:
        if not a.flags.c_contiguous:
            raise ValueError(f"{what} must be contiguous")
        dt, n, addr = str(a.dtype), a.size, a.ctypes.data
    if dt not in _HOST_KINDS[kind]:
        raise ValueError(f"{what} must be {kind}, got {dt}")
    if n < need:
        raise ValueError(f"{what} holds {n} elements, the call touches {need}")
    return addr


def zs_host_adamw_step(hp, grad, master, m, v, param=None, n=None, n_threads=1):
    if n is None:
        n = master.numel() if hasattr(master, "numel") else master.size
    _check(_lib.zs_host_adamw_step(ctypes.byref(hp), _host_ptr(grad, "bf16", n, "grad"),
                                   _host_ptr(master, "f32", n, "master"), _host_ptr(m, "f32", n, "m"),
                                   _host_ptr(v, "f32", n, "v"), _host_ptr(param, "bf16", n, "param"), n, n_threads))


def zs_offload_adamw_step(plan, hp, grad_dev, master_host, m_host, v_host, grad_host, param_host, param_dev=None,
                          full_dev=None, chunk_elems=1 << 24, n_threads=8, stream=None):
    S, r = plan.shard_numel, plan.rank
    _check(_lib.zs_offload_adamw_step(plan.handle, ctypes.byref(hp), _ptr(grad_dev, "bf16", S, "grad_dev"),
                                      _host_ptr(master_host, "f32", S, "master_host"),
                                      _host_ptr(m_host, "f32", S, "m_host"), _host_ptr(v_host, "f32", S, "v_host"),
                                      _host_ptr(grad_host, "bf16", S, "grad_host"),
                                      _host_ptr(param_host, "bf16", S, "param_host"),
                                      _ptr(param_dev, "bf16", S, "param_dev"),
                                      _ptr(full_dev, "bf16", (r + 1) * S, "full_dev"), chunk_elems, n_threads,
                                      _stream(stream)))


# ---------------------------------------------------------------- multi-tensor


def zs_multi_workspace_bytes(plan, n_contribs):
    n = _lib.zs_multi_workspace_bytes(plan.handle, n_contribs)
    if n < 0:
        raise ZsError(ZS_EINVAL, "multi-tensor workspace needs a PER_TENSOR plan")
    return n


# Bound workspaces, keyed by device address: the workspace tensor and every
# tensor whose address its table holds. Keeping them referenced until
# zs_multi_unbind means no bound buffer can be freed (and its memory reused by
# the caching allocator) while a step may still write through the table.
_bindings = {}


def zs_multi_bind(plan, pieces, contribs, workspace, stream=None):
    """pieces[i]: dict with keys grad, master, m, v, param, full (tensors or
    None) for tensor i; contribs: None or contribs[q][i] = rank q's piece of
    tensor i. workspace: a CUDA uint8 tensor of zs_multi_workspace_bytes.
    The binding keeps references to the workspace and every bound tensor
    until zs_multi_unbind(workspace)."""
    n = plan.num_tensors
    if len(pieces) != n:
        raise ValueError(f"{len(pieces)} piece records for a plan of {n} tensors")
    recs = (PiecePtrs * max(n, 1))()
    for i, pc in enumerate(pieces):
        info = plan.tensor(i)
        Si = info.own_hi - info.own_lo
        recs[i] = PiecePtrs(_ptr(pc.get("grad"), "bf16", Si, f"pieces[{i}].grad"),
                            _ptr(pc.get("master"), "f32", Si, f"pieces[{i}].master"),
                            _ptr(pc.get("m"), "f32", Si, f"pieces[{i}].m"),
                            _ptr(pc.get("v"), "f32", Si, f"pieces[{i}].v"),
                            _ptr(pc.get("param"), "bf16", Si, f"pieces[{i}].param"),
                            _ptr(pc.get("full"), "bf16", info.padded_numel, f"pieces[{i}].full"))
    nq = 0 if contribs is None else len(contribs)
    flat = []
    for q in range(nq):
        if len(contribs[q]) != n:
            raise ValueError(f"contribs[{q}] has {len(contribs[q])} pieces, the plan has {n}")
        for i in range(n):
            info = plan.tensor(i)
            flat.append(_ptr(contribs[q][i], "bf16", info.own_hi - info.own_lo, f"contribs[{q}][{i}]"))
    import torch
    if not (isinstance(workspace, torch.Tensor) and workspace.is_cuda):
        raise ValueError("workspace must be a CUDA tensor")
    _check(_lib.zs_multi_bind(plan.handle, recs, _ptr_array(flat) if nq else None, nq,
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              _stream(stream)))
    refs = [t for pc in pieces for t in pc.values() if t is not None and not isinstance(t, int)]
    if nq:
        refs += [t for row in contribs for t in row if not isinstance(t, int)]
    _bindings[workspace.data_ptr()] = (workspace, refs)


def zs_multi_unbind(workspace, stream=None):
    _check(_lib.zs_multi_unbind(workspace.data_ptr(), _stream(stream)))
    _bindings.pop(workspace.data_ptr(), None)


def zs_reduce_shard_multi(plan, workspace, stream=None):
    _check(_lib.zs_reduce_shard_multi(plan.handle, workspace.data_ptr(), _stream(stream)))


def zs_adamw_shard_step_multi(plan, hp, workspace, stream=None):
    _check(_lib.zs_adamw_shard_step_multi(plan.handle, ctypes.byref(hp), workspace.data_ptr(),
                                          _stream(stream)))


def zs_gather_params_multi(plan, workspace, stream=None):
    _check(_lib.zs_gather_params_multi(plan.handle, workspace.data_ptr(), _stream(stream)))


def zs_fused_shard_step_multi(plan, hp, workspace, stream=None):
    _check(_lib.zs_fused_shard_step_multi(plan.handle, ctypes.byref(hp), workspace.data_ptr(),
                                          _stream(stream)))


def _hp_array(hps):
    if not hps:
        raise ValueError("at least one set of hyperparameters is needed")
    return (AdamWHParams * len(hps))(*hps), len(hps)


def zs_adamw_shard_step_multi_groups(plan, hps, workspace, stream=None):
    arr, n = _hp_array(hps)
    _check(_lib.zs_adamw_shard_step_multi_groups(plan.handle, arr, n, workspace.data_ptr(), _stream(stream)))


def zs_fused_shard_step_multi_groups(plan, hps, workspace, stream=None):
    arr, n = _hp_array(hps)
    _check(_lib.zs_fused_shard_step_multi_groups(plan.handle, arr, n, workspace.data_ptr(), _stream(stream)))


# ---------------------------------------------------------------- accumulation and clipping


def _scalar_ptr(t, dtype_name, what):
    if t is None:
        return None
    import torch
    if not (isinstance(t, torch.Tensor) and t.is_cuda and str(t.dtype).endswith(dtype_name) and t.numel() >= 1):
        raise ValueError(f"{what} must be a CUDA {dtype_name} tensor of at least one element")
    return t.data_ptr()


def zs_accumulate_shard(plan, contribs, acc, off=0, length=None, first=False, stream=None):
    S = plan.shard_numel
    length = S - off if length is None else length
    end = min(max(off + length, 0), S)
    ptrs = [_ptr(c, "bf16", end, f"contribs[{q}]") for q, c in enumerate(contribs)]
    _check(_lib.zs_accumulate_shard(plan.handle, _ptr_array(ptrs), len(ptrs), _ptr(acc, "f32", end, "acc"), off,
                                    length, 1 if first else 0, _stream(stream)))


def zs_grad_stats_workspace_bytes(plan):
    return _lib.zs_grad_stats_workspace_bytes(plan.handle)


def zs_grad_stats(plan, acc, grad_divisor, sumsq_out, nonfinite_out, workspace, stream=None):
    """sumsq_out: CUDA float64 tensor (>= 1 element); nonfinite_out: CUDA int32
    tensor; workspace: CUDA uint8 tensor of zs_grad_stats_workspace_bytes."""
    _check(_lib.zs_grad_stats(plan.handle, _ptr(acc, "f32", plan.shard_numel, "acc"), grad_divisor,
                              _scalar_ptr(sumsq_out, "float64", "sumsq_out"),
                              _scalar_ptr(nonfinite_out, "int32", "nonfinite_out"), workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), _stream(stream)))


def zs_grad_stats_noalloc(plan, acc, grad_divisor, sumsq_out, nonfinite_out, stream=None):
    """zs_grad_stats with the partials in the library's static device array
    (no workspace, no allocation); shards up to GRAD_STATS_NOALLOC_MAX_ELEMS."""
    _check(_lib.zs_grad_stats_noalloc(plan.handle, _ptr(acc, "f32", plan.shard_numel, "acc"),
                                      ctypes.c_float(grad_divisor), _scalar_ptr(sumsq_out, "float64", "sumsq_out"),
                                      _scalar_ptr(nonfinite_out, "int32", "nonfinite_out"), _stream(stream)))


def zs_clip_scale(sumsq, nonfinite, max_norm, scale_out, skip_out, stream=None):
    """sumsq: CUDA float64 tensor of the ranks' squared norms; nonfinite: CUDA
    int32 tensor of their flags (same length)."""
    n = sumsq.numel()
    if nonfinite.numel() != n:
        raise ValueError("sumsq and nonfinite must have one entry per rank")
    _check(_lib.zs_clip_scale(_scalar_ptr(sumsq, "float64", "sumsq"), _scalar_ptr(nonfinite, "int32", "nonfinite"),
                              n, max_norm, _scalar_ptr(scale_out, "float32", "scale_out"),
                              _scalar_ptr(skip_out, "int32", "skip_out"), _stream(stream)))


def zs_adamw_shard_step_accum(plan, hp, acc, grad_divisor, master, m, v, scale=None, skip=None, param=None,
                              full=None, stream=None):
    S, r = plan.shard_numel, plan.rank
    _check(_lib.zs_adamw_shard_step_accum(plan.handle, ctypes.byref(hp), _ptr(acc, "f32", S, "acc"), grad_divisor,
                                          _scalar_ptr(scale, "float32", "scale"), _scalar_ptr(skip, "int32", "skip"),
                                          _ptr(master, "f32", S, "master"), _ptr(m, "f32", S, "m"),
                                          _ptr(v, "f32", S, "v"), _ptr(param, "bf16", S, "param"),
                                          _ptr(full, "bf16", (r + 1) * S, "full"), _stream(stream)))


# ---------------------------------------------------------------- scalars in device memory


def zs_adamw_coefs_compute(hp):
    """The fp32 scalars of hp's step (an AdamWCoefs; .values() lists them in
    the order a device buffer holds them)."""
    out = AdamWCoefs()
    _check(_lib.zs_adamw_coefs_compute(ctypes.byref(hp), ctypes.byref(out)))
    return out


def _coefs_ptr(coefs, n_sets=1):
    return _ptr(coefs, "f32", 9 * n_sets, "coefs")


def zs_fused_shard_step_dc(plan, coefs, contribs, master, m, v, grad=None, param=None, full=None, stream=None):
    S, r = plan.shard_numel, plan.rank
    ptrs = [_ptr(c, "bf16", S, f"contribs[{q}]") for q, c in enumerate(contribs)]
    _check(_lib.zs_fused_shard_step_dc(plan.handle, _coefs_ptr(coefs), _ptr_array(ptrs), len(ptrs),
                                       _ptr(master, "f32", S, "master"), _ptr(m, "f32", S, "m"),
                                       _ptr(v, "f32", S, "v"), _ptr(grad, "bf16", S, "grad"),
                                       _ptr(param, "bf16", S, "param"), _ptr(full, "bf16", (r + 1) * S, "full"),
                                       _stream(stream)))


def zs_adamw_shard_step_dc(plan, coefs, grad, master, m, v, param, stream=None):
    S = plan.shard_numel
    _check(_lib.zs_adamw_shard_step_dc(plan.handle, _coefs_ptr(coefs), _ptr(grad, "bf16", S, "grad"),
                                       _ptr(master, "f32", S, "master"), _ptr(m, "f32", S, "m"),
                                       _ptr(v, "f32", S, "v"), _ptr(param, "bf16", S, "param"), _stream(stream)))


def zs_adamw_shard_step_accum_dc(plan, coefs, acc, grad_divisor, master, m, v, scale=None, skip=None, param=None,
                                 full=None, stream=None):
    S, r = plan.shard_numel, plan.rank
    _check(_lib.zs_adamw_shard_step_accum_dc(plan.handle, _coefs_ptr(coefs), _ptr(acc, "f32", S, "acc"),
                                             grad_divisor, _scalar_ptr(scale, "float32", "scale"),
                                             _scalar_ptr(skip, "int32", "skip"), _ptr(master, "f32", S, "master"),
                                             _ptr(m, "f32", S, "m"), _ptr(v, "f32", S, "v"),
                                             _ptr(param, "bf16", S, "param"), _ptr(full, "bf16", (r + 1) * S, "full"),
                                             _stream(stream)))


def zs_fused_shard_step_multi_dc(plan, coefs, n_groups, workspace, stream=None):
    _check(_lib.zs_fused_shard_step_multi_dc(plan.handle, _coefs_ptr(coefs, n_groups), n_groups,
                                             workspace.data_ptr(), _stream(stream)))


def zs_last_error():
    return _lib.zs_last_error().decode()


def zs_version():
    return _lib.zs_version().decode()
