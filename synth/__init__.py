"""Seeded synthetic inputs shared by the oracle side and the GPU side.

The bits come from ``synth_def.h`` (counter-based SplitMix64 output function,
Irwin-Hall approximate normals), built once for the host (``libsynth_cpu.so``)
and once for the GPU (``libsynth_gpu.so``). Both builds give identical values
for the same (seed, stream, step, global index), so the oracle reads its inputs
from the host build while the GPU path reads device buffers filled by the GPU
build, and no input of either side is produced by the other.

Nothing in here computes any part of the optimizer step.
"""

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

from . import shapes  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_CPU_LIB = os.path.join(_HERE, "libsynth_cpu.so")
_GPU_LIB = os.path.join(_HERE, "libsynth_gpu.so")

# Stream ids: which buffer a value belongs to.
STREAM_MASTER = 1
STREAM_ZERO_MASK = 2
STREAM_CONTRIB = 0x1000  # + contribution (rank) index q

DEFAULT_SEED = 0x5A5EED


class SynthSpec(ctypes.Structure):
    _fields_ = [
        ("key", ctypes.c_uint64),
        ("zero_key", ctypes.c_uint64),
        ("sigma", ctypes.c_float),
        ("tail_sigma", ctypes.c_float),
        ("tail_thresh", ctypes.c_uint32),
        ("zero_thresh", ctypes.c_uint32),
        ("valid_hi", ctypes.c_int64),
    ]


_cpu = None
_gpu = None
_i64 = ctypes.c_int64


def cpu_lib():
    global _cpu
    if _cpu is None:
        if not os.path.exists(_CPU_LIB):
            from . import build as _b
            _b.build_cpu()
        L = ctypes.CDLL(_CPU_LIB)
        L.synth_cpu_key.restype = ctypes.c_uint64
        L.synth_cpu_key.argtypes = [ctypes.c_uint64] * 3
        sp = ctypes.POINTER(SynthSpec)
        L.synth_cpu_fill_f32.argtypes = [ctypes.c_void_p, _i64, _i64, sp]
        L.synth_cpu_fill_bf16.argtypes = [ctypes.c_void_p, _i64, _i64, sp]
        L.synth_cpu_at_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, _i64, sp]
        L.synth_cpu_at_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, _i64, sp]
        _cpu = L
    return _cpu


def gpu_lib():
    global _gpu
    if _gpu is None:
        if not os.path.exists(_GPU_LIB):
            raise RuntimeError(f"{_GPU_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_GPU_LIB)
        sp = ctypes.POINTER(SynthSpec)
        for name in ("synth_gpu_fill_f32", "synth_gpu_fill_bf16"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_void_p, _i64, _i64, sp, ctypes.c_void_p]
        L.synth_gpu_fill_u16.restype = ctypes.c_int
        L.synth_gpu_fill_u16.argtypes = [ctypes.c_void_p, _i64, ctypes.c_uint16, ctypes.c_void_p]
        _gpu = L
    return _gpu


def _thresh(p):
    return int(min(max(round(p * 2.0**32), 0), 2**32 - 1))


def key(seed, stream, step):
    return int(cpu_lib().synth_cpu_key(seed, stream, step))


def spec(seed, stream, step, sigma, valid_hi=2**62, tail_sigma=0.0, tail_prob=0.0,
         zero_prob=0.0):
    s = SynthSpec()
    s.key = key(seed, stream, step)
    s.zero_key = key(seed, STREAM_ZERO_MASK, 0)
    s.sigma = sigma
    s.tail_sigma = tail_sigma
    s.tail_thresh = _thresh(tail_prob)
    s.zero_thresh = _thresh(zero_prob)
    s.valid_hi = valid_hi
    return s


# ---------------------------------------------------------------- host build


def _fill_threaded(fn, out, base, sp, threads):
    """fn(ptr, n, base, spec) over contiguous slices of out on `threads` host
    threads (the foreign call releases the GIL); element j is always the
    value of global index base + j."""
    n = out.size
    if threads <= 1 or n < (1 << 20):
        fn(out.ctypes.data, n, base, ctypes.byref(sp))
        return out
    from concurrent.futures import ThreadPoolExecutor
    step = (n + threads - 1) // threads
    item = out.itemsize

    def part(k):
        lo = k * step
        hi = min(n, lo + step)
        if hi > lo:
            fn(out.ctypes.data + lo * item, hi - lo, base + lo, ctypes.byref(sp))

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(part, range(threads)))
    return out


def cpu_f32(n, base, sp, threads=1):
    out = np.empty(n, dtype=np.float32)
    return _fill_threaded(cpu_lib().synth_cpu_fill_f32, out, base, sp, threads)


def cpu_bf16(n, base, sp, threads=1):
    out = np.empty(n, dtype=np.uint16)
    return _fill_threaded(cpu_lib().synth_cpu_fill_bf16, out, base, sp, threads)


def cpu_at_f32(idx, sp):
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.float32)
    cpu_lib().synth_cpu_at_f32(out.ctypes.data, idx.ctypes.data, idx.size, ctypes.byref(sp))
    return out


def cpu_at_bf16(idx, sp):
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.uint16)
    cpu_lib().synth_cpu_at_bf16(out.ctypes.data, idx.ctypes.data, idx.size, ctypes.byref(sp))
    return out


# ---------------------------------------------------------------- GPU build


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def gpu_f32(t, base, sp, stream=None):
    """Fill the float32 CUDA tensor ``t`` (contiguous) with the values of global
    indices base .. base + t.numel() - 1."""
    import torch
    assert t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()
    rc = gpu_lib().synth_gpu_fill_f32(t.data_ptr(), t.numel(), base, ctypes.byref(sp),
                                      _stream_handle(stream))
    if rc != 0:
        raise RuntimeError("synth_gpu_fill_f32 launch failed")


def gpu_bf16(t, base, sp, stream=None):
    import torch
    assert t.is_cuda and t.dtype in (torch.bfloat16, torch.int16, torch.uint16) and t.is_contiguous()
    rc = gpu_lib().synth_gpu_fill_bf16(t.data_ptr(), t.numel(), base, ctypes.byref(sp),
                                       _stream_handle(stream))
    if rc != 0:
        raise RuntimeError("synth_gpu_fill_bf16 launch failed")


def gpu_fill_u16(t, value, stream=None):
    assert t.is_cuda and t.element_size() == 2 and t.is_contiguous()
    rc = gpu_lib().synth_gpu_fill_u16(t.data_ptr(), t.numel(), value & 0xFFFF,
                                      _stream_handle(stream))
    if rc != 0:
        raise RuntimeError("synth_gpu_fill_u16 launch failed")


# ---------------------------------------------------------------- workloads


@dataclass
class Workload:
    """One synthetic workload: model shape, world size, owned rank, plan layout,
    value distributions and AdamW hyperparameters."""
    name: str
    numels: list
    world: int
    rank: int
    layout: str = "flat"  # "flat" | "per_tensor"
    align: int = 1
    master_sigma: float = 0.02
    contrib_sigma: float = 1e-3
    zero_prob: float = 0.0
    tail_prob: float = 0.0
    tail_sigma: float = 0.1
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    first_step: int = 1  # AdamW step t of the first measured step
    warm_steps: int = 0  # steps run from m = v = 0 before the measured one
    steps: int = 1
    bucket_elems: int = 0  # reduce bucket size in owned elements (0: one call)
    seed: int = DEFAULT_SEED
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def master_spec(self, valid_hi=2**62):
        return spec(self.seed, STREAM_MASTER, 0, self.master_sigma, valid_hi)

    def contrib_spec(self, q, step, valid_hi=2**62):
        return spec(self.seed, STREAM_CONTRIB + q, step, self.contrib_sigma, valid_hi,
                    self.tail_sigma, self.tail_prob, self.zero_prob)


def workloads():
    from .shapes import llama_7b, llama_70b, qwen25_3b, tiny
    return {
        "tiny": Workload("tiny", tiny(), 4, 1, "flat", 1, steps=3,
                         notes="1,000,003-elem fp32 param padded to N*8, N=4, rank 1, 3 steps"),
        "qwen3b": Workload("qwen3b", qwen25_3b(), 4, 0, "flat", 128, warm_steps=1, first_step=2,
                           notes="Qwen2.5-3B shape flattened with 128-elem alignment, N=4, rank 0; "
                                 "m/v from one warm step, measured step t=2"),
        "llama7b": Workload("llama7b", llama_7b(), 8, 0, "flat", 128, zero_prob=0.01, steps=10,
                            bucket_elems=25_000_000,
                            notes="Llama-7B shape, N=8, rank 0; 1% shared exact zeros; "
                                  "reduce in 25M-elem buckets; steps 1..10"),
        "llama7b_wrap": Workload("llama7b_wrap", llama_7b(), 8, 0, "per_tensor", 1,
                                 notes="Llama-7B shape wrapped per tensor (291 pieces), N=8, rank 0, "
                                       "multi-tensor apply"),
        "llama70b": Workload("llama70b", llama_70b(), 64, 0, "flat", 128, tail_prob=0.001,
                             tail_sigma=0.1,
                             notes="Llama-70B shape, N=64, rank 0; 0.1% heavy-tail N(0,0.1) draws; "
                                   "fused reduce+AdamW+gather"),
    }
