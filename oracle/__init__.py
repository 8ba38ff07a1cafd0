"""CPU oracle for the shard-local step (reduce -> mixed-precision AdamW -> gather).

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's
CPU-baseline leg are its only users; the product library never imports it.

The element arithmetic lives in ``zs_oracle.c`` (plain C, one fp32 rounding per
operation); the integer shard plan lives in ``plan.py``. This module marshals
numpy arrays into the C functions. bf16 arrays are numpy ``uint16`` holding the
raw bit patterns.
"""

import ctypes
import os

import numpy as np

from .plan import OraclePlan, ReshardSlice, plan_flat, plan_per_tensor, reshard_slice, roundup  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libzs_oracle.so")
_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.ora_f32_to_bf16.restype = ctypes.c_uint16
        L.ora_f32_to_bf16.argtypes = [ctypes.c_float]
        L.ora_bf16_to_f32.restype = ctypes.c_float
        L.ora_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.ora_f32_to_bf16_array.argtypes = [_f32p, _u16p, _i64]
        L.ora_reduce.argtypes = [ctypes.POINTER(_u16p), _i32, _i64, _i64, _u16p]
        L.ora_adamw_coef.argtypes = [ctypes.c_double] * 5 + [_i64, _f32p]
        L.ora_adamw.argtypes = [_f32p, _u16p, _f32p, _f32p, _f32p, _u16p, _i64, _i64]
        L.ora_gather.argtypes = [_u16p, _i64, _i32, _i64, _i64, _u16p]
        L.ora_shard_step.argtypes = [_f32p, ctypes.POINTER(_u16p), _i32, _u16p, _f32p, _f32p, _f32p,
                                     _u16p, _u16p, _i64, _i32, _i64, _i64]
        L.ora_time_shard_step.restype = ctypes.c_int
        L.ora_time_shard_step.argtypes = [_f32p, ctypes.POINTER(_u16p), _i32, _u16p, _f32p, _f32p,
                                          _f32p, _u16p, _u16p, _i64, _i32, _i64, _i32, _i32,
                                          ctypes.POINTER(ctypes.c_double)]
        L.ora_accumulate.argtypes = [ctypes.POINTER(_u16p), _i32, _f32p, _i32, _i64, _i64]
        L.ora_grad_sumsq.restype = ctypes.c_double
        L.ora_grad_sumsq.argtypes = [_f32p, ctypes.c_float, _i64, _i64, ctypes.POINTER(_i32)]
        L.ora_clip_scale.restype = ctypes.c_float
        L.ora_clip_scale.argtypes = [ctypes.POINTER(ctypes.c_double), _i32, ctypes.c_double]
        L.ora_adamw_f32grad.argtypes = [_f32p, _f32p, ctypes.c_float, ctypes.c_float, _i32, _f32p, _f32p,
                                        _f32p, _u16p, _i64, _i64]
        _u8p = ctypes.POINTER(ctypes.c_uint8)
        L.ora_quantize.argtypes = [_u16p, _i64, _i32, _i32, _u8p, _f32p]
        L.ora_dequantize.argtypes = [_u8p, _f32p, _i64, _i32, _i32, _u16p]
        _lib = L
    return _lib


def _p16(a):
    assert a.dtype == np.uint16 and a.flags.c_contiguous
    return a.ctypes.data_as(_u16p)


def _p32(a):
    assert a.dtype == np.float32 and a.flags.c_contiguous
    return a.ctypes.data_as(_f32p)


def _contrib_table(contribs):
    arr = (_u16p * len(contribs))()
    for q, c in enumerate(contribs):
        arr[q] = _p16(c)
    return arr


# ---------------------------------------------------------------- bf16


def f32_to_bf16(x):
    """RNE narrowing of a float32 array (any shape) to bf16 bit patterns (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().ora_f32_to_bf16_array(_p32(x.reshape(-1)), _p16(out.reshape(-1)), x.size)
    return out


def bf16_to_f32(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- AdamW scalars


def adamw_coef(lr, beta1, beta2, eps, weight_decay, step):
    c = np.zeros(9, dtype=np.float32)
    lib().ora_adamw_coef(lr, beta1, beta2, eps, weight_decay, step, _p32(c))
    return c


class HParams:
    def __init__(self, lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1):
        self.lr, self.beta1, self.beta2 = lr, beta1, beta2
        self.eps, self.weight_decay, self.step = eps, weight_decay, step

    def coef(self):
        return adamw_coef(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay, self.step)

    def at(self, step):
        return HParams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay, step)


# ---------------------------------------------------------------- element ops


def reduce(contribs, lo=0, hi=None, out=None):
    """Averaged bf16 gradient over owned elements [lo, hi) of N bf16 contributions."""
    n = len(contribs)
    S = contribs[0].size
    hi = S if hi is None else hi
    for c in contribs:
        assert c.size == S
    out = np.zeros(S, dtype=np.uint16) if out is None else out
    lib().ora_reduce(_contrib_table(contribs), n, lo, hi, _p16(out))
    return out


def adamw(hp, g, master, m, v, p, lo=0, hi=None):
    """In-place AdamW on fp32 master/m/v; writes bf16 p. Arrays are 1-D, same length."""
    hi = g.size if hi is None else hi
    lib().ora_adamw(_p32(hp.coef()), _p16(g), _p32(master), _p32(m), _p32(v), _p16(p), lo, hi)


def gather(p, rank, full, lo=0, hi=None):
    S = p.size
    hi = S if hi is None else hi
    assert full.size >= (rank + 1) * S
    lib().ora_gather(_p16(p), S, rank, lo, hi, _p16(full))


def gather_to_slice(p, own_off, slice_buf):
    """The own updated bf16 shard p written into the kept k-way slice that
    holds it (plan.reshard_slice's owner_slice), at own_off; nothing else of
    the slice is touched."""
    assert own_off >= 0 and own_off + p.size <= slice_buf.size
    slice_buf[own_off:own_off + p.size] = p


def gather_slice(shards, slice_buf):
    """The receiving side of the group's gather: shard i (the updated shard of
    the slice's i-th source rank) at i*S of the kept slice."""
    S = shards[0].size
    assert len(shards) * S == slice_buf.size
    for i, sh in enumerate(shards):
        assert sh.size == S
        slice_buf[i * S:(i + 1) * S] = sh


def shard_step(hp, contribs, g, master, m, v, p, full, rank, lo=0, hi=None):
    S = g.size
    hi = S if hi is None else hi
    lib().ora_shard_step(_p32(hp.coef()), _contrib_table(contribs), len(contribs), _p16(g),
                         _p32(master), _p32(m), _p32(v), _p16(p),
                         _p16(full) if full is not None else None, S, rank, lo, hi)


def time_shard_step(hp, contribs, g, master, m, v, p, full, nthreads, reps):
    """Wall-clock seconds of ``reps`` whole-window shard steps over all of g's
    elements, split over ``nthreads`` host threads; the window is rank 0's, so
    its gather writes full[0:len(g)]."""
    S = g.size
    secs = (ctypes.c_double * reps)()
    rc = lib().ora_time_shard_step(_p32(hp.coef()), _contrib_table(contribs), len(contribs),
                                   _p16(g), _p32(master), _p32(m), _p32(v), _p16(p),
                                   _p16(full) if full is not None else None, S, 0, S, nthreads,
                                   reps, secs)
    if rc != 0:
        raise RuntimeError("oracle timing failed")
    return list(secs)


# ---------------------------------------------------------------- whole plans


def plan_step(plan, hp, contribs_by_piece, state_by_piece, full_by_tensor=None, hp_of_piece=None):
    """One shard step over every owned piece of a PER_TENSOR or FLAT plan.

    contribs_by_piece[i] is the list of N bf16 arrays of piece i (length = piece
    length); state_by_piece[i] = (g, master, m, v, p) arrays of piece i; the
    gathered tensor i (padded, T_i) receives the piece at own_lo when
    full_by_tensor is given. hp_of_piece optionally gives each piece its own
    hyperparameters (parameter groups).
    """
    for k, pc in enumerate(plan.pieces):
        g, master, m, v, p = state_by_piece[k]
        if g.size == 0:
            continue
        reduce(contribs_by_piece[k], out=g)
        adamw(hp if hp_of_piece is None else hp_of_piece[k], g, master, m, v, p)
        if full_by_tensor is not None:
            full_by_tensor[pc.tensor][pc.own_lo:pc.own_hi] = p


# ---------------------------------------------------------------- accumulation and clipping


def accumulate(contribs, acc, first, lo=0, hi=None):
    """acc += f32(bf16(average of the contributions)) (acc := that value when first)."""
    hi = acc.size if hi is None else hi
    lib().ora_accumulate(_contrib_table(contribs), len(contribs), _p32(acc), 1 if first else 0, lo, hi)


def grad_sumsq(acc, divisor=1.0):
    """(sum of (acc/divisor)^2 in double, nonfinite flag)."""
    flag = _i32(0)
    s = lib().ora_grad_sumsq(_p32(acc), divisor, 0, acc.size, ctypes.byref(flag))
    return s, flag.value


def clip_scale(sumsq_per_rank, max_norm):
    arr = (ctypes.c_double * len(sumsq_per_rank))(*sumsq_per_rank)
    return lib().ora_clip_scale(arr, len(sumsq_per_rank), max_norm)


def adamw_f32grad(hp, acc, divisor, scale, skip, master, m, v, p, lo=0, hi=None):
    hi = acc.size if hi is None else hi
    lib().ora_adamw_f32grad(_p32(hp.coef()), _p32(acc), divisor, scale, 1 if skip else 0, _p32(master),
                            _p32(m), _p32(v), _p16(p), lo, hi)


# ---------------------------------------------------------------- quantized parameter gather


def quant_bytes(n, bits):
    """Code bytes of n elements at ``bits`` (8 or 4) per element."""
    return n if bits == 8 else (n + 1) // 2


def quant_blocks(n, block):
    return -(-n // block)


def _p8(a):
    assert a.dtype == np.uint8 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def quantize(p, bits, block):
    """Block-wise symmetric quantization of a bf16 (uint16) array: (codes uint8, scales float32)."""
    if bits not in (4, 8) or block < 1:
        raise ValueError("bits must be 4 or 8 and block >= 1")
    p = np.ascontiguousarray(p, dtype=np.uint16)
    q = np.zeros(quant_bytes(p.size, bits), np.uint8)
    sc = np.zeros(quant_blocks(p.size, block), np.float32)
    lib().ora_quantize(_p16(p), p.size, bits, block, _p8(q), _p32(sc))
    return q, sc


def dequantize(q, scales, n, bits, block):
    """bf16 (uint16) array of n elements from codes and block scales."""
    out = np.zeros(n, np.uint16)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    assert q.size >= quant_bytes(n, bits) and scales.size >= quant_blocks(n, block)
    lib().ora_dequantize(_p8(q), _p32(scales), n, bits, block, _p16(out))
    return out


def dequant_gather(q_all, scales_all, S, world, bits, block):
    """Gathered bf16 buffer of world*S elements from every rank's payload, laid
    end to end in rank order (codes: world * quant_bytes(S) bytes; scales:
    world * quant_blocks(S) floats)."""
    qb, nb = quant_bytes(S, bits), quant_blocks(S, block)
    return np.concatenate([dequantize(q_all[r * qb:(r + 1) * qb], scales_all[r * nb:(r + 1) * nb], S, bits, block)
                           for r in range(world)]) if world else np.zeros(0, np.uint16)
