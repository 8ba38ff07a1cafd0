"""Pins of the oracle's fp32 -> bf16 narrowing (IEEE round to nearest, ties to even).

* hand-derived cases from the rounding rule (tests/golden/bf16_rne_cases.txt);
* every one of the 2^32 fp32 bit patterns that is not a NaN against a library
  routine (PyTorch's CPU float32 -> bfloat16 conversion, round to nearest even);
* every NaN class keeps NaN-ness, sign and gets its quiet bit;
* a brute-force nearest-even search in double on a random sample.
"""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_rne_cases.txt")


def _bits_to_f32(u):
    return np.asarray(u, dtype=np.uint32).view(np.float32)


def test_hand_cases(ora):
    n = 0
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            src, want, *_ = line.split()
            x = _bits_to_f32(np.array([int(src, 16)], dtype=np.uint32))
            got = int(ora.f32_to_bf16(x)[0])
            assert got == int(want, 16), f"{src}: got {got:04X}, want {want}"
            n += 1
    assert n >= 20


def test_exhaustive_non_nan_vs_torch(ora):
    import ctypes
    L = ora.lib()
    chunk = 1 << 24
    base = np.arange(chunk, dtype=np.uint32)
    u = np.empty(chunk, dtype=np.uint32)
    ours = np.empty(chunk, dtype=np.uint16)
    ref = torch.empty(chunk, dtype=torch.bfloat16)
    ref_bits = ref.view(torch.int16).numpy().view(np.uint16)
    x = torch.from_numpy(u.view(np.float32))
    pf = u.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    ph = ours.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))
    for start in range(0, 1 << 32, chunk):
        np.add(base, np.uint32(start), out=u)
        L.ora_f32_to_bf16_array(pf, ph, chunk)
        ref.copy_(x)  # library conversion, round to nearest even
        diff = ours != ref_bits
        if diff.any():
            nan = (u & 0x7FFFFFFF) > 0x7F800000
            bad = diff & ~nan
            assert not bad.any(), f"mismatch at bits {u[bad][:4]}"


def test_nan_classes(ora):
    rng = np.random.default_rng(1)
    payload = rng.integers(1, 1 << 23, size=1 << 16, dtype=np.uint32)
    for sign in (0, 0x80000000):
        u = (np.uint32(sign) | np.uint32(0x7F800000) | payload).astype(np.uint32)
        out = ora.f32_to_bf16(u.view(np.float32)).astype(np.uint32)
        assert np.all((out & 0x7F80) == 0x7F80)  # exponent all ones
        assert np.all(out & 0x0040)  # quiet
        assert np.all((out & 0x8000) == (sign >> 16))  # sign kept


def test_nearest_even_brute_force_sample(ora):
    # Independent of the carry trick: find both bf16 neighbours in double and
    # pick the nearer, ties to the even kept half.
    # Magnitudes only; the sign is copied. The upper neighbour is the lower one
    # plus one bf16 ulp in double, so above the largest finite bf16 it is 2^128
    # and choosing it means overflow to infinity, as IEEE rounding requires.
    rng = np.random.default_rng(2)
    u = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate([u, np.arange(0x7F7F0000, 0x7F800000, 97, dtype=np.uint32)])
    u = u[(u & 0x7F800000) != 0x7F800000]  # finite only
    sign = (u >> 16) & 0x8000
    a = u & 0x7FFFFFFF
    x = a.view(np.float32).astype(np.float64)
    down = (a >> 16).astype(np.int64)  # truncation toward zero
    e = (down >> 7) & 0xFF
    ulp = np.ldexp(1.0, np.maximum(e, 1) - 134)
    xd = (down.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xu = xd + ulp
    dd = x - xd
    du = xu - x
    pick_up = (du < dd) | ((du == dd) & ((down & 1) == 1))
    want = (np.where(pick_up, down + 1, down) | sign).astype(np.uint16)
    got = ora.f32_to_bf16(u.view(np.float32))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("h", [0x0000, 0x8000, 0x0001, 0x3F80, 0xC2F7, 0x7F80, 0x7FC1])
def test_widen_is_exact(ora, h):
    x = ora.bf16_to_f32(np.array([h], dtype=np.uint16))
    assert (x.view(np.uint32)[0] >> 16) == h and (x.view(np.uint32)[0] & 0xFFFF) == 0
