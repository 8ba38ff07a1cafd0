"""Helpers shared by the GPU parity tests: host<->device marshalling and the
tolerance checks (fp32 state: relative error <= 1e-6 and exact where the
oracle gives 0; bf16: at most 1 ulp apart with the same sign; NaN where the
oracle has NaN).

NaN sign and payload are not compared: IEEE 754 leaves the NaN an invalid
operation produces unspecified, and x86 (the oracle's host) produces the
negative default NaN where CDNA produces the positive one. The returned
counts of non-bit-identical elements therefore cover non-NaN elements only."""
import numpy as np

F32_RTOL = 1e-6
BF16_ULPS = 1


def dev16(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def dev32(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host16(t):
    return t.detach().cpu().numpy().view(np.uint16)


def host32(t):
    return t.detach().cpu().numpy()


def _ordered16(h):
    h = h.astype(np.int32)
    return np.where(h & 0x8000, -(h & 0x7FFF), h)


def check_bf16(gpu, ora, what):
    """Returns the number of elements that are not bit-identical."""
    gpu = np.asarray(gpu, dtype=np.uint16)
    ora = np.asarray(ora, dtype=np.uint16)
    assert gpu.shape == ora.shape, what
    nan_o = (ora & 0x7F80) == 0x7F80
    nan_o &= (ora & 0x7F) != 0
    nan_g = ((gpu & 0x7F80) == 0x7F80) & ((gpu & 0x7F) != 0)
    assert np.array_equal(nan_o, nan_g), f"{what}: NaN positions differ"
    fin = ~nan_o
    d = np.abs(_ordered16(gpu[fin]) - _ordered16(ora[fin]))
    same_sign = ((gpu[fin] ^ ora[fin]) & 0x8000) == 0
    bad = (d > BF16_ULPS) | (~same_sign & (d > 0))
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} elements beyond {BF16_ULPS} ulp, e.g. idx {i} "
                             f"gpu {gpu[fin][i]} ora {ora[fin][i]}")
    return int((gpu[fin] != ora[fin]).sum())


def check_f32(gpu, ora, what):
    """Returns the number of elements that are not bit-identical."""
    gpu = np.asarray(gpu, dtype=np.float32)
    ora = np.asarray(ora, dtype=np.float32)
    assert gpu.shape == ora.shape, what
    nan_o, nan_g = np.isnan(ora), np.isnan(gpu)
    assert np.array_equal(nan_o, nan_g), f"{what}: NaN positions differ"
    fin = ~nan_o
    o = ora[fin].astype(np.float64)
    g = gpu[fin].astype(np.float64)
    zero = o == 0
    assert np.all(g[zero] == 0), f"{what}: nonzero where the oracle is 0"
    with np.errstate(invalid="ignore"):
        rel = np.abs(g - o) / np.abs(o)
    rel[zero] = 0
    inf = np.isinf(o)
    rel[inf] = np.where(g[inf] == o[inf], 0.0, np.inf)
    if np.any(rel > F32_RTOL):
        i = np.flatnonzero(rel > F32_RTOL)[:5]
        raise AssertionError(f"{what}: max rel err {rel.max():.3g} > {F32_RTOL}, e.g. idx {i}")
    return int((gpu[fin].view(np.uint32) != ora[fin].view(np.uint32)).sum())
