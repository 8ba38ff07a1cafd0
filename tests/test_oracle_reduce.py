"""Pins of the oracle's averaged reduce (the reduce-scatter share of one rank).

Special cases with exact answers, a brute-force exact average in float64 with
the error bound of a sequential fp32 sum, and IEEE facts about signed zeros
and non-finite values.
"""
import numpy as np
import pytest
import torch


def _bf16_random(rng, n, sigma):
    x = (rng.standard_normal(n) * sigma).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 8, 64])
def test_identical_contributions_average_to_themselves(ora, N):
    rng = np.random.default_rng(N)
    x = _bf16_random(rng, 4096, 1e-3)
    g = ora.reduce([x.copy() for _ in range(N)])
    assert np.array_equal(g, x)


@pytest.mark.parametrize("N", [2, 4, 8, 64])
def test_single_nonzero_rank_is_divided_exactly(ora, N):
    rng = np.random.default_rng(10 + N)
    x = _bf16_random(rng, 4096, 1.0)
    for k in (0, N - 1):
        cs = [np.zeros(4096, np.uint16) for _ in range(N)]
        cs[k] = x
        g = ora.reduce(cs)
        want = (ora.bf16_to_f32(x) / np.float32(N)).astype(np.float32)  # exact: power of two
        assert np.array_equal(ora.bf16_to_f32(g), want)


@pytest.mark.parametrize("N", [3, 4, 8, 64])
def test_against_exact_average(ora, N):
    rng = np.random.default_rng(100 + N)
    S = 20_000
    cs = [_bf16_random(rng, S, 1e-3) for _ in range(N)]
    g = ora.reduce(cs)
    vals = torch.stack([torch.from_numpy(ora.bf16_to_f32(c).astype(np.float64)) for c in cs])
    exact = vals.sum(0) / N  # exact in float64 for these magnitudes, then one rounding
    absum = vals.abs().sum(0) / N
    got = torch.from_numpy(ora.bf16_to_f32(g).astype(np.float64))
    # a sequential fp32 sum of N terms errs by at most (N-1) u sum|c| (u = 2^-24),
    # then the division and the bf16 narrowing add half a bf16 ulp each side.
    bf_ulp = torch.from_numpy(np.abs(ora.bf16_to_f32(g)).astype(np.float64)) * 2.0**-7
    bound = (N - 1) * 2.0**-24 * absum + 2.0**-24 * exact.abs() + 0.5 * bf_ulp + 0.5 * 2.0**-7 * exact.abs() + 1e-45
    assert bool(((got - exact).abs() <= bound).all())
    # and the bf16 result equals the library's rounding of the exact average
    # except where the fp32 sum sits within its error of a rounding boundary
    lib = torch.from_numpy(exact.numpy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.mean(lib == g) > 0.995


def test_signed_zero_sum_starts_from_plus_zero(ora):
    neg0 = np.full(64, 0x8000, dtype=np.uint16)
    assert np.all(ora.reduce([neg0, neg0, neg0]) == 0x0000)


def test_non_finite_propagate(ora):
    one = np.full(8, 0x3F80, np.uint16)
    inf = np.full(8, 0x7F80, np.uint16)
    ninf = np.full(8, 0xFF80, np.uint16)
    nan = np.full(8, 0x7FC0, np.uint16)
    assert np.all(ora.reduce([one, inf]) == 0x7F80)
    g = ora.reduce([inf, ninf])
    assert np.all((g & 0x7F80) == 0x7F80) and np.all(g & 0x7F)
    g = ora.reduce([one, nan, one])
    assert np.all((g & 0x7FC0) == 0x7FC0)


def test_range_only_touches_range(ora):
    rng = np.random.default_rng(7)
    cs = [_bf16_random(rng, 1000, 1e-3) for _ in range(4)]
    out = np.full(1000, 0xBEEF, np.uint16)
    ora.reduce(cs, 200, 520, out)
    full = ora.reduce(cs)
    assert np.all(out[:200] == 0xBEEF) and np.all(out[520:] == 0xBEEF)
    assert np.array_equal(out[200:520], full[200:520])
