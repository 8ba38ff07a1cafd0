"""Pins of the oracle's block-wise quantizer for the parameter gather.

ZeRO++ moves the gathered parameters as 4-bit codes for up to four times less
traffic ("ZeRO vs FSDP: A Rigorous Dissection...", section 5.2). The oracle's
reading is symmetric block-wise quantization with an fp32 scale per block.
What fixes it here, independently of its own code:

* hand-worked cases (tests/golden/quant_cases.txt): ties to even, nibble order,
  the zero block, the ragged last block, the NaN block, an inexact scale;
* exact round trips on grids the codes can represent;
* every code is a nearest level of the block's grid, checked with exact
  rational arithmetic;
* the reconstruction error bound of half a grid step (plus the bf16 rounding);
* sign symmetry and the page's "up to 4x" payload ratio.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_cases.txt")


def _cases():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "case":
            cur = dict(bits=int(vals[0]), block=int(vals[1]), n=int(vals[2]))
            cases.append(cur)
        else:
            cur[key] = [int(v, 16) for v in vals]
    return cases


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"int{c['bits']}_B{c['block']}_n{c['n']}")
def test_hand_worked_cases(case):
    p = np.array(case["in"], np.uint16)
    q, sc = oracle.quantize(p, case["bits"], case["block"])
    assert list(q) == case["codes"]
    assert list(sc.view(np.uint32)) == case["scales"]
    out = oracle.dequantize(q, sc, case["n"], case["bits"], case["block"])
    assert list(out) == case["out"]


@pytest.mark.parametrize("bits", [4, 8])
def test_exact_grid_round_trips(bits):
    """Values k * 2^e with |k| <= qmax and qmax present: scale = 2^e exactly,
    codes = k, dequantized values identical to the inputs."""
    qmax = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(bits)
    B = 64
    for e in (-20, -10, 0, 3):
        k = rng.integers(-qmax, qmax + 1, 4 * B)
        k[::B] = qmax * np.where(rng.random(4) < 0.5, 1, -1)  # each block reaches +-qmax
        x = (k * 2.0**e).astype(np.float32)
        p = oracle.f32_to_bf16(x)
        assert np.array_equal(oracle.bf16_to_f32(p), x)  # |k| <= 127 fits bf16's 8 significant bits
        q, sc = oracle.quantize(p, bits, B)
        assert np.all(sc == np.float32(2.0**e))
        back = oracle.dequantize(q, sc, p.size, bits, B)
        assert np.array_equal(back, p)


def _codes(q, n, bits):
    if bits == 8:
        return q[:n].view(np.int8).astype(np.int64)
    lo = (q & 0xF).astype(np.int64)
    hi = (q >> 4).astype(np.int64)
    c = np.empty(2 * q.size, np.int64)
    c[0::2], c[1::2] = lo, hi
    c = c[:n]
    return np.where(c >= 8, c - 16, c)


@pytest.mark.parametrize("bits,B", [(4, 32), (4, 256), (8, 64), (8, 128)])
def test_codes_are_nearest_levels(bits, B):
    """Exact rational check: code k minimizes |x - k*scale| over [-qmax, qmax]
    up to the rounding of the fp32 quotient (a tie may only be decided the
    other way when the exact quotient lies within one fp32 ulp of a half)."""
    qmax = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(100 + bits + B)
    x = (rng.standard_normal(3 * B + 24) * 0.02).astype(np.float32)
    x[rng.random(x.size) < 0.01] *= 50  # heavy tail
    p = oracle.f32_to_bf16(x)
    q, sc = oracle.quantize(p, bits, B)
    k = _codes(q, p.size, bits)
    xv = oracle.bf16_to_f32(p)
    for j in range(p.size):
        s = Fraction(float(sc[j // B]))
        xf = Fraction(float(xv[j]))
        exact = xf / s
        best = min(range(-qmax, qmax + 1), key=lambda c: (abs(xf - c * s), c % 2))
        if k[j] != best:
            half = Fraction(2 * int(np.floor(exact)) + 1, 2)
            assert abs(exact - half) <= Fraction(2) ** -21 * abs(exact), (j, float(exact), k[j], best)


@pytest.mark.parametrize("bits", [4, 8])
def test_error_bound_and_extremes(bits):
    qmax = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(7 + bits)
    B = 128
    x = (rng.standard_normal(40 * B + 40) * 0.02).astype(np.float32)
    p = oracle.f32_to_bf16(x)
    q, sc = oracle.quantize(p, bits, B)
    k = _codes(q, p.size, bits)
    back = oracle.bf16_to_f32(oracle.dequantize(q, sc, p.size, bits, B)).astype(np.float64)
    xv = oracle.bf16_to_f32(p).astype(np.float64)
    s = np.repeat(sc.astype(np.float64), B)[:p.size]
    # half a grid step (plus the quotient's rounding) and the final bf16 rounding
    assert np.all(np.abs(back - xv) <= s * (0.5 + 2.0**-20) + np.abs(back) * 2.0**-8)
    assert np.all(np.abs(k) <= qmax)
    for b in range(sc.size):
        blk = xv[b * B:(b + 1) * B]
        i = int(np.argmax(np.abs(blk)))
        assert abs(k[b * B + i]) == qmax  # the largest element maps to the end of the grid
        assert sc[b] == np.float32(np.max(np.abs(blk)) / np.float32(qmax))


@pytest.mark.parametrize("bits", [4, 8])
def test_sign_symmetry(bits):
    rng = np.random.default_rng(11)
    p = oracle.f32_to_bf16((rng.standard_normal(1000) * 0.02).astype(np.float32))
    neg = p ^ np.uint16(0x8000)
    q1, s1 = oracle.quantize(p, bits, 64)
    q2, s2 = oracle.quantize(neg, bits, 64)
    assert np.array_equal(s1, s2)
    assert np.array_equal(_codes(q1, 1000, bits), -_codes(q2, 1000, bits))


def test_zero_and_non_finite_blocks_are_local():
    B = 16
    x = np.full(4 * B, 0.01, np.float32)
    x[B:2 * B] = 0.0
    x[2 * B + 3] = np.inf
    p = oracle.f32_to_bf16(x)
    p[3 * B + 5] = 0x7FC0  # NaN in block 3
    for bits in (4, 8):
        q, sc = oracle.quantize(p, bits, B)
        out = oracle.bf16_to_f32(oracle.dequantize(q, sc, p.size, bits, B))
        assert sc[1] == 0.0 and np.all(out[B:2 * B] == 0.0)
        assert np.isnan(sc[2]) and np.isnan(sc[3]) and np.all(np.isnan(out[2 * B:]))
        assert np.all(np.abs(out[:B] - 0.01) <= 0.01 / ((1 << (bits - 1)) - 1) / 2 + 1e-4)


def test_payload_ratio_matches_the_four_times_claim():
    """4-bit codes plus one fp32 scale per 256 elements move 3.88x fewer bytes
    than bf16; the ratio tends to 4 as the block grows (the pages' "up to 4x")."""
    n = 1 << 20
    bf16_bytes = 2 * n
    for B, lo in ((64, 3.55), (256, 3.87), (4096, 3.99)):
        payload = oracle.quant_bytes(n, 4) + 4 * oracle.quant_blocks(n, B)
        assert lo < bf16_bytes / payload < 4.0
    assert bf16_bytes / (oracle.quant_bytes(n, 8) + 4 * oracle.quant_blocks(n, 256)) < 2.0


def test_dequant_gather_places_ranks_in_order():
    S, N, bits, B = 96, 4, 4, 32
    rng = np.random.default_rng(3)
    shards = [oracle.f32_to_bf16((rng.standard_normal(S) * (r + 1)).astype(np.float32)) for r in range(N)]
    pay = [oracle.quantize(s, bits, B) for s in shards]
    full = oracle.dequant_gather(np.concatenate([q for q, _ in pay]), np.concatenate([s for _, s in pay]), S, N,
                                 bits, B)
    for r in range(N):
        assert np.array_equal(full[r * S:(r + 1) * S], oracle.dequantize(*pay[r], S, bits, B))
