"""Pins of the oracle's gradient accumulation, global-norm clipping and
non-finite skip.

Checked against exact special cases, float64 library sums, PyTorch's
``torch.nn.utils.clip_grad_norm_`` and ``torch.optim.AdamW`` (float64), and
the already pinned bf16-gradient AdamW.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import HParams


def _bf16(rng, n, sigma):
    x = (rng.standard_normal(n) * sigma).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("G,N", [(1, 4), (3, 4), (8, 8), (5, 3)])
def test_identical_micro_batches(G, N):
    rng = np.random.default_rng(G * 10 + N)
    x = _bf16(rng, 4096, 1e-3)
    acc = np.full(4096, np.nan, np.float32)  # garbage: the first micro-step overwrites
    for k in range(G):
        oracle.accumulate([x] * N, acc, first=(k == 0))
    assert np.array_equal(acc, (oracle.bf16_to_f32(x) * np.float32(G)).astype(np.float32))
    final = acc / np.float32(G)
    assert np.array_equal(final, oracle.bf16_to_f32(x))


def test_accumulation_against_float64():
    rng = np.random.default_rng(1)
    G, N, n = 6, 4, 20_000
    acc = np.zeros(n, np.float32)
    exact = np.zeros(n, np.float64)
    for k in range(G):
        cs = [_bf16(rng, n, 1e-3) for _ in range(N)]
        oracle.accumulate(cs, acc, first=(k == 0))
        avg = torch.from_numpy(np.mean([oracle.bf16_to_f32(c).astype(np.float64) for c in cs], axis=0))
        micro = avg.to(torch.bfloat16).to(torch.float64).numpy()  # library RNE of the exact average
        exact += micro
    # fp32 running sum of G terms: error <= (G-1) u sum|terms| plus the rare
    # double rounding of a micro-average (at most one bf16 ulp of that term)
    bound = (G - 1) * 2.0**-24 * np.abs(exact) * 4 + np.abs(exact) * 2.0**-7
    assert np.all(np.abs(acc - exact) <= bound + 1e-30)
    assert np.mean(np.abs(acc - exact) <= G * 2.0**-24 * np.abs(exact) + 1e-30) > 0.99


def test_sumsq_against_float64_dot():
    rng = np.random.default_rng(2)
    acc = (rng.standard_normal(100_003) * 1e-3).astype(np.float32)
    for G in (1.0, 3.0, 4.0):
        s, flag = oracle.grad_sumsq(acc, G)
        g = (acc / np.float32(G)).astype(np.float64)
        ref = float(np.dot(g, g))
        assert flag == 0 and abs(s - ref) <= 1e-12 * ref


def test_sumsq_flags_non_finite():
    acc = np.ones(64, np.float32)
    assert oracle.grad_sumsq(acc)[1] == 0
    for bad in (np.nan, np.inf, -np.inf):
        a = acc.copy()
        a[37] = bad
        assert oracle.grad_sumsq(a)[1] == 1
    a = acc.copy()
    a[0] = 3e38
    assert oracle.grad_sumsq(a, 0.5)[1] == 1  # the final gradient overflows


def test_sharded_sumsq_adds_up():
    rng = np.random.default_rng(3)
    g = (rng.standard_normal(4 * 250_008) * 1e-3).astype(np.float32)
    parts = [oracle.grad_sumsq(g[r * 250_008:(r + 1) * 250_008])[0] for r in range(4)]
    whole = oracle.grad_sumsq(g)[0]
    assert abs(sum(parts) - whole) <= 1e-12 * whole


@pytest.mark.parametrize("max_norm", [1e-3, 0.05, 10.0])
def test_clip_scale_against_torch(max_norm):
    rng = np.random.default_rng(4)
    shards = [(rng.standard_normal(5000) * 1e-3).astype(np.float32) for _ in range(4)]
    sumsq = [oracle.grad_sumsq(s)[0] for s in shards]
    scale = oracle.clip_scale(sumsq, max_norm)
    params = [torch.nn.Parameter(torch.zeros(5000, dtype=torch.float64)) for _ in shards]
    for p, s in zip(params, shards):
        p.grad = torch.from_numpy(s.astype(np.float64))
    torch.nn.utils.clip_grad_norm_(params, max_norm)
    ref = params[0].grad.numpy() / shards[0].astype(np.float64)
    ref_scale = float(np.median(ref))
    assert abs(scale - ref_scale) <= 2.0**-23 * ref_scale
    if max_norm >= 10.0:
        assert scale == 1.0


def test_no_clip_equals_plain_adamw():
    rng = np.random.default_rng(5)
    n = 10_000
    g = _bf16(rng, n, 1e-3)
    acc = np.zeros(n, np.float32)
    oracle.accumulate([g, g], acc, first=True)  # average of two identical contributions = g
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    a = [master.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)]
    b = [master.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)]
    sumsq, _ = oracle.grad_sumsq(acc)
    scale = oracle.clip_scale([sumsq], 1.0)
    assert scale == 1.0
    for t in (1, 2, 3):
        oracle.adamw_f32grad(HParams().at(t), acc, 1.0, scale, False, *a)
        oracle.adamw(HParams().at(t), g, *b)
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()


def test_skip_leaves_state_unchanged():
    rng = np.random.default_rng(6)
    n = 512
    acc = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    st = [(rng.standard_normal(n) * 0.02).astype(np.float32), rng.random(n).astype(np.float32),
          rng.random(n).astype(np.float32), np.arange(n, dtype=np.uint16)]
    before = [x.tobytes() for x in st]
    oracle.adamw_f32grad(HParams(), acc, 1.0, 1.0, True, *st)
    assert [x.tobytes() for x in st] == before


def test_accumulate_clip_adamw_against_torch():
    """Three micro-batches of four ranks' contributions, global-norm clip, AdamW: float64 PyTorch."""
    rng = np.random.default_rng(7)
    n, N, G, steps, max_norm = 8_000, 4, 3, 5, 0.02
    lr, wd = 1e-3, 0.1
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m, v, p = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    w64 = torch.nn.Parameter(torch.from_numpy(master.astype(np.float64)))
    opt = torch.optim.AdamW([w64], lr=lr, betas=(0.9, 0.95), eps=1e-8, weight_decay=wd, foreach=False)
    acc = np.zeros(n, np.float32)
    hp = HParams(lr=lr, weight_decay=wd)
    clipped_any = False
    for t in range(1, steps + 1):
        micro64 = np.zeros(n, np.float64)
        for k in range(G):
            cs = [_bf16(rng, n, 1e-3) for _ in range(N)]
            oracle.accumulate(cs, acc, first=(k == 0))
            avg = torch.from_numpy(np.mean([oracle.bf16_to_f32(c).astype(np.float64) for c in cs], axis=0))
            micro64 += avg.to(torch.bfloat16).to(torch.float64).numpy()
        sumsq, flag = oracle.grad_sumsq(acc, float(G))
        scale = oracle.clip_scale([sumsq], max_norm)
        clipped_any |= scale < 1.0
        oracle.adamw_f32grad(hp.at(t), acc, float(G), scale, flag != 0, master, m, v, p)
        w64.grad = torch.from_numpy(micro64 / G)
        torch.nn.utils.clip_grad_norm_([w64], max_norm)
        opt.step()
        ref = w64.detach().numpy()
        tol = 8 * t * 2.0**-24 * (np.abs(ref) + lr) + lr * 1e-5
        assert np.all(np.abs(master - ref) <= tol), np.max(np.abs(master - ref) / tol)
    assert clipped_any
