"""Pins of the oracle's mixed-precision AdamW.

The pages give no AdamW value, so the update is pinned by closed forms and
invariants of decoupled-weight-decay Adam with bias correction, and by a
library routine: PyTorch's CPU ``torch.optim.AdamW`` run in float64, which
applies the same textbook algorithm with its own operation order.
"""
import numpy as np
import pytest
import torch

from oracle import HParams


def _state(rng, n, sigma=0.02):
    master = (rng.standard_normal(n) * sigma).astype(np.float32)
    return master, np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)


def _bf16(rng, n, sigma):
    x = (rng.standard_normal(n) * sigma).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_step1_closed_form_is_sign_step(ora):
    # m = v = 0, t = 1: mhat = g, vhat = g^2, so with wd = 0 the step is
    # -lr * g / (|g| + eps) -> -lr * sign(g) when eps << |g|.
    rng = np.random.default_rng(1)
    n = 50_000
    master, m, v, p = _state(rng, n)
    g = _bf16(rng, n, 1e-3)
    gf = ora.bf16_to_f32(g).astype(np.float64)
    keep = gf != 0
    p0 = master.astype(np.float64).copy()
    hp = HParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, step=1)
    ora.adamw(hp, g, master, m, v, p)
    delta = master.astype(np.float64) - p0
    err = np.abs(delta + hp.lr * np.sign(gf))
    bound = hp.lr * hp.eps / np.abs(gf[keep]) + 8 * 2.0**-24 * (np.abs(p0[keep]) + hp.lr)
    assert np.all(err[keep] <= bound)
    # the moments hold (1-b1) g and (1-b2) g^2 exactly as fp32 products
    assert np.array_equal(m, (np.float32(0.1) * ora.bf16_to_f32(g)).astype(np.float32))
    assert np.array_equal(v, np.float32(1 - 0.95) * (ora.bf16_to_f32(g) * ora.bf16_to_f32(g)))
    # where g == 0 the update is exactly zero
    assert np.array_equal(master[~keep], p0[~keep].astype(np.float32))
    # and the bf16 parameter is the rounding of the new master weight
    assert np.array_equal(p, ora.f32_to_bf16(master))


def test_zero_grad_is_pure_decay(ora):
    rng = np.random.default_rng(2)
    n = 10_000
    master, m, v, p = _state(rng, n)
    g = np.zeros(n, np.uint16)
    p0 = master.copy()
    hp = HParams(lr=1e-2, weight_decay=0.5)
    decay32 = np.float32(1 - 1e-2 * 0.5)
    it = p0.copy()
    for t in range(1, 11):
        ora.adamw(hp.at(t), g, master, m, v, p)
        it = (it * decay32).astype(np.float32)
        assert not m.any() and not v.any()
        assert np.array_equal(master, it)  # the iterated fp32 product
        closed = p0.astype(np.float64) * (1 - 1e-2 * 0.5) ** t
        assert np.all(np.abs(master - closed) <= (t + 1) * 2.0**-23 * np.abs(closed) + 1e-45)


def test_no_decay_no_grad_is_identity(ora):
    rng = np.random.default_rng(3)
    master, m, v, p = _state(rng, 4096)
    p0 = master.copy()
    hp = HParams(weight_decay=0.0)
    for t in range(1, 4):
        ora.adamw(hp.at(t), np.zeros(4096, np.uint16), master, m, v, p)
    assert np.array_equal(master, p0)


def test_lr_zero_keeps_master_but_moves_moments(ora):
    rng = np.random.default_rng(4)
    master, m, v, p = _state(rng, 4096)
    p0 = master.copy()
    g = _bf16(rng, 4096, 1e-3)
    ora.adamw(HParams(lr=0.0, weight_decay=0.1), g, master, m, v, p)
    assert np.array_equal(master, p0)
    assert np.array_equal(m != 0, g != 0)


def test_padding_stays_zero(ora):
    z = np.zeros(64, np.float32)
    master, m, v = z.copy(), z.copy(), z.copy()
    p = np.full(64, 0xFFFF, np.uint16)
    for t in range(1, 5):
        ora.adamw(HParams().at(t), np.zeros(64, np.uint16), master, m, v, p)
    for a in (master, m, v):
        assert np.all(a.view(np.uint32) == 0)  # +0 exactly
    assert np.all(p == 0)


@pytest.mark.parametrize("lr,wd,eps,b1,b2", [
    (1e-4, 0.1, 1e-8, 0.9, 0.95),
    (1e-2, 0.5, 1e-3, 0.8, 0.9),  # large eps and decay: placement of both shows
    (3e-3, 0.0, 1e-6, 0.5, 0.999),
])
def test_against_torch_adamw_float64(ora, lr, wd, eps, b1, b2):
    rng = np.random.default_rng(5)
    n, steps = 10_000, 10
    master, m, v, p = _state(rng, n)
    w64 = torch.nn.Parameter(torch.from_numpy(master.astype(np.float64)))
    opt = torch.optim.AdamW([w64], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    hp = HParams(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd)
    for t in range(1, steps + 1):
        g = _bf16(rng, n, 1e-3)
        ora.adamw(hp.at(t), g, master, m, v, p)
        w64.grad = torch.from_numpy(ora.bf16_to_f32(g).astype(np.float64))
        opt.step()
        ref = w64.detach().numpy()
        st = opt.state[w64]
        # fp32 state against float64: a few fp32 roundings per step, accumulated
        tol_w = 4 * t * 2.0**-24 * (np.abs(ref) + lr * 1.0) + lr * 1e-6
        assert np.all(np.abs(master - ref) <= tol_w), np.max(np.abs(master - ref) / tol_w)
        mref = st["exp_avg"].numpy()
        vref = st["exp_avg_sq"].numpy()
        assert np.max(np.abs(m - mref)) <= 4 * t * 2.0**-24 * 4e-3
        assert np.max(np.abs(v - vref)) <= 4 * t * 2.0**-24 * 2e-5
    # a wrong sign, a missing bias correction or a dropped decay moves master
    # by ~lr per step, orders of magnitude above these tolerances.


def test_non_finite_propagates(ora):
    master = np.array([0.01, 0.02], np.float32)
    m = np.zeros(2, np.float32)
    v = np.zeros(2, np.float32)
    p = np.zeros(2, np.uint16)
    g = np.array([0x7FC0, 0x3F80], np.uint16)  # NaN, 1.0
    ora.adamw(HParams(), g, master, m, v, p)
    assert np.isnan(master[0]) and np.isfinite(master[1])
    assert (p[0] & 0x7FC0) == 0x7FC0
