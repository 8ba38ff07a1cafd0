"""Randomized GPU <-> oracle parity across the entry points and their options.

Each seed draws a plan (FLAT or PER_TENSOR, tensor sizes with ragged tails,
world size including runtime-N and two-pass sizes, a rank, hybrid replica
groups, a persistence threshold and hyperparameter groups for per-tensor
plans), hyperparameters (zero beta1, zero eps, zero decay and large step
counts included), and for each of two steps one way to run it (fused,
bucketed reduce + AdamW + gather, fused per bucket in shuffled order, the
device-scalar call; multi-tensor fused or unfused, by value or device
scalars) and which optional outputs to write. Inputs are host-generated from
numpy's seeded generator; every output must equal the oracle's bit for bit
(after the usual tolerance checks).
"""
import random

import numpy as np
import pytest

import oracle
from gpu_util import check_bf16, check_f32, dev16, dev32, host16, host32

pytestmark = pytest.mark.gpu

SENT = 0x5A5A


@pytest.fixture(scope="module")
def zs():
    import torch

    import fsdp_sharded_mixed_flatten_amd as m
    torch.cuda.init()
    return m


def _bf16(rng, n, sigma):
    x = (rng.standard_normal(n) * sigma).astype(np.float32)
    return oracle.f32_to_bf16(x)


def _random_hp(zs, rnd, t):
    return zs.AdamWHParams(lr=rnd.choice([1e-5, 3e-4, 1e-2]), beta1=rnd.choice([0.0, 0.9, 0.99]),
                           beta2=rnd.choice([0.95, 0.999]), eps=rnd.choice([0.0, 1e-8, 1e-6]),
                           weight_decay=rnd.choice([0.0, 0.1]), step=t)


def _ohp(hp):
    return oracle.HParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step)


def _coefs(zs, hps):
    import torch
    return torch.tensor([x for hp in hps for x in zs.zs_adamw_coefs_compute(hp).values()], dtype=torch.float32,
                        device="cuda")


@pytest.mark.parametrize("seed", range(24))
def test_random_flat(zs, seed):
    import torch
    rnd = random.Random(seed)
    rng = np.random.default_rng(seed)
    numels = [rnd.choice([1, 9, 255, 4093, 30_011, 70_000]) for _ in range(rnd.randint(1, 6))]
    world = rnd.choice([1, 2, 3, 4, 7, 8, 12, 16, 24, 48, 56, 64, 65])
    replicas = rnd.choice([1, 1, 2, 3]) if world * 3 <= 256 else 1
    rank = rnd.randrange(world)
    align = rnd.choice([1, 8, 128])
    plan = zs.zs_shard_plan(numels, world, rank, align)
    oplan = oracle.plan_flat(numels, world, rank, align)
    T, S = plan.padded_numel, plan.shard_numel
    assert (T, S) == (oplan.T, oplan.S)
    pad = np.frombuffer(bytes(oplan.padding_mask_full()), dtype=np.uint8).astype(bool)
    lo = rank * S
    master0 = (rng.standard_normal(T) * 0.02).astype(np.float32)
    master0[pad] = 0
    d = dict(master=dev32(master0[lo:lo + S]), m=torch.zeros(S, device="cuda"), v=torch.zeros(S, device="cuda"),
             g=dev16(np.full(S, SENT, np.uint16)), p=dev16(np.full(S, SENT, np.uint16)),
             full=dev16(np.full(T, SENT, np.uint16)))
    o = dict(g=np.full(S, SENT, np.uint16), master=master0[lo:lo + S].copy(), m=np.zeros(S, np.float32),
             v=np.zeros(S, np.float32), p=np.full(S, SENT, np.uint16), full=np.full(T, SENT, np.uint16))
    written = set()
    for t in (1, rnd.choice([2, 50, 10**5])):
        hp = _random_hp(zs, rnd, t)
        cs = []
        for _ in range(world * replicas):
            c = _bf16(rng, T, 1e-3)
            c[pad] = 0
            cs.append(c)
        mine = [c[lo:lo + S].copy() for c in cs]
        dc = [dev16(c) for c in mine]
        way = rnd.choice(["fused", "unfused", "buckets", "dc"])
        outs = {k: rnd.random() < 0.7 for k in ("g", "p", "full")}
        if way == "unfused":
            outs = dict(g=True, p=True, full=outs["full"])
        kw = dict(grad=d["g"] if outs["g"] else None, param=d["p"] if outs["p"] else None,
                  full=d["full"] if outs["full"] else None)
        if way == "fused":
            zs.zs_fused_shard_step(plan, hp, dc, d["master"], d["m"], d["v"], **kw)
        elif way == "dc":
            zs.zs_fused_shard_step_dc(plan, _coefs(zs, [hp]), dc, d["master"], d["m"], d["v"], **kw)
        elif way == "buckets":
            B = 8 * rnd.randint(1, max(1, S // 8))
            bk = [(b, min(B, S - b)) for b in range(0, S, B)]
            rnd.shuffle(bk)
            for off, n in bk:
                zs.zs_fused_shard_step_bucket(plan, hp, dc, d["master"], d["m"], d["v"], off, n, **kw)
        else:
            B = 8 * rnd.randint(1, max(1, S // 8))
            for b in range(0, S, B):
                zs.zs_reduce_shard(plan, dc, d["g"], b, min(B, S - b))
            zs.zs_adamw_shard_step(plan, hp, d["g"], d["master"], d["m"], d["v"], d["p"])
            if outs["full"]:
                zs.zs_gather_params(plan, d["p"], d["full"])
        # oracle
        g = np.zeros(S, np.uint16)
        oracle.reduce(mine, out=g)
        p = np.zeros(S, np.uint16)
        oracle.adamw(_ohp(hp), g, o["master"], o["m"], o["v"], p)
        if outs["g"]:
            o["g"] = g
            written.add("g")
        if outs["p"]:
            o["p"] = p
            written.add("p")
        if outs["full"]:
            o["full"][lo:lo + S] = p
    torch.cuda.synchronize()
    nd = check_f32(host32(d["master"]), o["master"], "master") + check_f32(host32(d["m"]), o["m"], "m")
    nd += check_f32(host32(d["v"]), o["v"], "v")
    nd += check_bf16(host16(d["g"]), o["g"], "grad") if "g" in written else 0
    nd += check_bf16(host16(d["p"]), o["p"], "param") if "p" in written else 0
    if "g" not in written:
        assert np.all(host16(d["g"]) == SENT)
    if "p" not in written:
        assert np.all(host16(d["p"]) == SENT)
    # NaN positions must agree, not their sign or payload (eps = 0 makes padding
    # 0/0 = NaN, whose sign x86 and CDNA choose differently)
    nd += check_bf16(host16(d["full"]), o["full"], "gathered buffer")
    assert nd == 0


@pytest.mark.parametrize("seed", range(16))
def test_random_per_tensor(zs, seed):
    import torch
    rnd = random.Random(100 + seed)
    rng = np.random.default_rng(100 + seed)
    numels = [rnd.choice([3, 64, 512, 4096, 12_345, 65_536]) for _ in range(rnd.randint(1, 10))]
    world = rnd.choice([1, 2, 4, 5, 8, 24, 56, 64])
    replicas = rnd.choice([1, 2]) if world <= 64 else 1
    rank = rnd.randrange(world)
    persist = rnd.choice([0, 0, 600, 5000])
    n_groups = rnd.choice([1, 2, 3])
    groups = [rnd.randrange(n_groups) for _ in numels]
    plan = zs.zs_shard_plan_ex(numels, world, rank, persist_below_elems=persist, groups=groups)
    oplan = oracle.plan_per_tensor(numels, world, rank, persist)
    N = world * replicas
    pieces, o = [], []
    for i, pc in enumerate(oplan.pieces):
        Si = pc.own_hi - pc.own_lo
        mst = (rng.standard_normal(Si) * 0.02).astype(np.float32)
        mst[max(0, min(Si, pc.real_hi - pc.own_lo)):] = 0  # padding of the piece
        pieces.append(dict(grad=dev16(np.full(Si, SENT, np.uint16)), master=dev32(mst),
                           m=torch.zeros(Si, device="cuda"), v=torch.zeros(Si, device="cuda"),
                           param=dev16(np.full(Si, SENT, np.uint16)),
                           full=dev16(np.full(oplan.padded[i], SENT, np.uint16))))
        o.append(dict(g=np.full(Si, SENT, np.uint16), master=mst.copy(), m=np.zeros(Si, np.float32),
                      v=np.zeros(Si, np.float32), p=np.full(Si, SENT, np.uint16),
                      full=np.full(oplan.padded[i], SENT, np.uint16)))
    for t in (1, rnd.choice([2, 7, 1000])):
        hps = [_random_hp(zs, rnd, t) for _ in range(n_groups)]
        host_c = []
        for q in range(N):
            row = []
            for i, pc in enumerate(oplan.pieces):
                Si = pc.own_hi - pc.own_lo
                c = _bf16(rng, Si, 1e-3)
                c[max(0, min(Si, pc.real_hi - pc.own_lo)):] = 0
                row.append(c)
            host_c.append(row)
        dev_c = [[dev16(c) for c in row] for row in host_c]
        ws = torch.zeros(zs.zs_multi_workspace_bytes(plan, N), dtype=torch.uint8, device="cuda")
        way = rnd.choice(["fused", "unfused", "dc"])
        zs.zs_multi_bind(plan, pieces, dev_c, ws)
        if way == "fused":
            zs.zs_fused_shard_step_multi_groups(plan, hps, ws)
        elif way == "dc":
            zs.zs_fused_shard_step_multi_dc(plan, _coefs(zs, hps), n_groups, ws)
        else:
            zs.zs_reduce_shard_multi(plan, ws)
            zs.zs_adamw_shard_step_multi_groups(plan, hps, ws)
            zs.zs_gather_params_multi(plan, ws)
        for i, pc in enumerate(oplan.pieces):
            oi = o[i]
            g = np.zeros(pc.own_hi - pc.own_lo, np.uint16)
            oracle.reduce([host_c[q][i] for q in range(N)], out=g)
            oi["g"] = g
            p = np.zeros_like(g)
            oracle.adamw(_ohp(hps[groups[pc.tensor]]), g, oi["master"], oi["m"], oi["v"], p)
            oi["p"] = p
            oi["full"][pc.own_lo:pc.own_hi] = p
        torch.cuda.synchronize()
        zs.zs_multi_unbind(ws)
    torch.cuda.synchronize()
    nd = 0
    for i, (oi, d) in enumerate(zip(o, pieces)):
        nd += check_f32(host32(d["master"]), oi["master"], f"master[{i}]")
        nd += check_f32(host32(d["m"]), oi["m"], f"m[{i}]") + check_f32(host32(d["v"]), oi["v"], f"v[{i}]")
        nd += check_bf16(host16(d["grad"]), oi["g"], f"grad[{i}]") + check_bf16(host16(d["param"]), oi["p"],
                                                                              f"param[{i}]")
        nd += check_bf16(host16(d["full"]), oi["full"], f"gathered tensor {i}")
    assert nd == 0


@pytest.mark.parametrize("seed", range(12))
def test_random_accum_clip(zs, seed):
    """G micro-steps (bucketed at random), norm, clip factor and skip, then the
    step from the accumulator by value or with device scalars; sometimes a
    NaN in one contribution (the step must be skipped)."""
    import torch
    rnd = random.Random(200 + seed)
    rng = np.random.default_rng(200 + seed)
    numels = [rnd.choice([9, 4093, 30_011, 70_000]) for _ in range(rnd.randint(1, 4))]
    world = rnd.choice([1, 2, 4, 5, 8, 13, 24, 48, 64])
    rank = rnd.randrange(world)
    plan = zs.zs_shard_plan(numels, world, rank, 1)
    oplan = oracle.plan_flat(numels, world, rank, 1)
    T, S = plan.padded_numel, plan.shard_numel
    lo = rank * S
    G = rnd.randint(1, 4)
    max_norm = rnd.choice([1e-4, 1e-2, 1e3])
    poison = rnd.random() < 0.25
    master0 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    micro = []
    for k in range(G):
        cs = [_bf16(rng, S, 1e-3) for _ in range(world)]
        if poison and k == G - 1:
            cs[0][rnd.randrange(S)] = 0x7FC0
        micro.append(cs)
    acc = torch.full((S,), float("nan"), device="cuda")
    for k in range(G):
        dc = [dev16(c) for c in micro[k]]
        B = 8 * rnd.randint(1, max(1, S // 8))
        for b in range(0, S, B):
            zs.zs_accumulate_shard(plan, dc, acc, b, min(B, S - b), first=(k == 0))
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    flag = torch.full((1,), 9, dtype=torch.int32, device="cuda")
    ws = torch.zeros(zs.zs_grad_stats_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    zs.zs_grad_stats(plan, acc, float(G), sumsq, flag, ws)
    scale = torch.zeros(1, device="cuda")
    skip = torch.full((1,), 9, dtype=torch.int32, device="cuda")
    zs.zs_clip_scale(sumsq, flag, max_norm, scale, skip)
    hp = _random_hp(zs, rnd, rnd.choice([1, 3, 100]))
    master, m, v = dev32(master0), torch.zeros(S, device="cuda"), torch.zeros(S, device="cuda")
    param = dev16(np.full(S, SENT, np.uint16))
    full = dev16(np.full(T, SENT, np.uint16))
    if rnd.random() < 0.5:
        zs.zs_adamw_shard_step_accum(plan, hp, acc, float(G), master, m, v, scale=scale, skip=skip, param=param,
                                     full=full)
    else:
        zs.zs_adamw_shard_step_accum_dc(plan, _coefs(zs, [hp]), acc, float(G), master, m, v, scale=scale, skip=skip,
                                        param=param, full=full)
    torch.cuda.synchronize()
    o_acc = np.zeros(S, np.float32)
    for k in range(G):
        oracle.accumulate(micro[k], o_acc, first=(k == 0))
    nd = check_f32(host32(acc), o_acc, "acc")
    o_sumsq, o_flag = oracle.grad_sumsq(o_acc, float(G))
    assert int(flag.cpu()[0]) == o_flag == (1 if poison else 0)
    got = float(sumsq.cpu()[0])
    if not poison:
        assert abs(got - o_sumsq) <= 1e-12 * o_sumsq
        assert float(scale.cpu()[0]) == oracle.clip_scale([got], max_norm)
    assert int(skip.cpu()[0]) == o_flag
    om, ov, op = np.zeros(S, np.float32), np.zeros(S, np.float32), np.full(S, SENT, np.uint16)
    omaster = master0.copy()
    oracle.adamw_f32grad(_ohp(hp), o_acc, float(G), float(scale.cpu()[0]), o_flag, omaster, om, ov, op)
    nd += check_f32(host32(master), omaster, "master") + check_f32(host32(m), om, "m") + check_f32(host32(v), ov, "v")
    nd += check_bf16(host16(param), op, "param")
    f_o = np.full(T, SENT, np.uint16)
    if not poison:
        f_o[lo:lo + S] = op
    nd += check_bf16(host16(full), f_o, "gathered buffer")
    assert nd == 0


@pytest.mark.parametrize("seed", range(12))
def test_random_quant(zs, seed):
    """The fused step writing codes (one- or two-pass, grad/param optional) on
    random shards with special blocks, then the dequantizing gather of every
    rank's payload."""
    import torch
    rnd = random.Random(300 + seed)
    rng = np.random.default_rng(300 + seed)
    numels = [rnd.choice([9, 4093, 30_011, 70_000]) for _ in range(rnd.randint(1, 4))]
    world = rnd.choice([1, 3, 4, 8, 24, 56, 64])
    rank = rnd.randrange(world)
    bits, block = rnd.choice([4, 8]), rnd.choice([8, 32, 128, 256])
    plan = zs.zs_shard_plan(numels, world, rank, 1)
    T, S = plan.padded_numel, plan.shard_numel
    master0 = (rng.standard_normal(S) * 0.02).astype(np.float32)
    if S >= 64:
        master0[:8] = 0.0  # an all-zero first block at B = 8
        master0[rnd.randrange(S)] = np.float32(np.inf) if rnd.random() < 0.3 else master0[0]
    cs = [_bf16(rng, S, 1e-3) for _ in range(world)]
    hp = _random_hp(zs, rnd, rnd.choice([1, 2, 9]))
    hp.eps = 1e-8  # keep padding finite
    nq, ns = zs.zs_quant_code_bytes(plan, bits), zs.zs_quant_num_scales(plan, block)
    codes = torch.zeros(nq, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(ns, dtype=torch.float32, device="cuda")
    master, m, v = dev32(master0), torch.zeros(S, device="cuda"), torch.zeros(S, device="cuda")
    grad = dev16(np.full(S, SENT, np.uint16)) if rnd.random() < 0.5 else None
    param = dev16(np.full(S, SENT, np.uint16)) if rnd.random() < 0.5 else None
    zs.zs_fused_shard_step_quant(plan, hp, [dev16(c) for c in cs], master, m, v, bits, block, codes, scales, grad=grad,
                                 param=param)
    g = np.zeros(S, np.uint16)
    oracle.reduce(cs, out=g)
    om, ov, op = np.zeros(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.uint16)
    omaster = master0.copy()
    oracle.adamw(_ohp(hp), g, omaster, om, ov, op)
    q, sc = oracle.quantize(op, bits, block)
    torch.cuda.synchronize()
    nd = check_f32(host32(master), omaster, "master") + check_f32(host32(m), om, "m") + check_f32(host32(v), ov, "v")
    if grad is not None:
        nd += check_bf16(host16(grad), g, "grad")
    if param is not None:
        nd += check_bf16(host16(param), op, "param")
    assert np.array_equal(codes.cpu().numpy(), q), "codes"
    got_sc = scales.cpu().numpy()
    assert np.array_equal(np.isnan(got_sc), np.isnan(sc))
    assert np.array_equal(got_sc[~np.isnan(sc)].view(np.uint32), sc[~np.isnan(sc)].view(np.uint32)), "scales"
    # every rank's payload (this rank's with its bytes rotated stands in for the others)
    payload_q = [np.roll(q, 3 * r) for r in range(world)]
    payload_s = [np.roll(sc, r) for r in range(world)]
    full = dev16(np.full(T + 64, SENT, np.uint16))
    zs.zs_dequant_gather(plan, bits, block, torch.from_numpy(np.concatenate(payload_q)).cuda(),
                         dev32(np.concatenate(payload_s)), full)
    ref = oracle.dequant_gather(np.concatenate(payload_q), np.concatenate(payload_s), S, world, bits, block)
    got = host16(full)
    nd += check_bf16(got[:T], ref, "gathered buffer")
    assert np.all(got[T:] == SENT)
    assert nd == 0
