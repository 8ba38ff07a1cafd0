"""GPU <-> oracle parity of gradient accumulation, global-norm clipping and
the non-finite skip (the C ABI's zs_accumulate_shard, zs_grad_stats,
zs_clip_scale, zs_adamw_shard_step_accum).

fp32 accumulators and optimizer state must be bit-identical to the oracle
(the tolerance bar of relative 1e-6 is asserted, then zero non-identical
elements); the squared norm is a double sum in another order, so it must
agree to relative 1e-12; the clip factor computed from the same partials must
be identical.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_bf16, check_f32, dev16, dev32, host16, host32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zs():
    import torch

    import fsdp_sharded_mixed_flatten_amd as m
    torch.cuda.init()
    return m


def _contribs(T, N, micro, seed, valid, nan_at=None):
    out = []
    for q in range(N):
        c = synth.cpu_bf16(T, 0, synth.spec(seed, synth.STREAM_CONTRIB + q, micro, 1e-3, valid))
        if nan_at is not None and q == 1:
            c[nan_at] = 0x7FC0
        out.append(c)
    return out


@pytest.mark.parametrize("G,max_norm,N", [(1, 1e-4, 4), (3, 1e-4, 4), (3, 100.0, 4), (4, 3e-5, 4),
                                          (3, 1e-4, 13), (2, 3e-5, 24)])
def test_accumulate_clip_step_all_ranks(zs, G, max_norm, N):
    """N = 13 and 24 take the runtime rank loop (a group of 8 plus 4 + 1, and
    three groups of 8 in the two register sets in turn)."""
    import torch
    numels = [1_000_003]
    plans = [zs.zs_shard_plan(numels, N, r, 1) for r in range(N)]
    T, S = plans[0].padded_numel, plans[0].shard_numel
    seed = 4242 + G
    micro = [_contribs(T, N, k + 1, seed, 1_000_003) for k in range(G)]
    master0 = synth.cpu_f32(T, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02, 1_000_003))
    hp = zs.AdamWHParams(lr=1e-3, weight_decay=0.1, step=1)
    # device: every rank accumulates its shard (bucketed), then its squared norm
    accs = [torch.full((S,), float("nan"), device="cuda") for _ in range(N)]
    sumsq = torch.zeros(N, dtype=torch.float64, device="cuda")
    flags = torch.full((N,), 7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(zs.zs_grad_stats_workspace_bytes(plans[0]), dtype=torch.uint8, device="cuda")
    for r in range(N):
        for k in range(G):
            mine = [dev16(c[r * S:(r + 1) * S]) for c in micro[k]]
            for off in range(0, S, 65_536):
                zs.zs_accumulate_shard(plans[r], mine, accs[r], off, min(65_536, S - off), first=(k == 0))
        zs.zs_grad_stats(plans[r], accs[r], float(G), sumsq[r:r + 1], flags[r:r + 1], ws)
    scale = torch.zeros(1, device="cuda")
    skip = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    zs.zs_clip_scale(sumsq, flags, max_norm, scale, skip)
    r = 1
    master = dev32(master0[r * S:(r + 1) * S])
    m = torch.zeros(S, device="cuda")
    v = torch.zeros(S, device="cuda")
    full = dev16(np.full(T, 0x5A5A, np.uint16))
    param = torch.zeros(S, dtype=torch.int16, device="cuda")
    zs.zs_adamw_shard_step_accum(plans[r], hp, accs[r], float(G), master, m, v, scale=scale, skip=skip,
                                 param=param, full=full)
    torch.cuda.synchronize()
    # oracle
    o_acc = [np.zeros(S, np.float32) for _ in range(N)]
    o_sumsq, o_flags = [], []
    for q in range(N):
        for k in range(G):
            oracle.accumulate([c[q * S:(q + 1) * S].copy() for c in micro[k]], o_acc[q], first=(k == 0))
        s, f = oracle.grad_sumsq(o_acc[q], float(G))
        o_sumsq.append(s)
        o_flags.append(f)
    o_scale = oracle.clip_scale(o_sumsq, max_norm)
    nd = 0
    for q in range(N):
        nd += check_f32(host32(accs[q]), o_acc[q], f"acc[{q}]")
    got_sumsq = sumsq.cpu().numpy()
    assert np.all(np.abs(got_sumsq - np.array(o_sumsq)) <= 1e-12 * np.array(o_sumsq))
    assert flags.cpu().numpy().tolist() == o_flags == [0] * N
    # the factor from the device's own partials equals the oracle's from those partials
    assert float(scale.cpu()[0]) == oracle.clip_scale(got_sumsq.tolist(), max_norm)
    assert abs(float(scale.cpu()[0]) - o_scale) <= 2.0**-23 * o_scale
    assert int(skip.cpu()[0]) == 0
    # the step itself, with the factor the device computed
    om, ov, op = np.zeros(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.uint16)
    omaster = master0[r * S:(r + 1) * S].copy()
    oracle.adamw_f32grad(oracle.HParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1), o_acc[r], float(G), float(scale.cpu()[0]),
                         False, omaster, om, ov, op)
    nd += check_f32(host32(master), omaster, "master") + check_f32(host32(m), om, "m")
    nd += check_f32(host32(v), ov, "v") + check_bf16(host16(param), op, "param")
    full_o = np.full(T, 0x5A5A, np.uint16)
    full_o[r * S:(r + 1) * S] = op
    assert np.array_equal(host16(full), full_o)
    assert nd == 0
    if max_norm >= 100.0:
        assert o_scale == 1.0


def test_non_finite_skips_step(zs):
    import torch
    numels, N, S = [8192 * 4], 4, 8192
    plan = zs.zs_shard_plan(numels, N, 0, 1)
    cs = _contribs(S, N, 1, 5, S, nan_at=1234)
    acc = torch.zeros(S, device="cuda")
    zs.zs_accumulate_shard(plan, [dev16(c) for c in cs], acc, first=True)
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(zs.zs_grad_stats_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    zs.zs_grad_stats(plan, acc, 1.0, sumsq, flag, ws)
    scale = torch.zeros(1, device="cuda")
    skip = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zs_clip_scale(sumsq, flag, 1.0, scale, skip)
    rng = np.random.default_rng(0)
    st0 = [(rng.standard_normal(S) * 0.02).astype(np.float32) for _ in range(3)]
    st = [dev32(a) for a in st0]
    param = dev16(np.full(S, 0x1234, np.uint16))
    zs.zs_adamw_shard_step_accum(plan, zs.AdamWHParams(), acc, 1.0, *st, scale=scale, skip=skip, param=param)
    torch.cuda.synchronize()
    assert int(flag.cpu()[0]) == 1 and int(skip.cpu()[0]) == 1
    for a, b in zip(st, st0):
        assert host32(a).tobytes() == b.tobytes()
    assert np.all(host16(param) == 0x1234)
    # the oracle agrees on the flag
    o = np.zeros(S, np.float32)
    oracle.accumulate(cs, o, first=True)
    assert oracle.grad_sumsq(o)[1] == 1


@pytest.mark.parametrize("divisor", [2.0, 3.0])
@pytest.mark.parametrize("outs", range(4), ids=lambda o: f"param{o & 1}-full{o >> 1}")
def test_accum_step_without_clipping(zs, divisor, outs):
    """The step from the accumulator with no clip factor and no skip flag
    (NULL: factor 1, never skipped), a divisor other than the number of
    micro-steps, and each subset of the optional outputs; disabled outputs
    keep their sentinels."""
    import torch
    numels, N, r, G = [200_003], 4, 3, 2
    plan = zs.zs_shard_plan(numels, N, r, 1)
    T, S = plan.padded_numel, plan.shard_numel
    micro = [_contribs(T, N, k + 1, 77, numels[0]) for k in range(G)]
    master0 = synth.cpu_f32(T, 0, synth.spec(77, synth.STREAM_MASTER, 0, 0.02, numels[0]))[r * S:(r + 1) * S].copy()
    acc = torch.zeros(S, device="cuda")
    for k in range(G):
        zs.zs_accumulate_shard(plan, [dev16(c[r * S:(r + 1) * S]) for c in micro[k]], acc, first=(k == 0))
    master, m, v = dev32(master0), torch.zeros(S, device="cuda"), torch.zeros(S, device="cuda")
    param = dev16(np.full(S + 64, 0x5A5A, np.uint16))
    full = dev16(np.full(T + 64, 0x5A5A, np.uint16))
    hp = zs.AdamWHParams(lr=1e-3, weight_decay=0.1, step=1)
    zs.zs_adamw_shard_step_accum(plan, hp, acc, divisor, master, m, v, param=param if outs & 1 else None,
                                 full=full if outs & 2 else None)
    torch.cuda.synchronize()
    o_acc = np.zeros(S, np.float32)
    for k in range(G):
        oracle.accumulate([c[r * S:(r + 1) * S].copy() for c in micro[k]], o_acc, first=(k == 0))
    om, ov, op = np.zeros(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.uint16)
    omaster = master0.copy()
    oracle.adamw_f32grad(oracle.HParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1), o_acc, divisor, 1.0, False, omaster, om, ov,
                         op)
    nd = check_f32(host32(master), omaster, "master") + check_f32(host32(m), om, "m") + check_f32(host32(v), ov, "v")
    p, f = host16(param), host16(full)
    if outs & 1:
        nd += check_bf16(p[:S], op, "param")
        assert np.all(p[S:] == 0x5A5A)
    else:
        assert np.all(p == 0x5A5A)
    f_o = np.full(T + 64, 0x5A5A, np.uint16)
    if outs & 2:
        f_o[r * S:(r + 1) * S] = op
    assert np.array_equal(f, f_o), "gathered buffer"
    assert nd == 0


def test_stats_deterministic(zs):
    import torch
    plan = zs.zs_shard_plan([3_000_000 * 8], 8, 0, 1)
    S = plan.shard_numel
    acc = torch.randn(S, device="cuda") * 1e-3
    ws = torch.zeros(zs.zs_grad_stats_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        s = torch.zeros(1, dtype=torch.float64, device="cuda")
        f = torch.zeros(1, dtype=torch.int32, device="cuda")
        zs.zs_grad_stats(plan, acc, 2.0, s, f, ws)
        outs.append(s.cpu().numpy().tobytes())
    assert outs[0] == outs[1] == outs[2]
    ref = float(((acc.double() / 2.0) ** 2).sum())  # different order: close, not identical
    assert abs(np.frombuffer(outs[0], np.float64)[0] - ref) <= 1e-12 * ref


def test_llama7b_shape_two_micro_steps_sampled(zs):
    """Full 842M-element shard: 2 micro-steps of 34 buckets, stats, clip, AdamW;
    sampled elements against the oracle, the norm against a float64 sum."""
    import torch
    free, _ = torch.cuda.mem_get_info()
    if free < 40 * 2**30:
        pytest.skip("needs ~30 GiB of free device memory")
    wl = synth.workloads()["llama7b"]
    plan = zs.zs_shard_plan(wl.numels, wl.world, wl.rank, wl.align)
    S, N, B, G = plan.shard_numel, wl.world, wl.bucket_elems, 2
    valid = sum(wl.numels)
    cs = [torch.empty(S, dtype=torch.int16, device="cuda") for _ in range(N)]
    acc = torch.empty(S, device="cuda")
    for k in range(G):
        for q, c in enumerate(cs):
            synth.gpu_bf16(c, 0, wl.contrib_spec(q, k + 1, valid))
        for off in range(0, S, B):
            zs.zs_accumulate_shard(plan, cs, acc, off, min(B, S - off), first=(k == 0))
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(zs.zs_grad_stats_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    zs.zs_grad_stats(plan, acc, float(G), sumsq, flag, ws)
    ref = float(((acc.double() / G) ** 2).sum())
    got = float(sumsq.cpu()[0])
    assert abs(got - ref) <= 1e-10 * ref and int(flag.cpu()[0]) == 0
    # a world of identical shards stands in for the other ranks' partials
    all_sumsq = sumsq.repeat(N)
    all_flags = flag.repeat(N)
    scale = torch.zeros(1, device="cuda")
    skip = torch.zeros(1, dtype=torch.int32, device="cuda")
    max_norm = 0.5 * (got * N) ** 0.5  # forces clipping
    zs.zs_clip_scale(all_sumsq, all_flags, max_norm, scale, skip)
    master = torch.empty(S, device="cuda")
    synth.gpu_f32(master, 0, wl.master_spec(valid))
    m = torch.zeros(S, device="cuda")
    v = torch.zeros(S, device="cuda")
    hp = zs.AdamWHParams(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, 1)
    zs.zs_adamw_shard_step_accum(plan, hp, acc, float(G), master, m, v, scale=scale, skip=skip)
    torch.cuda.synchronize()
    sc = float(scale.cpu()[0])
    assert sc == oracle.clip_scale([got] * N, max_norm) and 0.4 < sc < 0.6
    rng = np.random.default_rng(3)
    idx = np.unique(np.concatenate([np.arange(4096), np.arange(S - 4096, S), rng.integers(0, S, 100_000),
                                    *[np.arange(b - 8, b + 8) for b in range(B, S, B)]])).astype(np.int64)
    o_acc = np.zeros(idx.size, np.float32)
    for k in range(G):
        oracle.accumulate([synth.cpu_at_bf16(idx, wl.contrib_spec(q, k + 1, valid)) for q in range(N)], o_acc,
                          first=(k == 0))
    omaster = synth.cpu_at_f32(idx, wl.master_spec(valid))
    om, ov, op = np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32), np.zeros(idx.size, np.uint16)
    oracle.adamw_f32grad(oracle.HParams(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, 1), o_acc, float(G), sc,
                         False, omaster, om, ov, op)
    d = torch.from_numpy(idx).cuda()
    nd = check_f32(acc.index_select(0, d).cpu().numpy(), o_acc, "acc")
    nd += check_f32(master.index_select(0, d).cpu().numpy(), omaster, "master")
    nd += check_f32(m.index_select(0, d).cpu().numpy(), om, "m")
    nd += check_f32(v.index_select(0, d).cpu().numpy(), ov, "v")
    assert nd == 0
