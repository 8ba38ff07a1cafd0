"""CPU-offloaded optimizer step against the oracle: the device grad shard is
copied to pinned host memory chunk by chunk, stepped on the host, and the
bf16 parameters copied back to the device shard and the gathered buffer.
Every byte must equal the oracle's step (same fp32 arithmetic)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_bf16, check_f32, dev16, host16

pytestmark = pytest.mark.gpu

SENT = 0x5A5A


@pytest.fixture(scope="module")
def zs():
    import torch

    import fsdp_sharded_mixed_flatten_amd as m
    torch.cuda.init()
    return m


def _pinned(n, dtype):
    import torch
    return torch.zeros(n, dtype=dtype, pin_memory=True)


@pytest.mark.parametrize("chunk,threads", [(4096, 4), (1 << 20, 1), (1024, 16)])
def test_offload_step_equals_oracle(zs, chunk, threads):
    import torch
    world, rank = 4, 2
    numels = [300_007, 4_099]
    plan = zs.zs_shard_plan(numels, world, rank, 1)
    S, T = plan.shard_numel, plan.padded_numel
    real = sum(numels)
    lo = rank * S
    master0 = synth.cpu_f32(T, 0, synth.spec(71, synth.STREAM_MASTER, 0, 0.02, real))[lo:lo + S].copy()
    hm, hmm, hv = _pinned(S, torch.float32), _pinned(S, torch.float32), _pinned(S, torch.float32)
    hm.copy_(torch.from_numpy(master0))
    gh, ph = _pinned(S, torch.int16), _pinned(S, torch.int16)
    o = dict(g=np.zeros(S, np.uint16), master=master0.copy(), m=np.zeros(S, np.float32), v=np.zeros(S, np.float32),
             p=np.zeros(S, np.uint16), full=np.full(T, SENT, np.uint16))
    pd = torch.zeros(S, dtype=torch.int16, device="cuda")
    full = dev16(np.full(T, SENT, np.uint16))
    gd = torch.zeros(S, dtype=torch.int16, device="cuda")
    for t in (1, 2, 3):
        cs = [synth.cpu_bf16(T, 0, synth.spec(71, synth.STREAM_CONTRIB + q, t, 1e-3, real))[lo:lo + S].copy()
              for q in range(world)]
        zs.zs_reduce_shard(plan, [dev16(c) for c in cs], gd)  # the grad shard on the device
        hp = zs.AdamWHParams(lr=2e-4, weight_decay=0.1, step=t)
        zs.zs_offload_adamw_step(plan, hp, gd, hm, hmm, hv, gh, ph, param_dev=pd, full_dev=full, chunk_elems=chunk,
                                 n_threads=threads)
        oracle.shard_step(oracle.HParams(lr=2e-4, weight_decay=0.1, step=t), cs, o["g"], o["master"], o["m"], o["v"],
                          o["p"], o["full"], rank)
        torch.cuda.synchronize()
        nd = check_bf16(gh.numpy().view(np.uint16), o["g"], "grad on host")
        nd += check_f32(hm.numpy(), o["master"], "master") + check_f32(hmm.numpy(), o["m"], "m")
        nd += check_f32(hv.numpy(), o["v"], "v")
        nd += check_bf16(ph.numpy().view(np.uint16), o["p"], "param on host")
        nd += check_bf16(host16(pd), o["p"], "param on device")
        assert nd == 0
        assert np.array_equal(host16(full), o["full"]), "gathered buffer"


def test_offload_steps_on_alternating_streams(zs):
    """Consecutive steps on different streams, with no synchronization between
    them: each step's host arithmetic overwrites the staging buffers the
    previous step's copy-outs read, so a step must wait for those copies even
    when its stream never saw them."""
    import torch
    world, rank, chunk = 2, 1, 2048
    numels = [262_147]
    plan = zs.zs_shard_plan(numels, world, rank, 1)
    S, T = plan.shard_numel, plan.padded_numel
    lo = rank * S
    master0 = synth.cpu_f32(T, 0, synth.spec(72, synth.STREAM_MASTER, 0, 0.02, numels[0]))[lo:lo + S].copy()
    hm, hmm, hv = _pinned(S, torch.float32), _pinned(S, torch.float32), _pinned(S, torch.float32)
    hm.copy_(torch.from_numpy(master0))
    gh, ph = _pinned(S, torch.int16), _pinned(S, torch.int16)
    o = dict(g=np.zeros(S, np.uint16), master=master0.copy(), m=np.zeros(S, np.float32), v=np.zeros(S, np.float32),
             p=np.zeros(S, np.uint16), full=np.full(T, SENT, np.uint16))
    full = dev16(np.full(T, SENT, np.uint16))
    streams = [torch.cuda.Stream() for _ in range(3)]
    steps = 4
    cs = {t: [synth.cpu_bf16(T, 0, synth.spec(72, synth.STREAM_CONTRIB + q, t, 1e-3, numels[0]))[lo:lo + S].copy()
              for q in range(world)] for t in range(1, steps + 1)}
    dcs = {t: [dev16(c) for c in cs[t]] for t in cs}
    gds = [torch.zeros(S, dtype=torch.int16, device="cuda") for _ in range(steps)]
    pds = [torch.zeros(S, dtype=torch.int16, device="cuda") for _ in range(steps)]
    want_p = []
    torch.cuda.synchronize()
    for t in range(1, steps + 1):
        s = streams[t % len(streams)]
        hp = zs.AdamWHParams(lr=2e-4, weight_decay=0.1, step=t)
        zs.zs_reduce_shard(plan, dcs[t], gds[t - 1], stream=s)
        zs.zs_offload_adamw_step(plan, hp, gds[t - 1], hm, hmm, hv, gh, ph, param_dev=pds[t - 1], full_dev=full,
                                 chunk_elems=chunk, n_threads=4, stream=s)
        oracle.shard_step(oracle.HParams(lr=2e-4, weight_decay=0.1, step=t), cs[t], o["g"], o["master"], o["m"],
                          o["v"], o["p"], o["full"], rank)
        want_p.append(o["p"].copy())  # each step copies its parameters into a device buffer of its own
    torch.cuda.synchronize()
    for t in range(1, steps + 1):
        assert check_bf16(host16(pds[t - 1]), want_p[t - 1], f"param on device, step {t}") == 0
    nd = check_f32(hm.numpy(), o["master"], "master") + check_f32(hmm.numpy(), o["m"], "m")
    nd += check_f32(hv.numpy(), o["v"], "v")
    assert nd == 0
    assert np.array_equal(host16(full), o["full"]), "gathered buffer"


def test_offload_rejects_pageable_staging(zs):
    import torch
    plan = zs.zs_shard_plan([8192], 2, 0)
    S = plan.shard_numel
    gd = torch.zeros(S, dtype=torch.int16, device="cuda")
    st = [torch.zeros(S) for _ in range(3)]
    with pytest.raises(zs.ZsError) as e:
        zs.zs_offload_adamw_step(plan, zs.AdamWHParams(), gd, *st, torch.zeros(S, dtype=torch.int16),
                                 torch.zeros(S, dtype=torch.int16), chunk_elems=1024)
    assert "page-locked" in e.value.message
    with pytest.raises(zs.ZsError):
        zs.zs_offload_adamw_step(plan, zs.AdamWHParams(), gd, *st, _pinned(S, torch.int16), _pinned(S, torch.int16),
                                 chunk_elems=1000)
    torch.cuda.synchronize()
