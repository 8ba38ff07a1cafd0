"""Checkpoint/resume and resize invariance of the shard step on the GPU.

A sharded checkpoint holds each rank's fp32 master/m/v shard, never a whole
model ("从 Data Parallel 到 ZeRO/FSDP", section "Checkpoint 不能假设每个 Rank
都有完整模型"); a job resumed from it, possibly at another world size
("一条可执行的落地路径", step 10: resume and resize must reproduce the
uninterrupted run), must continue exactly as if it had never stopped:

* resume: the device state is written to host memory after step k, every
  device buffer is freed, new ones are allocated from the host copies, and
  steps k+1.. continue; the result equals the uninterrupted run bit for bit,
  and both equal the oracle.
* resize: four ranks' shards run steps 1..k at N=4 (four gradient
  contributions per step), the four shards are joined on the host and re-cut
  for an N=8 plan (its own padding), and eight ranks continue with eight
  contributions per step. The shards joined at the end equal an unsharded
  run (one rank holding the whole flat buffer, N=1, averaging the same 4 and
  then 8 contributions) bit for bit, and the oracle.

Inputs come from the seeded generator on the host (padding +0) and are
copied to the device; the steps run through the C ABI.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_bf16, check_f32, dev16, dev32, host16, host32

pytestmark = pytest.mark.gpu

SENT = 0x5A5A


@pytest.fixture(scope="module")
def zs():
    import torch

    import fsdp_sharded_mixed_flatten_amd as m
    torch.cuda.init()
    return m


def _contribs(seed, n_valid, T, count, t):
    """count bf16 contributions of T elements for step t (padding +0)."""
    return [synth.cpu_bf16(T, 0, synth.spec(seed, synth.STREAM_CONTRIB + q, t, 1e-3, n_valid))
            for q in range(count)]


def test_resume_after_host_round_trip_equals_continuous(zs):
    import torch
    numels, N, rank, steps, k = [123_457, 4093, 77], 4, 2, 6, 3
    seed = 4242
    plan = zs.zs_shard_plan(numels, N, rank, 8, zs.ZS_LAYOUT_FLAT)
    oplan = oracle.plan_flat(numels, N, rank, 8)
    T, S = plan.padded_numel, plan.shard_numel
    assert (T, S) == (oplan.T, oplan.S)
    lo = rank * S
    pad = np.frombuffer(bytes(oplan.padding_mask_full()), dtype=np.uint8).astype(bool)
    master0 = synth.cpu_f32(T, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02))
    master0[pad] = 0
    cs = {}
    for t in range(1, steps + 1):
        cs[t] = _contribs(seed, 2**62, T, N, t)
        for c in cs[t]:
            c[pad] = 0
    hp = zs.AdamWHParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1)

    def fresh():
        return dict(master=dev32(master0[lo:lo + S]), m=torch.zeros(S, device="cuda"),
                    v=torch.zeros(S, device="cuda"), full=dev16(np.full(T, SENT, np.uint16)))

    def run(st, t0, t1):
        for t in range(t0, t1 + 1):
            mine = [dev16(c[lo:lo + S]) for c in cs[t]]
            zs.zs_fused_shard_step(plan, hp.at(t), mine, st["master"], st["m"], st["v"], full=st["full"])
        torch.cuda.synchronize()

    a = fresh()
    run(a, 1, steps)
    b = fresh()
    run(b, 1, k)
    # checkpoint: this rank's fp32 state and its gathered slice to host memory
    saved = {key: (host32(b[key]).copy() if key != "full" else host16(b[key]).copy()) for key in b}
    del b
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    b = dict(master=dev32(saved["master"]), m=dev32(saved["m"]), v=dev32(saved["v"]), full=dev16(saved["full"]))
    run(b, k + 1, steps)
    for key in ("master", "m", "v"):
        assert np.array_equal(host32(a[key]).view(np.uint32), host32(b[key]).view(np.uint32)), key
    assert np.array_equal(host16(a["full"]), host16(b["full"]))
    # and both equal the oracle's uninterrupted run
    o = dict(master=master0[lo:lo + S].copy(), m=np.zeros(S, np.float32), v=np.zeros(S, np.float32),
             g=np.zeros(S, np.uint16), p=np.zeros(S, np.uint16))
    o_full = np.full(T, SENT, np.uint16)
    for t in range(1, steps + 1):
        oracle.shard_step(oracle.HParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t),
                          [c[lo:lo + S].copy() for c in cs[t]], o["g"], o["master"], o["m"], o["v"], o["p"],
                          o_full, rank)
    nd = check_f32(host32(b["master"]), o["master"], "master")
    nd += check_f32(host32(b["m"]), o["m"], "m")
    nd += check_f32(host32(b["v"]), o["v"], "v")
    nd += check_bf16(host16(b["full"]), o_full, "gathered buffer")
    assert nd == 0, f"{nd} elements not bit-identical to the oracle"
    mask = np.ones(T, bool)
    mask[lo:lo + S] = False
    assert np.all(host16(b["full"])[mask] == SENT)


def test_resize_world_4_to_8_equals_unsharded(zs):
    import torch
    n = 100_037  # padded to 100,064 at N=4 (8*N = 32), to 100,096 at N=8, to 100,040 at N=1
    steps, k = 5, 2  # 4 contributions per step up to step k, 8 after it
    seed = 3131
    hp = zs.AdamWHParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1)
    master0 = synth.cpu_f32(n, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02, n))
    T1 = zs.zs_shard_plan([n], 1, 0, 1).padded_numel
    Tmax = 100_096
    cs = {t: _contribs(seed, n, Tmax, 4 if t <= k else 8, t) for t in range(1, steps + 1)}

    def sharded(world, state, t0, t1):
        """world ranks' shards (each its own device buffers) from the joined
        state `state` (n real elements); returns the joined state after step t1
        and the gathered buffer."""
        plans = [zs.zs_shard_plan([n], world, r, 1) for r in range(world)]
        T, S = plans[0].padded_numel, plans[0].shard_numel
        dev = []
        for r in range(world):
            sl = slice(r * S, (r + 1) * S)
            st = {}
            for key in ("master", "m", "v"):
                a = np.zeros(T, np.float32)
                a[:n] = state[key][:n]
                st[key] = dev32(a[sl])
            dev.append(st)
        full = dev16(np.full(T, SENT, np.uint16))
        for t in range(t0, t1 + 1):
            for r in range(world):
                mine = [dev16(c[r * S:(r + 1) * S]) for c in cs[t]]
                zs.zs_fused_shard_step(plans[r], hp.at(t), mine, dev[r]["master"], dev[r]["m"], dev[r]["v"],
                                       full=full)
        torch.cuda.synchronize()
        joined = {key: np.concatenate([host32(d[key]) for d in dev]) for key in ("master", "m", "v")}
        return joined, host16(full), T

    zero = {"master": master0, "m": np.zeros(n, np.float32), "v": np.zeros(n, np.float32)}
    # N=4 for steps 1..k, re-cut to N=8, steps k+1..steps
    half, _, T4 = sharded(4, zero, 1, k)
    assert T4 == 100_064
    for key in ("master", "m", "v"):
        assert not half[key][n:].view(np.uint32).any(), f"padding of {key} left +0"
    st8, full8, T8 = sharded(8, half, k + 1, steps)
    assert T8 == Tmax
    # unsharded: one rank holds the whole buffer (N=1), averaging the same contributions
    one, full1, _ = sharded(1, zero, 1, steps)
    for key in ("master", "m", "v"):
        assert np.array_equal(st8[key][:n].view(np.uint32), one[key][:n].view(np.uint32)), key
        assert not st8[key][n:].view(np.uint32).any(), key
    assert np.array_equal(full8[:n], full1[:n])
    # and the oracle over the whole buffer
    o = dict(master=master0.copy(), m=np.zeros(n, np.float32), v=np.zeros(n, np.float32),
             g=np.zeros(n, np.uint16), p=np.zeros(n, np.uint16))
    for t in range(1, steps + 1):
        oracle.shard_step(oracle.HParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t),
                          [c[:n].copy() for c in cs[t]], o["g"], o["master"], o["m"], o["v"], o["p"], None, 0)
    nd = check_f32(st8["master"][:n], o["master"], "master")
    nd += check_f32(st8["m"][:n], o["m"], "m")
    nd += check_f32(st8["v"][:n], o["v"], "v")
    nd += check_bf16(full8[:n], o["p"], "gathered params")
    assert nd == 0, f"{nd} elements not bit-identical to the oracle"
    assert T1 == 100_040
