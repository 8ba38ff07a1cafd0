"""Whole-step invariants of the oracle.

* Sharding invariance: each of the N ranks reduces its slice, runs AdamW on it
  and writes its bf16 slice into one gathered buffer; the result equals the
  unsharded update every replica runs under DDP (average over the full
  contributions, then AdamW on the full buffer) -- the same parameters and the
  same averaged gradient give the same new parameters ("从 Data Parallel 到
  ZeRO/FSDP" section "Data Parallel 保证的数学语义"; AllReduce = ReduceScatter +
  AllGather, section "DDP 为什么单卡仍是 16P").
* Resume: state saved after k steps and reloaded continues bit-identically.
* Resize: a state sharded for N=4 re-sliced for N=8 continues identically on
  every real element (padding holds +0 state and stays +0).
"""
import numpy as np

import synth
from oracle import HParams, plan_flat


def _inputs(numels, world, steps, seed=11):
    p = plan_flat(numels, world, 0, 1)
    real = sum(numels)
    master = synth.cpu_f32(p.T, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02, real))
    contribs = {t: [synth.cpu_bf16(p.T, 0, synth.spec(seed, synth.STREAM_CONTRIB + q, t, 1e-3, real))
                    for q in range(world)] for t in range(1, steps + 1)}
    return p, master, contribs


def test_sharding_invariance_tiny(ora):
    numels, N, steps = [1_000_003], 4, 3
    p, master0, contribs = _inputs(numels, N, steps)
    T, S = p.T, p.S
    hp = HParams(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)

    # DDP: every replica averages the full gradients and updates everything.
    ddp = dict(g=np.zeros(T, np.uint16), master=master0.copy(), m=np.zeros(T, np.float32),
               v=np.zeros(T, np.float32), p=np.zeros(T, np.uint16))
    # Sharded: rank r owns [rS, (r+1)S) of every array.
    sh = [dict(g=np.zeros(S, np.uint16), master=master0[r * S:(r + 1) * S].copy(),
               m=np.zeros(S, np.float32), v=np.zeros(S, np.float32), p=np.zeros(S, np.uint16))
          for r in range(N)]
    full = np.full(T, 0xDEAD, np.uint16)
    for t in range(1, steps + 1):
        h = hp.at(t)
        ora.reduce(contribs[t], out=ddp["g"])
        ora.adamw(h, ddp["g"], ddp["master"], ddp["m"], ddp["v"], ddp["p"])
        for r in range(N):
            mine = [c[r * S:(r + 1) * S].copy() for c in contribs[t]]
            st = sh[r]
            ora.shard_step(h, mine, st["g"], st["master"], st["m"], st["v"], st["p"], full, r)
        for key in ("g", "master", "m", "v", "p"):
            cat = np.concatenate([sh[r][key] for r in range(N)])
            assert np.array_equal(cat.view(np.uint8), ddp[key].view(np.uint8)), (t, key)
        assert np.array_equal(full, ddp["p"])
    # the 29 padding elements hold +0 everywhere
    pad = slice(1_000_003, T)
    for key in ("g", "master", "m", "v", "p"):
        assert not ddp[key][pad].view(np.uint8).any()


def test_hybrid_sharding_invariance(ora):
    """Hybrid sharding: shards cut 4 ways inside a group, 2 groups replicating
    them, 8 data-parallel contributions. The 4 shard ranks' steps, gathered,
    equal the DDP update over all 8 contributions and the full-shard update
    over 8 ranks ("ZeRO vs FSDP..." section 3.1, HYBRID_SHARD; the averaged
    gradient is the same whatever the sharding)."""
    numels, Ns, R, steps = [70_001, 333], 4, 2, 3
    N = Ns * R
    ph = plan_flat(numels, Ns, 0, 1)
    pf = plan_flat(numels, N, 0, 1)
    T = max(ph.T, pf.T)
    real = sum(numels)
    master0 = synth.cpu_f32(T, 0, synth.spec(41, synth.STREAM_MASTER, 0, 0.02, real))
    hp = HParams(lr=3e-4, weight_decay=0.05)

    def fresh(n, lo=0):
        return dict(g=np.zeros(n, np.uint16), master=master0[lo:lo + n].copy(), m=np.zeros(n, np.float32),
                    v=np.zeros(n, np.float32), p=np.zeros(n, np.uint16))

    ddp = fresh(T)
    hyb = [fresh(ph.S, r * ph.S) for r in range(Ns)]
    fs = [fresh(pf.S, r * pf.S) for r in range(N)]
    full_h = np.full(ph.T, 0xDEAD, np.uint16)
    full_f = np.full(pf.T, 0xDEAD, np.uint16)
    for t in range(1, steps + 1):
        cs = [synth.cpu_bf16(T, 0, synth.spec(41, synth.STREAM_CONTRIB + q, t, 1e-3, real)) for q in range(N)]
        h = hp.at(t)
        ora.reduce(cs, out=ddp["g"])
        ora.adamw(h, ddp["g"], ddp["master"], ddp["m"], ddp["v"], ddp["p"])
        for r, st in enumerate(hyb):
            mine = [c[r * ph.S:(r + 1) * ph.S].copy() for c in cs]
            ora.shard_step(h, mine, st["g"], st["master"], st["m"], st["v"], st["p"], full_h, r)
        for r, st in enumerate(fs):
            mine = [c[r * pf.S:(r + 1) * pf.S].copy() for c in cs]
            ora.shard_step(h, mine, st["g"], st["master"], st["m"], st["v"], st["p"], full_f, r)
        for key in ("g", "master", "m", "v", "p"):
            a = np.concatenate([st[key] for st in hyb])
            b = np.concatenate([st[key] for st in fs])
            assert a.tobytes() == ddp[key][:ph.T].tobytes(), (t, key)
            assert b.tobytes() == ddp[key][:pf.T].tobytes(), (t, key)
        assert np.array_equal(full_h, ddp["p"][:ph.T]) and np.array_equal(full_f, ddp["p"][:pf.T])


def test_gather_touches_only_own_slice(ora):
    S, N = 1000, 4
    p = np.arange(S, dtype=np.uint16)
    for r in range(N):
        full = np.full(N * S, 0xABCD, np.uint16)
        ora.gather(p, r, full)
        assert np.array_equal(full[r * S:(r + 1) * S], p)
        mask = np.ones(N * S, bool)
        mask[r * S:(r + 1) * S] = False
        assert np.all(full[mask] == 0xABCD)


def test_resume_equals_continuous(ora):
    numels, N, steps = [123_457], 4, 6
    p, master0, contribs = _inputs(numels, N, steps, seed=21)
    S = p.S
    hp = HParams()

    def run(state, t0, t1):
        for t in range(t0, t1 + 1):
            mine = [c[:S].copy() for c in contribs[t]]
            ora.shard_step(hp.at(t), mine, state["g"], state["master"], state["m"], state["v"],
                           state["p"], None, 0)

    a = dict(g=np.zeros(S, np.uint16), master=master0[:S].copy(), m=np.zeros(S, np.float32),
             v=np.zeros(S, np.float32), p=np.zeros(S, np.uint16))
    run(a, 1, steps)
    b = dict(g=np.zeros(S, np.uint16), master=master0[:S].copy(), m=np.zeros(S, np.float32),
             v=np.zeros(S, np.float32), p=np.zeros(S, np.uint16))
    run(b, 1, 3)
    saved = {k: v.tobytes() for k, v in b.items()}
    b2 = {k: np.frombuffer(saved[k], dtype=b[k].dtype).copy() for k in b}
    run(b2, 4, steps)
    for k in a:
        assert a[k].tobytes() == b2[k].tobytes()


def test_resize_world_4_to_8(ora):
    n = 100_037  # padded to 100,064 at N=4 (N*8 = 32) and to 100,096 at N=8
    steps = 4
    hp = HParams()
    seed = 31
    master0 = synth.cpu_f32(n, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02, n))

    def contrib(world, t, T):
        return [synth.cpu_bf16(T, 0, synth.spec(seed, synth.STREAM_CONTRIB + q, t, 1e-3, n))
                for q in range(world)]

    def shard_run(world, state_full, t0, t1, contribs_world):
        p = plan_flat([n], world, 0, 1)
        T, S = p.T, p.S
        st = {k: np.zeros(T, np.float32) for k in ("master", "m", "v")}
        for k in st:
            st[k][:n] = state_full[k][:n]
        out = np.zeros(T, np.uint16)
        for t in range(t0, t1 + 1):
            cs = contribs_world(t, T)
            for r in range(world):
                sl = slice(r * S, (r + 1) * S)
                mine = [c[sl].copy() for c in cs]
                g = np.zeros(S, np.uint16)
                sub = {k: st[k][sl].copy() for k in st}
                pp = np.zeros(S, np.uint16)
                ora.shard_step(hp.at(t), mine, g, sub["master"], sub["m"], sub["v"], pp, out, r)
                for k in st:
                    st[k][sl] = sub[k]
        return st, out

    # Resizing changes who owns which slice, not the averaged gradient: both
    # runs reduce the same 4 contributions, so only the re-slicing is tested.
    def c4(t, T):
        return contrib(4, t, T)

    zero = {"master": master0, "m": np.zeros(n, np.float32), "v": np.zeros(n, np.float32)}
    cont, out_c = shard_run(4, zero, 1, steps, c4)
    half, _ = shard_run(4, zero, 1, 2, c4)

    def run8(t, T):
        return c4(t, T)

    # re-slice the N=4 state to an N=8 plan
    st8, out8 = shard_run(8, half, 3, steps, run8)
    for k in ("master", "m", "v"):
        assert np.array_equal(st8[k][:n].view(np.uint32), cont[k][:n].view(np.uint32)), k
        assert not st8[k][n:].view(np.uint32).any()
    assert np.array_equal(out8[:n], out_c[:n])
