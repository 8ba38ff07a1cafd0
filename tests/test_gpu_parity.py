"""GPU <-> oracle parity at sizes the oracle covers element by element.

Every case builds its inputs on the host from the seeded generator (padding
positions +0), copies them to the device, runs the HIP path through the C
ABI and compares every output element with the CPU oracle: fp32 master/m/v
within relative 1e-6 (exact where the oracle is 0), bf16 grad/param/gathered
values within 1 ulp, untouched memory bit-identical. The path mirrors the
oracle's operation order, so the tests also count elements that are not
bit-identical and require that count to be zero.
"""
import random

import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_bf16, check_f32, dev16, dev32, host16, host32

pytestmark = pytest.mark.gpu

SENT = 0x5A5A  # sentinel for memory the step must not touch


@pytest.fixture(scope="module")
def zs():
    import torch

    import fsdp_sharded_mixed_flatten_amd as m
    torch.cuda.init()
    return m


def _flat_inputs(numels, world, align, steps, seed, zero_prob=0.0, tail_prob=0.0, replicas=1):
    plan = oracle.plan_flat(numels, world, 0, align)
    T = plan.T
    pad = np.frombuffer(bytes(plan.padding_mask_full()), dtype=np.uint8).astype(bool)
    master = synth.cpu_f32(T, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02))
    master[pad] = 0
    contribs = {}
    for t in range(1, steps + 1):
        cs = []
        for q in range(world * replicas):
            c = synth.cpu_bf16(T, 0, synth.spec(seed, synth.STREAM_CONTRIB + q, t, 1e-3, 2**62, 0.1,
                                                tail_prob, zero_prob))
            c[pad] = 0
            cs.append(c)
        contribs[t] = cs
    return T, master, contribs


class FlatRun:
    """Oracle and GPU state of one rank over several steps of a FLAT plan."""

    def __init__(self, zs, numels, world, rank, align, steps, seed, hp, bucket=0, fused=False,
                 zero_prob=0.0, tail_prob=0.0, replicas=1):
        import torch
        self.zs = zs
        self.plan = zs.zs_shard_plan(numels, world, rank, align, zs.ZS_LAYOUT_FLAT)
        T, S = self.plan.padded_numel, self.plan.shard_numel
        self.T, self.S, self.rank, self.world = T, S, rank, world
        T2, master, contribs = _flat_inputs(numels, world, align, steps, seed, zero_prob, tail_prob, replicas)
        assert T2 == T
        lo = rank * S
        self.mine = {t: [c[lo:lo + S].copy() for c in cs] for t, cs in contribs.items()}
        self.hp = hp
        self.bucket = bucket
        self.fused = fused
        # oracle state
        self.o = dict(g=np.zeros(S, np.uint16), master=master[lo:lo + S].copy(),
                      m=np.zeros(S, np.float32), v=np.zeros(S, np.float32), p=np.zeros(S, np.uint16),
                      full=np.full(T, SENT, np.uint16))
        # device state, with a guard band after each buffer
        G = 64
        self.G = G

        def guarded32(a):
            return dev32(np.concatenate([a, np.full(G, 7.0, np.float32)]))

        def guarded16(a):
            return dev16(np.concatenate([a, np.full(G, SENT, np.uint16)]))

        self.d = dict(g=guarded16(np.zeros(S, np.uint16)), master=guarded32(self.o["master"]),
                      m=guarded32(np.zeros(S, np.float32)), v=guarded32(np.zeros(S, np.float32)),
                      p=guarded16(np.zeros(S, np.uint16)), full=guarded16(np.full(T, SENT, np.uint16)))
        self.dc = {t: [dev16(c) for c in cs] for t, cs in self.mine.items()}
        torch.cuda.synchronize()

    def step(self, t):
        zs, d, hp = self.zs, self.d, self.hp.at(t)
        S = self.S
        if self.fused:
            zs.zs_fused_shard_step(self.plan, hp, self.dc[t], d["master"], d["m"], d["v"],
                                   grad=d["g"], param=d["p"], full=d["full"])
        else:
            B = self.bucket or max(S, 8)
            for off in range(0, S, B):
                zs.zs_reduce_shard(self.plan, self.dc[t], d["g"], off, min(B, S - off))
            zs.zs_adamw_shard_step(self.plan, hp, d["g"], d["master"], d["m"], d["v"], d["p"])
            zs.zs_gather_params(self.plan, d["p"], d["full"])
        o = self.o
        oracle.shard_step(oracle.HParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t),
                          self.mine[t], o["g"], o["master"], o["m"], o["v"], o["p"], o["full"], self.rank)

    def check(self, exact=True):
        import torch
        torch.cuda.synchronize()
        S, T, G = self.S, self.T, self.G
        d, o = self.d, self.o
        diffs = {}
        diffs["g"] = check_bf16(host16(d["g"])[:S], o["g"], "grad")
        diffs["master"] = check_f32(host32(d["master"])[:S], o["master"], "master")
        diffs["m"] = check_f32(host32(d["m"])[:S], o["m"], "m")
        diffs["v"] = check_f32(host32(d["v"])[:S], o["v"], "v")
        diffs["p"] = check_bf16(host16(d["p"])[:S], o["p"], "param")
        full = host16(d["full"])
        # placement in the gathered buffer and every untouched byte: bit-exact
        assert np.array_equal(full[:T], o["full"]), "gathered buffer differs"
        for k in ("g", "p", "full"):
            assert np.all(host16(d[k])[-G:] == SENT), f"guard band after {k} overwritten"
        for k in ("master", "m", "v"):
            assert np.all(host32(d[k])[-G:] == 7.0), f"guard band after {k} overwritten"
        if exact:
            assert not any(diffs.values()), f"not bit-identical: {diffs}"
        return diffs


def _hp(zs, **kw):
    base = dict(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
    base.update(kw)
    return zs.AdamWHParams(**base)


@pytest.mark.parametrize("fused", [False, True])
def test_tiny_config_three_steps(zs, fused):
    """1,000,003-element param padded to N*8, N=4, rank 1, 3 AdamW steps."""
    run = FlatRun(zs, [1_000_003], 4, 1, 1, 3, synth.DEFAULT_SEED, _hp(zs), bucket=65536, fused=fused)
    for t in (1, 2, 3):
        run.step(t)
        run.check()


def test_tiny_all_ranks_equal_unsharded_update(zs):
    """Sharding invariance on the GPU: N ranks' gathered updates == DDP update."""
    import torch
    numels, N, steps = [1_000_003], 4, 2
    T, master, contribs = _flat_inputs(numels, N, 1, steps, 99)
    hp = _hp(zs)
    plans = [zs.zs_shard_plan(numels, N, r, 1) for r in range(N)]
    S = plans[0].shard_numel
    full = dev16(np.full(T, SENT, np.uint16))
    st = [dict(master=dev32(master[r * S:(r + 1) * S]), m=torch.zeros(S, device="cuda"),
               v=torch.zeros(S, device="cuda")) for r in range(N)]
    for t in range(1, steps + 1):
        for r in range(N):
            mine = [dev16(c[r * S:(r + 1) * S]) for c in contribs[t]]
            zs.zs_fused_shard_step(plans[r], hp.at(t), mine, st[r]["master"], st[r]["m"], st[r]["v"],
                                   full=full)
    # DDP reference: every replica reduces the full buffers and updates all of it
    g = np.zeros(T, np.uint16)
    mo, mm, mv, mp = master.copy(), np.zeros(T, np.float32), np.zeros(T, np.float32), np.zeros(T, np.uint16)
    for t in range(1, steps + 1):
        oracle.reduce(contribs[t], out=g)
        oracle.adamw(oracle.HParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t), g, mo, mm, mv, mp)
    torch.cuda.synchronize()
    assert np.array_equal(host16(full), mp)
    got_master = np.concatenate([host32(s["master"]) for s in st])
    assert check_f32(got_master, mo, "master") == 0


@pytest.mark.parametrize("seed", range(12))
def test_random_flat_plans(zs, seed):
    """Alignment gaps, tail padding, odd world sizes (runtime-N kernels), ragged buckets."""
    rnd = random.Random(seed)
    numels = [rnd.choice([1, 7, 64, 100, 768, 4093, 20_000, 65_537]) for _ in range(rnd.randint(1, 8))]
    world = rnd.choice([1, 2, 3, 4, 5, 8, 16, 32, 64, 100])
    rank = rnd.randrange(world)
    align = rnd.choice([1, 8, 128])
    plan = oracle.plan_flat(numels, world, rank, align)
    if plan.S == 0:
        pytest.skip("empty shard")
    bucket = rnd.choice([0, 8, 4096, 8 * rnd.randint(1, 4000)])
    fused = rnd.random() < 0.5
    hp = _hp(zs, lr=rnd.choice([1e-4, 1e-3]), weight_decay=rnd.choice([0.0, 0.1]))
    run = FlatRun(zs, numels, world, rank, align, 2, 1000 + seed, hp, bucket=bucket, fused=fused,
                  zero_prob=0.05)
    for t in (1, 2):
        run.step(t)
    run.check()


@pytest.mark.parametrize("N", [1, 2, 4, 8, 16, 32, 64, 3, 7, 9, 12, 15, 24, 31, 40, 48, 51, 52, 63, 65, 100, 256])
def test_world_sizes(zs, N):
    """Every compiled rank-loop variant (N = 1..64) and the runtime loop:
    remainders of 0 to 7 ranks after its groups of 8, no full group (3, 7),
    one (9..15), odd and even numbers of groups in the two register sets
    taken in turn (24, 40, 48, 256), and both sides of the two-pass
    threshold."""
    rank = N - 1 if N <= 100 else N // 2  # a rank that owns real elements and some padding
    for fused in (False, True):
        run = FlatRun(zs, [50_001], N, rank, 1, 1, 7 + N, _hp(zs), fused=fused)
        run.step(1)
        run.check()


def test_fused_equals_unfused_bit_exact(zs):
    a = FlatRun(zs, [300_017, 5], 8, 3, 128, 3, 5, _hp(zs), bucket=8192, fused=False)
    b = FlatRun(zs, [300_017, 5], 8, 3, 128, 3, 5, _hp(zs), fused=True)
    for t in (1, 2, 3):
        a.step(t)
        b.step(t)
    for k in ("g", "master", "m", "v", "p", "full"):
        assert np.array_equal(a.d[k].cpu().numpy(), b.d[k].cpu().numpy()), k


@pytest.mark.parametrize("N", [4, 64])
def test_fused_buckets_equal_whole_shard(zs, N):
    """The fused step bucket by bucket (ragged buckets and an empty one, in a
    shuffled order) leaves the same bytes as the whole-shard call, which
    matches the oracle; at N=64 each bucket runs in the two-pass form."""
    import torch
    whole = FlatRun(zs, [70_001, 77], N, 1, 1, 2, 400 + N, _hp(zs), fused=True)
    part = FlatRun(zs, [70_001, 77], N, 1, 1, 2, 400 + N, _hp(zs), fused=True)
    S = whole.S
    rng = random.Random(N)
    edges = sorted({0, S} | {8 * k for k in rng.sample(range(1, S // 8), 5)})
    buckets = list(zip(edges[:-1], edges[1:])) + [(edges[2], edges[2])]
    rng.shuffle(buckets)
    d = part.d
    for t in (1, 2):
        whole.step(t)
        for lo, hi in buckets:
            zs.zs_fused_shard_step_bucket(part.plan, part.hp.at(t), part.dc[t], d["master"], d["m"], d["v"], lo,
                                          hi - lo, grad=d["g"], param=d["p"], full=d["full"])
    whole.check()
    torch.cuda.synchronize()
    for k in ("g", "master", "m", "v", "p", "full"):
        a, b = whole.d[k], d[k]
        if a.dtype == torch.float32:
            a, b = a.view(torch.int32), b.view(torch.int32)
        assert torch.equal(a, b), f"bucketed != whole shard: {k}"


@pytest.mark.parametrize("N", [4, 64])
@pytest.mark.parametrize("outs", range(8), ids=lambda o: f"grad{o & 1}-param{(o >> 1) & 1}-full{(o >> 2) & 1}")
def test_fused_optional_outputs(zs, N, outs):
    """Every subset of the fused step's optional outputs (grad shard, param
    shard, gathered slice), in the one-pass form (N=4) and at N=64, where
    the step runs as two passes when the grad shard is written: enabled
    outputs equal the oracle's, disabled ones keep their sentinel bytes."""
    import torch
    want_g, want_p, want_f = bool(outs & 1), bool(outs & 2), bool(outs & 4)
    run = FlatRun(zs, [40_003, 77], N, N - 1, 1, 2, 300 + outs, _hp(zs), fused=True)
    S, T = run.S, run.T
    for buf in ("g", "p", "full"):
        run.d[buf].fill_(SENT)
    d = run.d
    for t in (1, 2):
        hp = run.hp.at(t)
        zs.zs_fused_shard_step(run.plan, hp, run.dc[t], d["master"], d["m"], d["v"], grad=d["g"] if want_g else None,
                               param=d["p"] if want_p else None, full=d["full"] if want_f else None)
        o = run.o
        oracle.shard_step(oracle.HParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t), run.mine[t],
                          o["g"], o["master"], o["m"], o["v"], o["p"], o["full"], run.rank)
    torch.cuda.synchronize()
    nd = check_f32(host32(d["master"])[:S], o["master"], "master") + check_f32(host32(d["m"])[:S], o["m"], "m")
    nd += check_f32(host32(d["v"])[:S], o["v"], "v")
    g, p, full = host16(d["g"]), host16(d["p"]), host16(d["full"])
    if want_g:
        nd += check_bf16(g[:S], o["g"], "grad")
    else:
        assert np.all(g == SENT), "grad written although not requested"
    if want_p:
        nd += check_bf16(p[:S], o["p"], "param")
    else:
        assert np.all(p == SENT), "param written although not requested"
    if want_f:
        assert np.array_equal(full[:T], o["full"]), "gathered buffer"
    else:
        assert np.all(full == SENT), "gathered buffer written although not requested"
    assert np.all(g[S:] == SENT) and np.all(p[S:] == SENT) and np.all(full[T:] == SENT), "guard bands"
    assert nd == 0


def test_edge_values(zs):
    """Signed zeros, subnormals, huge values, inf and NaN in the contributions."""
    import torch
    S, N = 4096, 4
    plan = zs.zs_shard_plan([S * N], N, 0, 1)
    rng = np.random.default_rng(3)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F,
                         0x7F80, 0xFF80, 0x7FC0, 0x3F80, 0xBF80, 0x1234, 0x9234, 0x4000], np.uint16)
    cs = [rng.choice(specials, S).astype(np.uint16) for _ in range(N)]
    master = rng.standard_normal(S).astype(np.float32) * 0.02
    master[:16] = [0, -0.0, 1e-45, -1e-45, 3e38, -3e38, 1e-38, np.inf, -np.inf, np.nan, 1, -1, 2, 0.5, 1e-30, 7]
    hp = _hp(zs, lr=1e-3)
    d_m, d_v = torch.zeros(S, device="cuda"), torch.zeros(S, device="cuda")
    d_master = dev32(master)
    d_g, d_p = dev16(np.zeros(S, np.uint16)), dev16(np.zeros(S, np.uint16))
    zs.zs_fused_shard_step(plan, hp, [dev16(c) for c in cs], d_master, d_m, d_v, grad=d_g, param=d_p)
    g = oracle.reduce(cs)
    m, v, p = np.zeros(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.uint16)
    mo = master.copy()
    oracle.adamw(oracle.HParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1), g, mo, m, v, p)
    torch.cuda.synchronize()
    nd = check_bf16(host16(d_g), g, "grad")
    nd += check_f32(host32(d_master), mo, "master")
    nd += check_f32(host32(d_m), m, "m")
    nd += check_f32(host32(d_v), v, "v")
    nd += check_bf16(host16(d_p), p, "param")
    assert nd == 0, f"{nd} non-NaN elements not bit-identical"
    assert np.isnan(mo).sum() > 100  # the case does exercise NaN propagation


def test_empty_and_minimal_shards(zs):
    import torch
    hp = _hp(zs)
    empty = zs.zs_shard_plan([], 4, 0)
    z = torch.zeros(8, device="cuda")
    z16 = torch.zeros(8, dtype=torch.int16, device="cuda")
    zs.zs_fused_shard_step(empty, hp, [z16] * 4, z, z, z, grad=z16, param=z16, full=z16)
    zs.zs_adamw_shard_step(empty, hp, z16, z, z, z, z16)
    zs.zs_gather_params(empty, z16, z16)
    run = FlatRun(zs, [3], 1, 0, 1, 2, 4, hp, fused=False)  # S = 8: one vector, 5 of it padding
    run.step(1)
    run.step(2)
    run.check()
    torch.cuda.synchronize()


def test_error_paths_on_device_buffers(zs):
    import torch
    plan = zs.zs_shard_plan([1024], 4, 0)
    S = plan.shard_numel
    cs = [torch.zeros(S, dtype=torch.int16, device="cuda") for _ in range(4)]
    g = torch.zeros(S + 8, dtype=torch.int16, device="cuda")
    with pytest.raises(zs.ZsError) as e:
        zs.zs_reduce_shard(plan, cs[:3], g)
    assert e.value.status == zs.ZS_EINVAL
    with pytest.raises(zs.ZsError) as e:
        zs.zs_reduce_shard(plan, cs, g[1:], 0, S)  # 2-byte misaligned output
    assert e.value.status == zs.ZS_EALIGN
    with pytest.raises(zs.ZsError) as e:
        zs.zs_reduce_shard(plan, cs, g, 8, S)  # bucket beyond the shard
    assert e.value.status in (zs.ZS_ERANGE,)
    with pytest.raises(ValueError):
        zs.zs_reduce_shard(plan, [c[:8] for c in cs], g)  # too short for the call
    bad = zs.AdamWHParams(step=0)
    with pytest.raises(zs.ZsError):
        zs.zs_adamw_shard_step(plan, bad, g, torch.zeros(S, device="cuda"), torch.zeros(S, device="cuda"),
                               torch.zeros(S, device="cuda"), g)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- multi-tensor


def _small_model(H=256, I=688, V=1000, L=2):
    sizes = [V * H]
    for _ in range(L):
        sizes += [H * H, H * H, H * H, H * H, I * H, I * H, H * I, H, H]
    sizes += [H, V * H, 1000, 3]  # plus two sizes that need per-tensor padding
    return sizes


class MultiRun:
    """PER_TENSOR multi-tensor step against the oracle. With ``hps`` (one set
    of hyperparameters per group) the *_groups calls run and piece i uses
    hps[groups[i]]; ``persist_below`` replicates the small tensors."""

    def __init__(self, zs, numels, world, rank, steps, seed, hp, persist_below=0, groups=None, hps=None,
                 replicas=1):
        import torch
        self.zs, self.hp, self.world, self.rank = zs, hp, world, rank
        self.n_contribs = world * replicas
        self.groups, self.hps = groups, hps
        if persist_below or groups is not None:
            self.plan = zs.zs_shard_plan_ex(numels, world, rank, persist_below_elems=persist_below, groups=groups)
        else:
            self.plan = zs.zs_shard_plan(numels, world, rank, 1, zs.ZS_LAYOUT_PER_TENSOR)
        self.oplan = oracle.plan_per_tensor(numels, world, rank, persist_below)
        self.pieces = []
        self.o = []
        self.contribs = {}
        for i, pc in enumerate(self.oplan.pieces):
            Si = pc.own_hi - pc.own_lo
            base = pc.full_off  # packed global index of the piece's first element
            valid = self.oplan.offsets[i] + numels[i]
            master = synth.cpu_f32(Si, base, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02, valid))
            self.o.append(dict(g=np.zeros(Si, np.uint16), master=master.copy(), m=np.zeros(Si, np.float32),
                               v=np.zeros(Si, np.float32), p=np.zeros(Si, np.uint16),
                               full=np.full(self.oplan.padded[i], SENT, np.uint16)))
            self.pieces.append(dict(grad=torch.zeros(Si, dtype=torch.int16, device="cuda"), master=dev32(master),
                                    m=torch.zeros(Si, device="cuda"), v=torch.zeros(Si, device="cuda"),
                                    param=torch.zeros(Si, dtype=torch.int16, device="cuda"),
                                    full=dev16(np.full(self.oplan.padded[i], SENT, np.uint16))))
            for t in range(1, steps + 1):
                for q in range(self.n_contribs):
                    c = synth.cpu_bf16(Si, base, synth.spec(seed, synth.STREAM_CONTRIB + q, t, 1e-3, valid))
                    self.contribs.setdefault(t, [[None] * len(numels) for _ in range(self.n_contribs)])[q][i] = c
        self.dcontribs = {t: [[dev16(c) for c in row] for row in cs] for t, cs in self.contribs.items()}
        nbytes = zs.zs_multi_workspace_bytes(self.plan, self.n_contribs)
        self.ws = {t: torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for t in self.contribs}
        for t in self.contribs:
            zs.zs_multi_bind(self.plan, self.pieces, self.dcontribs[t], self.ws[t])

    def step(self, t, fused):
        zs = self.zs
        hp = self.hp.at(t)
        hps = None if self.hps is None else [x.at(t) for x in self.hps]
        if fused and hps is None:
            zs.zs_fused_shard_step_multi(self.plan, hp, self.ws[t])
        elif fused:
            zs.zs_fused_shard_step_multi_groups(self.plan, hps, self.ws[t])
        else:
            zs.zs_reduce_shard_multi(self.plan, self.ws[t])
            if hps is None:
                zs.zs_adamw_shard_step_multi(self.plan, hp, self.ws[t])
            else:
                zs.zs_adamw_shard_step_multi_groups(self.plan, hps, self.ws[t])
            zs.zs_gather_params_multi(self.plan, self.ws[t])

        def ohp(x):
            return oracle.HParams(x.lr, x.beta1, x.beta2, x.eps, x.weight_decay, t)

        for i, pc in enumerate(self.oplan.pieces):
            h = ohp(hp) if hps is None else ohp(hps[self.groups[pc.tensor] if self.groups else 0])
            o = self.o[i]
            if o["g"].size == 0:
                continue
            cs = [self.contribs[t][q][i] for q in range(self.n_contribs)]
            oracle.reduce(cs, out=o["g"])
            oracle.adamw(h, o["g"], o["master"], o["m"], o["v"], o["p"])
            o["full"][pc.own_lo:pc.own_hi] = o["p"]

    def check(self):
        import torch
        torch.cuda.synchronize()
        nd = 0
        for i, (o, d) in enumerate(zip(self.o, self.pieces)):
            nd += check_bf16(host16(d["grad"]), o["g"], f"grad[{i}]")
            nd += check_f32(host32(d["master"]), o["master"], f"master[{i}]")
            nd += check_f32(host32(d["m"]), o["m"], f"m[{i}]")
            nd += check_f32(host32(d["v"]), o["v"], f"v[{i}]")
            nd += check_bf16(host16(d["param"]), o["p"], f"param[{i}]")
            assert np.array_equal(host16(d["full"]), o["full"]), f"gathered tensor {i}"
        assert nd == 0, f"{nd} elements not bit-identical"


@pytest.mark.parametrize("world", [8, 64])
@pytest.mark.parametrize("fused", [False, True])
def test_multi_tensor_apply(zs, fused, world):
    """At 64 ranks the fused call (grad bound) runs as two launches."""
    run = MultiRun(zs, _small_model(), world, 3, 2, 77, _hp(zs))
    for t in (1, 2):
        run.step(t, fused)
        run.check()


@pytest.mark.parametrize("world", [8, 64])
@pytest.mark.parametrize("outs", range(8), ids=lambda o: f"grad{o & 1}-param{(o >> 1) & 1}-full{(o >> 2) & 1}")
def test_multi_tensor_fused_optional_fields(zs, outs, world):
    """The fused multi-tensor step bound with every subset of its optional
    fields (grad, param, gathered tensor): bound outputs equal the oracle's,
    unbound ones are never written (at 64 ranks with grad bound: the
    two-launch form)."""
    import torch
    run = MultiRun(zs, _small_model(), world, 5, 2, 90 + outs, _hp(zs))
    keep = dict(grad=bool(outs & 1), param=bool(outs & 2), full=bool(outs & 4))
    for d in run.pieces:
        for k in keep:
            d[k].fill_(SENT)
    for t in (1, 2):
        ws = torch.zeros(zs.zs_multi_workspace_bytes(run.plan, run.n_contribs), dtype=torch.uint8, device="cuda")
        zs.zs_multi_bind(run.plan, [{k: (v if keep.get(k, True) else None) for k, v in d.items()}
                                    for d in run.pieces], run.dcontribs[t], ws)
        zs.zs_fused_shard_step_multi(run.plan, run.hp.at(t), ws)
        h = oracle.HParams(run.hp.lr, run.hp.beta1, run.hp.beta2, run.hp.eps, run.hp.weight_decay, t)
        for i, pc in enumerate(run.oplan.pieces):
            o = run.o[i]
            cs = [run.contribs[t][q][i] for q in range(run.n_contribs)]
            oracle.reduce(cs, out=o["g"])
            oracle.adamw(h, o["g"], o["master"], o["m"], o["v"], o["p"])
            o["full"][pc.own_lo:pc.own_hi] = o["p"]
    torch.cuda.synchronize()
    nd = 0
    for i, (o, d) in enumerate(zip(run.o, run.pieces)):
        nd += check_f32(host32(d["master"]), o["master"], f"master[{i}]")
        nd += check_f32(host32(d["m"]), o["m"], f"m[{i}]") + check_f32(host32(d["v"]), o["v"], f"v[{i}]")
        g, p, f = host16(d["grad"]), host16(d["param"]), host16(d["full"])
        if keep["grad"]:
            nd += check_bf16(g, o["g"], f"grad[{i}]")
        else:
            assert np.all(g == SENT), f"grad[{i}] written although not bound"
        if keep["param"]:
            nd += check_bf16(p, o["p"], f"param[{i}]")
        else:
            assert np.all(p == SENT), f"param[{i}] written although not bound"
        if keep["full"]:
            assert np.array_equal(f, o["full"]), f"gathered tensor {i}"
        else:
            assert np.all(f == SENT), f"gathered tensor {i} written although not bound"
    assert nd == 0


def test_multi_tensor_unbound_workspace_is_inert(zs):
    """A workspace whose table was unbound, or whose memory was overwritten
    after binding, launches nothing that touches the pieces."""
    import torch
    run = MultiRun(zs, _small_model(H=128, I=344, V=300, L=1), 4, 1, 1, 81, _hp(zs))
    before = [{k: v.clone() for k, v in d.items()} for d in run.pieces]
    ws = run.ws[1]
    ws.zero_()  # the host still records the binding; the table's tag is gone
    zs.zs_fused_shard_step_multi(run.plan, _hp(zs), ws)
    zs.zs_reduce_shard_multi(run.plan, ws)
    zs.zs_gather_params_multi(run.plan, ws)
    torch.cuda.synchronize()
    for d, b in zip(run.pieces, before):
        for k in d:
            assert torch.equal(d[k], b[k]), k
    zs.zs_multi_unbind(ws)
    with pytest.raises(zs.ZsError):
        zs.zs_fused_shard_step_multi(run.plan, _hp(zs), ws)
    with pytest.raises(zs.ZsError):
        zs.zs_multi_unbind(ws)


@pytest.mark.parametrize("N", [5, 24])
def test_multi_tensor_runtime_world(zs, N):
    run = MultiRun(zs, _small_model(H=128, I=344, V=300, L=1), N, N - 1, 1, 78, _hp(zs))
    run.step(1, True)
    run.check()


@pytest.mark.parametrize("world,replicas,fused", [(4, 2, False), (4, 2, True), (8, 8, True), (2, 3, True)])
def test_hybrid_sharding(zs, world, replicas, fused):
    """Shards cut `world` ways, `replicas` groups: world*replicas contributions
    averaged (8*8 = 64 takes the two-pass large-N fused path)."""
    run = FlatRun(zs, [300_007, 4099], world, world - 1, 1, 2, 57, _hp(zs), bucket=40_000, fused=fused,
                  replicas=replicas)
    for t in (1, 2):
        run.step(t)
        run.check()


def test_multi_tensor_hybrid(zs):
    """Per-tensor pieces of a 4-way shard with 3 replica groups (12 contributions)."""
    run = MultiRun(zs, _small_model(H=128, I=344, V=300, L=1), 4, 2, 2, 79, _hp(zs), replicas=3)
    for t in (1, 2):
        run.step(t, True)
        run.check()


def _norm_groups(numels, H):
    """Group 1 (no weight decay, other lr) for vectors such as norm weights, group 0 otherwise."""
    return [1 if n <= H or n in (1000, 3) else 0 for n in numels]


@pytest.mark.parametrize("fused", [False, True])
def test_multi_tensor_persistence_and_groups(zs, fused):
    """Tensors below the threshold are replicated (whole tensor reduced and
    updated on every rank); norms and odd sizes use a second hyperparameter
    group without weight decay."""
    numels = _small_model()
    groups = _norm_groups(numels, 256)
    hps = [_hp(zs), zs.AdamWHParams(lr=3e-4, beta1=0.8, beta2=0.99, eps=1e-6, weight_decay=0.0)]
    run = MultiRun(zs, numels, 8, 5, 3, 91, _hp(zs), persist_below=2048, groups=groups, hps=hps)
    assert any(run.plan.tensor_replicated(i) for i in range(len(numels)))
    assert any(not run.plan.tensor_replicated(i) for i in range(len(numels)))
    for t in (1, 2, 3):
        run.step(t, fused)
        run.check()


def test_multi_tensor_groups_all_replicated(zs):
    """Every tensor below the threshold: the step is plain data parallelism on each rank."""
    numels = [100, 7, 2000, 3, 9]
    hps = [_hp(zs), zs.AdamWHParams(lr=1e-3, weight_decay=0.0)]
    run = MultiRun(zs, numels, 4, 0, 2, 92, _hp(zs), persist_below=1 << 20, groups=[0, 1, 0, 1, 1], hps=hps)
    assert run.plan.shard_numel == sum((n + 7) // 8 * 8 for n in numels)
    for t in (1, 2):
        run.step(t, True)
        run.check()


def test_generator_gpu_equals_host(zs):
    import torch
    n = 1_000_003
    for sp in (synth.spec(3, synth.STREAM_MASTER, 0, 0.02, n - 5),
               synth.spec(3, synth.STREAM_CONTRIB + 5, 2, 1e-3, 2**62, 0.1, 0.001, 0.01)):
        a = torch.empty(n, dtype=torch.float32, device="cuda")
        synth.gpu_f32(a, 12345, sp)
        b = torch.empty(n, dtype=torch.int16, device="cuda")
        synth.gpu_bf16(b, 12345, sp)
        torch.cuda.synchronize()
        assert np.array_equal(host32(a).view(np.uint32), synth.cpu_f32(n, 12345, sp).view(np.uint32))
        assert np.array_equal(host16(b), synth.cpu_bf16(n, 12345, sp))
