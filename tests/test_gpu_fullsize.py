"""GPU <-> oracle parity at the workloads' full sizes, on sampled elements.

Inputs are generated on the device by the GPU build of the seeded generator;
the oracle recomputes each sampled element from the host build's values of the
same global indices (no input of the oracle comes from the device). Each
workload runs through the entry points the benchmark times, in the same
launch configuration: the one-pass fused kernel at N <= 8, and at N = 64 the
fused entry point with the grad shard given, which runs the reduce and then
AdamW writing the gathered slice (the one-pass form is checked there too).
Samples: the first and last 2,048 owned elements, both sides of every
reduce-bucket boundary, and random positions; fused and unfused results are
also compared on every element. Ranks other than 0 are included, so the owned
slice of the gathered buffer starts at a nonzero offset r*S.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_bf16, check_f32

pytestmark = pytest.mark.gpu

SENT = 0x5A5A


@pytest.fixture(scope="module")
def zs():
    import torch

    import fsdp_sharded_mixed_flatten_amd as m
    torch.cuda.init()
    return m


def _free_gib():
    import torch
    free, _ = torch.cuda.mem_get_info()
    return free / 2**30


def _release():
    import gc

    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _samples(S, bucket, n_random, seed):
    rng = np.random.default_rng(seed)
    idx = [np.arange(0, min(S, 2048)), np.arange(max(0, S - 2048), S), rng.integers(0, S, n_random)]
    if bucket:
        for b in range(bucket, S, bucket):
            idx.append(np.arange(b - 8, min(b + 8, S)))
    return np.unique(np.concatenate(idx)).astype(np.int64)


class FlatBig:
    """One rank's FLAT shard at full size; device inputs from the GPU generator."""

    def __init__(self, zs, wl, n_random=200_000, rank=None):
        import torch
        self.zs, self.wl = zs, wl
        self.rank = wl.rank if rank is None else rank
        self.plan = zs.zs_shard_plan(wl.numels, wl.world, self.rank, wl.align, zs.ZS_LAYOUT_FLAT)
        self.S, self.T = self.plan.shard_numel, self.plan.padded_numel
        self.base = self.rank * self.S
        self.valid_hi = sum(wl.numels)  # only tail padding in these shapes (checked below)
        assert oracle.plan_flat(wl.numels, wl.world, self.rank, wl.align).T == self.T
        assert all(n % wl.align == 0 for n in wl.numels[:-1])
        self.idx = _samples(self.S, wl.bucket_elems, n_random, 17)
        self.didx = torch.from_numpy(self.idx).cuda()
        S = self.S
        print(f"[{wl.name}] N={wl.world} rank={self.rank} S={S:,} samples={self.idx.size:,}", flush=True)
        self.contribs = [torch.empty(S, dtype=torch.int16, device="cuda") for _ in range(wl.world)]
        self.master = torch.empty(S, dtype=torch.float32, device="cuda")
        synth.gpu_f32(self.master, self.base, wl.master_spec(self.valid_hi))
        self.m = torch.zeros(S, dtype=torch.float32, device="cuda")
        self.v = torch.zeros(S, dtype=torch.float32, device="cuda")
        # oracle state on the samples
        gi = self.base + self.idx
        self.o_master = synth.cpu_at_f32(gi, wl.master_spec(self.valid_hi))
        K = self.idx.size
        self.o_m, self.o_v = np.zeros(K, np.float32), np.zeros(K, np.float32)
        self.o_g, self.o_p = np.zeros(K, np.uint16), np.zeros(K, np.uint16)

    def gen_contribs(self, t):
        for q, c in enumerate(self.contribs):
            synth.gpu_bf16(c, self.base, self.wl.contrib_spec(q, t, self.valid_hi))

    def oracle_step(self, t, hp):
        gi = self.base + self.idx
        cs = [synth.cpu_at_bf16(gi, self.wl.contrib_spec(q, t, self.valid_hi)) for q in range(self.wl.world)]
        oracle.reduce(cs, out=self.o_g)
        oracle.adamw(oracle.HParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t), self.o_g,
                     self.o_master, self.o_m, self.o_v, self.o_p)

    def pick16(self, t):
        return t.index_select(0, self.didx).cpu().numpy().view(np.uint16)

    def pick32(self, t):
        return t.index_select(0, self.didx).cpu().numpy()

    def check_state(self, tag):
        nd = check_f32(self.pick32(self.master), self.o_master, f"{tag} master")
        nd += check_f32(self.pick32(self.m), self.o_m, f"{tag} m")
        nd += check_f32(self.pick32(self.v), self.o_v, f"{tag} v")
        return nd


def _hp(zs, wl):
    return zs.AdamWHParams(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, 1)


def test_qwen3b_shape_fused_after_warm_step(zs):
    import torch
    wl = synth.workloads()["qwen3b"]
    if _free_gib() < 40:
        pytest.skip("needs ~30 GiB of free device memory")
    run = FlatBig(zs, wl)
    S = run.S
    assert S == 771_484_672
    hp = _hp(zs, wl)
    full = torch.full((run.T,), SENT, dtype=torch.int16, device="cuda")
    grad = torch.empty(S, dtype=torch.int16, device="cuda")
    param = torch.empty(S, dtype=torch.int16, device="cuda")
    for t in range(1, wl.first_step + 1):  # warm step t=1 from m = v = 0, then the measured t=2
        run.gen_contribs(t)
        zs.zs_fused_shard_step(run.plan, hp.at(t), run.contribs, run.master, run.m, run.v,
                               grad=grad, param=param, full=full)
        run.oracle_step(t, hp)
    torch.cuda.synchronize()
    nd = run.check_state("qwen3b")
    nd += check_bf16(run.pick16(grad), run.o_g, "grad")
    nd += check_bf16(run.pick16(param), run.o_p, "param")
    assert np.array_equal(run.pick16(full[:S]), run.o_p)  # rank 0: the owned slice starts at 0
    tail = full[S:S + 1_000_000].cpu().numpy().view(np.uint16)
    assert np.all(tail == SENT), "the gather wrote outside the owned slice"
    assert nd == 0, f"{nd} sampled elements not bit-identical"
    del run, full, grad, param
    _release()


def test_llama7b_shape_ten_steps_bucketed_and_fused(zs):
    import torch
    wl = synth.workloads()["llama7b"]
    if _free_gib() < 60:
        pytest.skip("needs ~50 GiB of free device memory")
    run = FlatBig(zs, wl)
    S, B = run.S, wl.bucket_elems
    assert S == 842_301_952
    hp = _hp(zs, wl)
    # a second state for the fused path
    f_master = run.master.clone()
    f_m, f_v = torch.zeros_like(run.m), torch.zeros_like(run.v)
    grad = torch.empty(S, dtype=torch.int16, device="cuda")
    f_grad = torch.empty_like(grad)
    param = torch.empty_like(grad)
    f_param = torch.empty_like(grad)
    full = torch.full((run.T,), SENT, dtype=torch.int16, device="cuda")
    for t in range(1, wl.steps + 1):
        run.gen_contribs(t)
        for off in range(0, S, B):  # 33 buckets of 25M + one of 17,301,952
            zs.zs_reduce_shard(run.plan, run.contribs, grad, off, min(B, S - off))
        zs.zs_adamw_shard_step(run.plan, hp.at(t), grad, run.master, run.m, run.v, param)
        zs.zs_gather_params(run.plan, param, full)
        zs.zs_fused_shard_step(run.plan, hp.at(t), run.contribs, f_master, f_m, f_v, grad=f_grad,
                               param=f_param)
        run.oracle_step(t, hp)
        if t in (1, wl.steps):
            torch.cuda.synchronize()
            nd = run.check_state(f"llama7b t={t}")
            nd += check_bf16(run.pick16(grad), run.o_g, "grad")
            nd += check_bf16(run.pick16(param), run.o_p, "param")
            assert nd == 0, f"{nd} sampled elements not bit-identical at t={t}"
            # the shared exact zeros: g == 0 exactly where every contribution is 0
            zero_frac = (run.o_g == 0).mean()
            assert 0.005 < zero_frac < 0.02
    torch.cuda.synchronize()
    for a, b, k in ((run.master, f_master, "master"), (run.m, f_m, "m"), (run.v, f_v, "v"),
                    (grad, f_grad, "grad"), (param, f_param, "param")):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b), f"fused != bucketed: {k}"
    assert torch.equal(full[:S], param)
    assert bool((full[S:] == SENT).all())
    del run, full, grad, param, f_master, f_m, f_v, f_grad, f_param
    _release()


@pytest.mark.parametrize("persist,world,rank", [(0, 8, 0), (100_000, 8, 0), (0, 64, 41)])
def test_llama7b_wrap_stress_multi_tensor(zs, persist, world, rank):
    """The 291-piece per-tensor plan; with persist=100,000 (the threshold the
    pages suggest) the 65 norm vectors are replicated and updated whole with a
    second hyperparameter group (no weight decay), as an FSDP2 model would
    hold them. At 64 ranks (rank 41) the fused call, with the grad pieces
    bound, runs as two launches."""
    import dataclasses

    import torch
    wl = dataclasses.replace(synth.workloads()["llama7b_wrap"], world=world, rank=rank)
    if _free_gib() < 60:
        pytest.skip("needs ~50 GiB of free device memory")
    groups = [1 if n < persist else 0 for n in wl.numels] if persist else None
    if persist:
        plan = zs.zs_shard_plan_ex(wl.numels, wl.world, wl.rank, persist_below_elems=persist, groups=groups)
    else:
        plan = zs.zs_shard_plan(wl.numels, wl.world, wl.rank, 1, zs.ZS_LAYOUT_PER_TENSOR)
    op = oracle.plan_per_tensor(wl.numels, wl.world, wl.rank, persist)
    assert len(op.pieces) == 291
    assert sum(1 for i in range(291) if zs.lib().zs_plan_tensor_replicated(plan.handle, i) == 1) == \
        (65 if persist else 0)
    print(f"[llama7b_wrap persist={persist}] pieces={len(op.pieces)} S={plan.shard_numel:,}", flush=True)
    rng = np.random.default_rng(5)
    pieces, contribs, samples = [], [[] for _ in range(wl.world)], []
    for i, pc in enumerate(op.pieces):
        Si = pc.own_hi - pc.own_lo
        valid = op.offsets[i] + wl.numels[i]
        d = dict(grad=torch.empty(Si, dtype=torch.int16, device="cuda"),
                 master=torch.empty(Si, dtype=torch.float32, device="cuda"),
                 m=torch.zeros(Si, dtype=torch.float32, device="cuda"),
                 v=torch.zeros(Si, dtype=torch.float32, device="cuda"),
                 param=torch.empty(Si, dtype=torch.int16, device="cuda"),
                 full=torch.full((op.padded[i],), SENT, dtype=torch.int16, device="cuda"))
        synth.gpu_f32(d["master"], pc.full_off, wl.master_spec(valid))
        pieces.append(d)
        for q in range(wl.world):
            c = torch.empty(Si, dtype=torch.int16, device="cuda")
            synth.gpu_bf16(c, pc.full_off, wl.contrib_spec(q, 1, valid))
            contribs[q].append(c)
        s = np.unique(np.concatenate([np.arange(min(Si, 16)), np.arange(max(0, Si - 16), Si),
                                      rng.integers(0, Si, 32)])).astype(np.int64)
        samples.append((s, valid))
    ws = torch.zeros(zs.zs_multi_workspace_bytes(plan, wl.world), dtype=torch.uint8, device="cuda")
    zs.zs_multi_bind(plan, pieces, contribs, ws)
    hp = _hp(zs, wl)
    hps = [hp, zs.AdamWHParams(wl.lr, wl.beta1, wl.beta2, wl.eps, 0.0, 1)]
    if persist:
        zs.zs_fused_shard_step_multi_groups(plan, hps, ws)
    else:
        zs.zs_fused_shard_step_multi(plan, hp, ws)
    torch.cuda.synchronize()
    nd = 0
    for i, pc in enumerate(op.pieces):
        x = hps[groups[pc.tensor]] if persist else hp
        h = oracle.HParams(x.lr, x.beta1, x.beta2, x.eps, x.weight_decay, 1)
        s, valid = samples[i]
        gi = pc.full_off + s
        cs = [synth.cpu_at_bf16(gi, wl.contrib_spec(q, 1, valid)) for q in range(wl.world)]
        g = oracle.reduce(cs)
        mst = synth.cpu_at_f32(gi, wl.master_spec(valid))
        m, v, p = np.zeros(s.size, np.float32), np.zeros(s.size, np.float32), np.zeros(s.size, np.uint16)
        oracle.adamw(h, g, mst, m, v, p)
        ds = torch.from_numpy(s).cuda()
        d = pieces[i]
        nd += check_bf16(d["grad"].index_select(0, ds).cpu().numpy().view(np.uint16), g, f"grad[{i}]")
        nd += check_f32(d["master"].index_select(0, ds).cpu().numpy(), mst, f"master[{i}]")
        nd += check_f32(d["m"].index_select(0, ds).cpu().numpy(), m, f"m[{i}]")
        nd += check_f32(d["v"].index_select(0, ds).cpu().numpy(), v, f"v[{i}]")
        nd += check_bf16(d["param"].index_select(0, ds).cpu().numpy().view(np.uint16), p, f"param[{i}]")
        full = d["full"]
        own = full[pc.own_lo:pc.own_hi]
        assert torch.equal(own, d["param"]), f"gathered tensor {i}"
        if pc.own_lo > 0:
            assert bool((full[:pc.own_lo] == SENT).all())
        assert bool((full[pc.own_hi:] == SENT).all())
    assert nd == 0, f"{nd} sampled elements not bit-identical"
    del pieces, contribs, ws
    _release()


@pytest.mark.parametrize("form,rank", [("two_pass", 63), ("one_pass", 0)])
def test_llama70b_shape_fused(zs, form, rank):
    """The 70B shard at N=64. two_pass: the fused entry point with the grad
    shard given, as the benchmark runs it (the reduce into the grad shard,
    then AdamW writing the gathered slice), at rank 63, whose owned slice
    starts at 63*S in the 70.6 G-element gathered buffer. one_pass: no grad
    shard, the single fused kernel, at rank 0."""
    import torch
    wl = synth.workloads()["llama70b"]
    _release()
    plan_o = oracle.plan_flat(wl.numels, wl.world, rank, wl.align)
    S, T = plan_o.S, plan_o.T
    need = (wl.world * 2 + 14) * S / 2**30 + 4
    free = _free_gib()
    # the owned slice of a nonzero rank lies at r*S, so it needs the whole T
    # gathered buffer; rank 0 can use [0, S) plus a guard band
    full_elems = T if (rank > 0 or free - need > T * 2 / 2**30 + 4) else S + 1_000_000
    need += full_elems * 2 / 2**30
    if free < need:
        pytest.skip(f"needs {need:.0f} GiB of free device memory, {free:.0f} GiB free")
    run = FlatBig(zs, wl, n_random=100_000, rank=rank)
    lo = rank * S
    hp = _hp(zs, wl)
    full = torch.full((full_elems,), SENT, dtype=torch.int16, device="cuda")
    grad = torch.full((S,), SENT, dtype=torch.int16, device="cuda") if form == "two_pass" else None
    print(f"[llama70b] {form} rank {rank}: gathered buffer elements {full_elems:,}", flush=True)
    run.gen_contribs(1)
    zs.zs_fused_shard_step(run.plan, hp, run.contribs, run.master, run.m, run.v, grad=grad, full=full)
    run.oracle_step(1, hp)
    torch.cuda.synchronize()
    nd = run.check_state(f"llama70b {form}")
    nd += check_bf16(run.pick16(full[lo:lo + S]), run.o_p, "gathered param")
    if grad is not None:
        nd += check_bf16(run.pick16(grad), run.o_g, "grad")
    assert nd == 0, f"{nd} sampled elements not bit-identical"
    # guard bands on both sides of the owned slice keep their sentinels
    if lo > 0:
        assert bool((full[lo - 1_000_000:lo] == SENT).all()), "the gather wrote before the owned slice"
    if lo + S < full_elems:
        assert bool((full[lo + S:lo + S + 1_000_000] == SENT).all()), "the gather wrote past the owned slice"
    # heavy tails are present in the sampled contributions' average
    assert np.abs(oracle.bf16_to_f32(run.o_g)).max() > 3e-3
    del run, full, grad
    _release()


def test_llama7b_shape_fused_at_rank_5(zs):
    """The 7B shard (N=8) of rank 5 through the one-pass fused kernel as the
    benchmark runs it (gathered slice written, no grad or param shard), two
    steps: the owned slice starts at 5*S of the gathered buffer, the ranks'
    slices around it keep their sentinels."""
    import torch
    wl = synth.workloads()["llama7b"]
    if _free_gib() < 60:
        pytest.skip("needs ~50 GiB of free device memory")
    rank = 5
    run = FlatBig(zs, wl, rank=rank)
    S, T = run.S, run.T
    lo = rank * S
    hp = _hp(zs, wl)
    full = torch.full((T,), SENT, dtype=torch.int16, device="cuda")
    for t in (1, 2):
        run.gen_contribs(t)
        zs.zs_fused_shard_step(run.plan, hp.at(t), run.contribs, run.master, run.m, run.v, full=full)
        run.oracle_step(t, hp)
    torch.cuda.synchronize()
    nd = run.check_state("llama7b rank 5")
    nd += check_bf16(run.pick16(full[lo:lo + S]), run.o_p, "gathered param")
    assert nd == 0, f"{nd} sampled elements not bit-identical"
    assert bool((full[:lo] == SENT).all()), "the gather wrote into lower ranks' slices"
    assert bool((full[lo + S:] == SENT).all()), "the gather wrote into higher ranks' slices"
    del run, full
    _release()


@pytest.mark.parametrize("world,rank", [(48, 47), (56, 13)])
def test_llama7b_shape_runtime_world_sizes(zs, world, rank):
    """The Llama-7B shape cut for world sizes without a compiled rank loop,
    through the runtime loop at full size: N=48 (six groups of 8, the one-pass
    fused kernel) and N=56 with the grad shard given (seven groups, the
    two-pass form), two steps each, at a nonzero rank whose slice of the
    gathered buffer starts at r*S; grad, param and gathered slice sampled
    against the oracle, the other ranks' slices kept."""
    import dataclasses

    import torch
    wl = dataclasses.replace(synth.workloads()["llama7b"], world=world, bucket_elems=0)
    if _free_gib() < 50:
        pytest.skip("needs ~40 GiB of free device memory")
    run = FlatBig(zs, wl, n_random=100_000, rank=rank)
    S, T = run.S, run.T
    lo = rank * S
    hp = _hp(zs, wl)
    full = torch.full((T,), SENT, dtype=torch.int16, device="cuda")
    two_pass = world >= zs.FUSED_TWO_PASS_MIN_CONTRIBS
    grad = torch.full((S,), SENT, dtype=torch.int16, device="cuda") if two_pass else None
    for t in (1, 2):
        run.gen_contribs(t)
        zs.zs_fused_shard_step(run.plan, hp.at(t), run.contribs, run.master, run.m, run.v, grad=grad, full=full)
        run.oracle_step(t, hp)
    torch.cuda.synchronize()
    nd = run.check_state(f"llama7b N={world} rank {rank}")
    nd += check_bf16(run.pick16(full[lo:lo + S]), run.o_p, "gathered param")
    if two_pass:
        nd += check_bf16(run.pick16(grad), run.o_g, "grad")
    assert nd == 0, f"{nd} sampled elements not bit-identical"
    assert bool((full[:lo] == SENT).all()), "the gather wrote into lower ranks' slices"
    assert bool((full[lo + S:] == SENT).all()), "the gather wrote into higher ranks' slices"
    del run, full, grad
    _release()


def _block_samples(S, B, n_blocks, seed):
    """Element indices of whole quantization blocks: the first, the last (ragged
    if S % B) and n_blocks random ones."""
    rng = np.random.default_rng(seed)
    nb = -(-S // B)
    blocks = np.unique(np.concatenate([[0, nb - 1], rng.integers(0, nb, n_blocks)]))
    return blocks, np.concatenate([np.arange(b * B, min((b + 1) * B, S)) for b in blocks]).astype(np.int64)


@pytest.mark.parametrize("bits,block", [(4, 256), (8, 64)])
def test_llama7b_shape_quantized_step_and_gather(zs, bits, block):
    """Fused step writing codes at the 7B shard (N=8), then the dequantizing
    gather of all ranks' payloads over the 6.7 G-element gathered buffer; whole
    blocks sampled (codes and scales bit-exact, decoded values bit-exact)."""
    import torch
    wl = synth.workloads()["llama7b"]
    if _free_gib() < 60:
        pytest.skip("needs ~50 GiB of free device memory")
    run = FlatBig(zs, wl, n_random=0)
    S, T = run.S, run.T
    blocks, idx = _block_samples(S, block, 400, 23)
    run.idx, run.didx = idx, torch.from_numpy(idx).cuda()
    gi = run.base + idx
    run.o_master = synth.cpu_at_f32(gi, wl.master_spec(run.valid_hi))
    K = idx.size
    run.o_m, run.o_v = np.zeros(K, np.float32), np.zeros(K, np.float32)
    run.o_g, run.o_p = np.zeros(K, np.uint16), np.zeros(K, np.uint16)
    hp = _hp(zs, wl)
    codes = torch.empty(zs.zs_quant_code_bytes(run.plan, bits), dtype=torch.uint8, device="cuda")
    scales = torch.empty(zs.zs_quant_num_scales(run.plan, block), dtype=torch.float32, device="cuda")
    for t in (1, 2):
        run.gen_contribs(t)
        zs.zs_fused_shard_step_quant(run.plan, hp.at(t), run.contribs, run.master, run.m, run.v, bits, block,
                                     codes, scales)
        run.oracle_step(t, hp)
    torch.cuda.synchronize()
    assert run.check_state("llama7b quant") == 0
    # oracle codes of each sampled block, from the oracle's parameters of the block
    o_codes, o_scales = [], []
    pos = 0
    for b in blocks:
        n = min(block, S - b * block)
        q, sc = oracle.quantize(run.o_p[pos:pos + n], bits, block)
        o_codes.append(q)
        o_scales.append(sc)
        pos += n
    g_scales = scales.index_select(0, torch.from_numpy(blocks).cuda()).cpu().numpy()
    assert np.array_equal(g_scales.view(np.uint32), np.concatenate(o_scales).view(np.uint32))
    byte_idx = np.concatenate([np.arange(b * block * bits // 8, (b * block + min(block, S - b * block)) * bits // 8)
                               for b in blocks])
    g_codes = codes.index_select(0, torch.from_numpy(byte_idx).cuda()).cpu().numpy()
    assert np.array_equal(g_codes, np.concatenate(o_codes)), "code bytes differ"
    # the gather: every rank's payload (copies of this rank's stand in for the others)
    for c in run.contribs:
        c.set_(torch.empty(0, dtype=torch.int16, device="cuda"))
    _release()
    full = torch.empty(T, dtype=torch.int16, device="cuda")
    zs.zs_dequant_gather(run.plan, bits, block, codes.repeat(wl.world), scales.repeat(wl.world), full)
    torch.cuda.synchronize()
    o_dec = np.concatenate([oracle.dequantize(q, sc, min(block, S - b * block), bits, block)
                            for q, sc, b in zip(o_codes, o_scales, blocks)])
    for r in (0, 3, wl.world - 1):
        got = full.index_select(0, torch.from_numpy(r * S + idx).cuda()).cpu().numpy().view(np.uint16)
        assert check_bf16(got, o_dec, f"gathered rank {r} slice") == 0
    del run, full, codes, scales
    _release()


def test_llama7b_shape_offloaded_step(zs):
    """The CPU-offloaded step at the 7B shard: pinned host state, chunked
    pipeline as the bench runs it; sampled host state and device parameters."""
    import torch
    wl = synth.workloads()["llama7b"]
    if _free_gib() < 40:
        pytest.skip("needs ~30 GiB of free device memory")
    run = FlatBig(zs, wl, n_random=100_000)
    S = run.S
    hp = _hp(zs, wl)
    hm = torch.empty(S, dtype=torch.float32, pin_memory=True)
    hm.copy_(run.master.cpu())
    hmm = torch.zeros(S, dtype=torch.float32, pin_memory=True)
    hv = torch.zeros(S, dtype=torch.float32, pin_memory=True)
    gh = torch.empty(S, dtype=torch.int16, pin_memory=True)
    ph = torch.empty(S, dtype=torch.int16, pin_memory=True)
    grad = torch.empty(S, dtype=torch.int16, device="cuda")
    full = torch.full((run.T,), SENT, dtype=torch.int16, device="cuda")
    for t in (1, 2):
        run.gen_contribs(t)
        zs.zs_reduce_shard(run.plan, run.contribs, grad)
        zs.zs_offload_adamw_step(run.plan, hp.at(t), grad, hm, hmm, hv, gh, ph, full_dev=full,
                                 chunk_elems=1 << 24, n_threads=16)
        run.oracle_step(t, hp)
    torch.cuda.synchronize()
    idx = torch.from_numpy(run.idx)
    nd = check_f32(hm.index_select(0, idx).numpy(), run.o_master, "host master")
    nd += check_f32(hmm.index_select(0, idx).numpy(), run.o_m, "host m")
    nd += check_f32(hv.index_select(0, idx).numpy(), run.o_v, "host v")
    nd += check_bf16(run.pick16(full), run.o_p, "gathered slice")
    assert nd == 0
    assert bool((full[S:S + 4096] == SENT).all())
    del run, full, grad, hm, hmm, hv, gh, ph
    _release()


def test_shard_beyond_2pow32_elements(zs):
    """The largest shard exercised: 4,295,032,832 owned elements (past 2^32)
    at N=2, rank 1, so the owned slice of the gathered buffer also starts past
    2^32; one tensor with 13 elements of tail padding. Every entry point runs
    on the same state: bucketed reduce (bucket edges at 2^31 + 8 and
    2^32 - 8), AdamW and gather at t=1; the fused step at t=2; one accumulated
    micro-step, the squared norm, the clip factor and the step from the
    accumulator at t=3; the quantized fused step (int4, B=256) at t=4 and the
    dequantizing gather of two payloads into the 8.6 G-element buffer.
    Samples are whole 256-element blocks: the first, the last, four on each
    side of 2^31 and 2^32, and 600 random ones."""
    import torch
    N, r, B = 2, 1, 256
    S = 2**32 + 65_536
    T = N * S
    numel = T - 13
    if _free_gib() < 125:
        pytest.skip("needs ~120 GiB of free device memory")
    plan = zs.zs_shard_plan([numel], N, r, 1, zs.ZS_LAYOUT_FLAT)
    assert (plan.shard_numel, plan.padded_numel) == (S, T)
    base = r * S
    seed = 0xB16
    master_sp = synth.spec(seed, synth.STREAM_MASTER, 0, 0.02, numel)

    def csp(q, t):
        return synth.spec(seed, synth.STREAM_CONTRIB + q, t, 1e-3, numel)

    nb = S // B
    special = [0, nb - 1]
    for e in (2**31, 2**32):
        special += list(range(e // B - 4, e // B + 4))
    blocks = np.unique(np.concatenate([special, np.random.default_rng(5).integers(0, nb, 600)])).astype(np.int64)
    idx = (blocks[:, None] * B + np.arange(B)[None, :]).ravel()
    didx = torch.from_numpy(idx).cuda()
    gi = base + idx
    print(f"[beyond 2^32] N={N} S={S:,} T={T:,} samples={idx.size:,}", flush=True)

    contribs = [torch.empty(S, dtype=torch.int16, device="cuda") for _ in range(N)]
    master = torch.empty(S, dtype=torch.float32, device="cuda")
    synth.gpu_f32(master, base, master_sp)
    m = torch.zeros(S, dtype=torch.float32, device="cuda")
    v = torch.zeros(S, dtype=torch.float32, device="cuda")
    grad = torch.empty(S, dtype=torch.int16, device="cuda")
    param = torch.empty(S, dtype=torch.int16, device="cuda")
    full = torch.empty(T, dtype=torch.int16, device="cuda")
    synth.gpu_fill_u16(full, SENT)
    K = idx.size
    o = dict(master=synth.cpu_at_f32(gi, master_sp), m=np.zeros(K, np.float32), v=np.zeros(K, np.float32),
             g=np.zeros(K, np.uint16), p=np.zeros(K, np.uint16))
    hp = zs.AdamWHParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)

    def ora_hp(t):
        return oracle.HParams(1e-3, 0.9, 0.95, 1e-8, 0.1, t)

    def gen(t):
        for q, c in enumerate(contribs):
            synth.gpu_bf16(c, base, csp(q, t))
        return [synth.cpu_at_bf16(gi, csp(q, t)) for q in range(N)]

    def pick16(x, at=didx):
        return x.index_select(0, at).cpu().numpy().view(np.uint16)

    def pick32(x):
        return x.index_select(0, didx).cpu().numpy()

    def check(tag, with_grad):
        torch.cuda.synchronize()
        nd = check_f32(pick32(master), o["master"], f"{tag} master") + check_f32(pick32(m), o["m"], f"{tag} m")
        nd += check_f32(pick32(v), o["v"], f"{tag} v") + check_bf16(pick16(param), o["p"], f"{tag} param")
        if with_grad:
            nd += check_bf16(pick16(grad), o["g"], f"{tag} grad")
        assert nd == 0, f"{tag}: {nd} sampled elements not bit-identical"

    own = torch.from_numpy(base + idx).cuda()
    other = torch.from_numpy(np.array([0, 2**31 - 1, 2**31, 2**32 - 1, 2**32, S - 1], np.int64)).cuda()

    # t=1: bucketed reduce, AdamW, gather
    cs = gen(1)
    edges = [0, 2**31 + 8, 2**32 - 8, S]
    for a, b in zip(edges[:-1], edges[1:]):
        zs.zs_reduce_shard(plan, contribs, grad, a, b - a)
    zs.zs_adamw_shard_step(plan, hp.at(1), grad, master, m, v, param)
    zs.zs_gather_params(plan, param, full)
    oracle.reduce(cs, out=o["g"])
    oracle.adamw(ora_hp(1), o["g"], o["master"], o["m"], o["v"], o["p"])
    check("t=1 bucketed", True)
    assert np.array_equal(pick16(full, own), o["p"])
    assert np.all(pick16(full, other) == SENT), "the gather wrote into rank 0's slice"
    assert np.all(o["p"][-13:] == 0) and np.all(o["master"][-13:] == 0)  # tail padding stays +0

    # t=2: fused step
    cs = gen(2)
    zs.zs_fused_shard_step(plan, hp.at(2), contribs, master, m, v, grad=grad, param=param, full=full)
    oracle.reduce(cs, out=o["g"])
    oracle.adamw(ora_hp(2), o["g"], o["master"], o["m"], o["v"], o["p"])
    check("t=2 fused", True)
    assert np.array_equal(pick16(full, own), o["p"])

    # t=3: one accumulated micro-step, norm, clip factor, step from the accumulator
    cs = gen(3)
    acc = torch.empty(S, dtype=torch.float32, device="cuda")
    ws = torch.zeros(zs.zs_grad_stats_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    flag = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    scale = torch.zeros(1, dtype=torch.float32, device="cuda")
    skip = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    max_norm = 10.0  # the gradient's norm is ~46: clipping is active
    zs.zs_accumulate_shard(plan, contribs, acc, first=True)
    zs.zs_grad_stats(plan, acc, 1.0, sumsq, flag, ws)
    zs.zs_clip_scale(sumsq, flag, max_norm, scale, skip)
    zs.zs_adamw_shard_step_accum(plan, hp.at(3), acc, 1.0, master, m, v, scale=scale, skip=skip, param=param,
                                 full=full)
    o_acc = np.zeros(K, np.float32)
    oracle.accumulate(cs, o_acc, first=True)
    torch.cuda.synchronize()
    assert check_f32(pick32(acc), o_acc, "t=3 acc") == 0
    assert int(flag.cpu()[0]) == 0 and int(skip.cpu()[0]) == 0
    got = float(sumsq.cpu()[0])
    ref = sum(float(acc[a:a + 2**28].double().square().sum()) for a in range(0, S, 2**28))
    assert abs(got - ref) <= 1e-12 * ref, (got, ref)
    sc = float(scale.cpu()[0])
    assert sc == oracle.clip_scale([got], max_norm) and 0.0 < sc < 1.0
    oracle.adamw_f32grad(ora_hp(3), o_acc, 1.0, sc, False, o["master"], o["m"], o["v"], o["p"])
    check("t=3 accumulated", False)
    assert np.array_equal(pick16(full, own), o["p"])
    del acc, ws
    _release()

    # t=4: quantized fused step, then the dequantizing gather of two payloads
    cs = gen(4)
    bits = 4
    codes = torch.empty(zs.zs_quant_code_bytes(plan, bits), dtype=torch.uint8, device="cuda")
    scales = torch.empty(zs.zs_quant_num_scales(plan, B), dtype=torch.float32, device="cuda")
    assert codes.numel() == S // 2 and scales.numel() == S // B
    zs.zs_fused_shard_step_quant(plan, hp.at(4), contribs, master, m, v, bits, B, codes, scales, grad=grad,
                                 param=param)
    oracle.reduce(cs, out=o["g"])
    oracle.adamw(ora_hp(4), o["g"], o["master"], o["m"], o["v"], o["p"])
    check("t=4 quantized", True)
    o_codes, o_scales, o_dec = [], [], []
    for k in range(blocks.size):
        q, s = oracle.quantize(o["p"][k * B:(k + 1) * B], bits, B)
        o_codes.append(q)
        o_scales.append(s)
        o_dec.append(oracle.dequantize(q, s, B, bits, B))
    g_scales = scales.index_select(0, torch.from_numpy(blocks).cuda()).cpu().numpy()
    assert np.array_equal(g_scales.view(np.uint32), np.concatenate(o_scales).view(np.uint32))
    byte_idx = (blocks[:, None] * (B // 2) + np.arange(B // 2)[None, :]).ravel()
    g_codes = codes.index_select(0, torch.from_numpy(byte_idx).cuda()).cpu().numpy()
    assert np.array_equal(g_codes, np.concatenate(o_codes)), "code bytes differ"
    for c in contribs:
        c.set_(torch.empty(0, dtype=torch.int16, device="cuda"))
    _release()
    zs.zs_dequant_gather(plan, bits, B, codes.repeat(N), scales.repeat(N), full)
    torch.cuda.synchronize()
    o_dec = np.concatenate(o_dec)
    for q in range(N):  # rank 0's payload is a copy of rank 1's
        got = pick16(full, torch.from_numpy(q * S + idx).cuda())
        assert check_bf16(got, o_dec, f"gathered slice of rank {q}") == 0
    del master, m, v, grad, param, full, codes, scales, contribs
    _release()


def test_multi_tensor_piece_beyond_2pow32(zs):
    """Multi-tensor apply with one piece of 4,295,032,832 owned elements (a
    tensor of 2^33 + 131,059 elements at N=2, rank 1, whose owned range of
    the gathered tensor also starts past 2^32) between two small pieces: the
    unfused calls (reduce, AdamW, gather) at t=1 and the fused call at t=2.
    The big piece is sampled in whole 256-element runs (first, last, both
    sides of 2^31 and 2^32, random); the small pieces are checked in full."""
    import torch
    N, r = 2, 1
    numels = [77, 2**33 + 131_059, 4096]
    if _free_gib() < 125:
        pytest.skip("needs ~110 GiB of free device memory")
    plan = zs.zs_shard_plan(numels, N, r, 1, zs.ZS_LAYOUT_PER_TENSOR)
    oplan = oracle.plan_per_tensor(numels, N, r, 0)
    sizes = [pc.own_hi - pc.own_lo for pc in oplan.pieces]
    assert sizes[1] == 2**32 + 65_536 and oplan.pieces[1].own_lo == sizes[1]
    seed = 0xB17
    valid = [oplan.offsets[i] + numels[i] for i in range(3)]

    def msp(i):
        return synth.spec(seed, synth.STREAM_MASTER, 0, 0.02, valid[i])

    def csp(i, q, t):
        return synth.spec(seed, synth.STREAM_CONTRIB + q, t, 1e-3, valid[i])

    S1 = sizes[1]
    nb = S1 // 256
    special = [0, nb - 1]
    for e in (2**31, 2**32):
        special += list(range(e // 256 - 4, e // 256 + 4))
    runs = np.unique(np.concatenate([special, np.random.default_rng(6).integers(0, nb, 400)])).astype(np.int64)
    samples = [np.arange(sizes[0]), (runs[:, None] * 256 + np.arange(256)[None, :]).ravel(), np.arange(sizes[2])]
    dsamples = [torch.from_numpy(x).cuda() for x in samples]
    bases = [pc.full_off for pc in oplan.pieces]  # packed global index of each piece's first owned element
    print(f"[multi beyond 2^32] pieces={sizes} samples={[x.size for x in samples]}", flush=True)

    pieces, o = [], []
    for i, Si in enumerate(sizes):
        d = dict(grad=torch.empty(Si, dtype=torch.int16, device="cuda"),
                 master=torch.empty(Si, dtype=torch.float32, device="cuda"),
                 m=torch.zeros(Si, dtype=torch.float32, device="cuda"),
                 v=torch.zeros(Si, dtype=torch.float32, device="cuda"),
                 param=torch.empty(Si, dtype=torch.int16, device="cuda"),
                 full=torch.empty(oplan.padded[i], dtype=torch.int16, device="cuda"))
        synth.gpu_f32(d["master"], bases[i], msp(i))
        synth.gpu_fill_u16(d["full"], SENT)
        pieces.append(d)
        K = samples[i].size
        o.append(dict(master=synth.cpu_at_f32(bases[i] + samples[i], msp(i)), m=np.zeros(K, np.float32),
                      v=np.zeros(K, np.float32), g=np.zeros(K, np.uint16), p=np.zeros(K, np.uint16)))
    contribs = [[torch.empty(Si, dtype=torch.int16, device="cuda") for Si in sizes] for _ in range(N)]
    ws = torch.zeros(zs.zs_multi_workspace_bytes(plan, N), dtype=torch.uint8, device="cuda")
    zs.zs_multi_bind(plan, pieces, contribs, ws)
    hp = zs.AdamWHParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)

    def step_oracle(t):
        for i in range(3):
            cs = [synth.cpu_at_bf16(bases[i] + samples[i], csp(i, q, t)) for q in range(N)]
            oracle.reduce(cs, out=o[i]["g"])
            oracle.adamw(oracle.HParams(1e-3, 0.9, 0.95, 1e-8, 0.1, t), o[i]["g"], o[i]["master"], o[i]["m"],
                         o[i]["v"], o[i]["p"])

    def check(tag):
        torch.cuda.synchronize()
        nd = 0
        for i, d in enumerate(pieces):
            at = dsamples[i]

            def pick(x):
                return x.index_select(0, at).cpu().numpy()

            nd += check_f32(pick(d["master"]), o[i]["master"], f"{tag} master[{i}]")
            nd += check_f32(pick(d["m"]), o[i]["m"], f"{tag} m[{i}]") + check_f32(pick(d["v"]), o[i]["v"],
                                                                                   f"{tag} v[{i}]")
            nd += check_bf16(pick(d["grad"]).view(np.uint16), o[i]["g"], f"{tag} grad[{i}]")
            nd += check_bf16(pick(d["param"]).view(np.uint16), o[i]["p"], f"{tag} param[{i}]")
            own = torch.from_numpy(oplan.pieces[i].own_lo + samples[i]).cuda()
            assert np.array_equal(d["full"].index_select(0, own).cpu().numpy().view(np.uint16), o[i]["p"])
            assert int(d["full"][0]) & 0xFFFF == SENT  # rank 0's range untouched
        assert nd == 0, f"{tag}: {nd} sampled elements not bit-identical"

    for t in (1, 2):
        for q in range(N):
            for i in range(3):
                synth.gpu_bf16(contribs[q][i], bases[i], csp(i, q, t))
        if t == 1:
            zs.zs_reduce_shard_multi(plan, ws)
            zs.zs_adamw_shard_step_multi(plan, hp.at(t), ws)
            zs.zs_gather_params_multi(plan, ws)
        else:
            zs.zs_fused_shard_step_multi(plan, hp.at(t), ws)
        step_oracle(t)
        check(f"t={t}")
    zs.zs_multi_unbind(ws)
    del pieces, contribs, ws
    _release()
