"""GPU <-> oracle parity of the quantized parameter gather.

Codes are integers decided by one fp32 division on both sides, so codes must
be bit-identical and scales bit-identical (NaN where the oracle has NaN); the
dequantized bf16 values too (NaN positions only for NaN). The fused step's
fp32 state and bf16 outputs use the tolerances of the other parity tests and
are required bit-identical as well.
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


def _hp(zs, **kw):
    base = dict(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
    base.update(kw)
    return zs.AdamWHParams(**base)


def _u8(n):
    import torch
    return torch.full((max(n, 1),), 0xEE, dtype=torch.uint8, device="cuda")


def _f32(n):
    import torch
    return torch.full((max(n, 1),), -7.0, dtype=torch.float32, device="cuda")


def _host8(t):
    return t.detach().cpu().numpy().view(np.uint8)


def _same_scales(gpu, ora, what):
    g, o = gpu.view(np.uint32), ora.view(np.uint32)
    nan_o, nan_g = np.isnan(ora), np.isnan(gpu)
    assert np.array_equal(nan_o, nan_g), f"{what}: NaN positions differ"
    assert np.array_equal(g[~nan_o], o[~nan_o]), f"{what}: {(g[~nan_o] != o[~nan_o]).sum()} scales differ"


def _special_shard(S, seed):
    """bf16 shard with Gaussian values, a heavy tail, an all-zero block, a
    block holding an infinity, one holding a NaN, subnormals and exact ties."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(S) * 0.02).astype(np.float32)
    x[rng.random(S) < 0.002] *= 100.0
    p = oracle.f32_to_bf16(x)
    if S >= 1024:
        p[256:512] = 0
        p[600] = 0x7F80  # +inf
        p[700] = 0xFFC1  # NaN
        p[800:808] = np.array([0x0001, 0x8003, 0x0040, 0x807F, 0, 0x8000, 0x0002, 0x0010], np.uint16)  # subnormals
        p[896:904] = oracle.f32_to_bf16(np.array([7, -7, 2.5, -2.5, 3.5, 0.5, 1.5, -3.5], np.float32))
    return p


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("block", [8, 32, 128, 256])
def test_quantize_shard(zs, bits, block):
    world, rank = 4, 2
    numels = [200_003, 1_000, 37]
    plan = zs.zs_shard_plan(numels, world, rank, 1)
    S = plan.shard_numel
    assert S % block != 0 or block == 8  # a ragged last block
    p = _special_shard(S, bits * 1000 + block)
    codes, scales = _u8(zs.zs_quant_code_bytes(plan, bits) + 64), _f32(zs.zs_quant_num_scales(plan, block) + 16)
    zs.zs_quantize_shard(plan, bits, block, dev16(p), codes, scales)
    oq, osc = oracle.quantize(p, bits, block)
    gq, gs = _host8(codes), host32(scales)
    assert np.array_equal(gq[:oq.size], oq), f"{(gq[:oq.size] != oq).sum()} code bytes differ"
    assert np.all(gq[oq.size:] == 0xEE), "codes written past the payload"
    _same_scales(gs[:osc.size], osc, "scales")
    assert np.all(gs[osc.size:] == -7.0), "scales written past the payload"


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("world,block", [(4, 64), (8, 256), (3, 16), (5, 128)])
def test_dequant_gather(zs, bits, world, block):
    import torch
    plan = zs.zs_shard_plan([123_457, 999], world, 0, 1)
    S = plan.shard_numel
    qs, ss = [], []
    for r in range(world):
        q, sc = oracle.quantize(_special_shard(S, 50 + r), bits, block)
        qs.append(q)
        ss.append(sc)
    codes_all, scales_all = np.concatenate(qs), np.concatenate(ss)
    full = torch.full((world * S + 64,), 0x5A5A, dtype=torch.int16, device="cuda")
    zs.zs_dequant_gather(plan, bits, block, torch.from_numpy(codes_all).cuda(), dev32(scales_all), full)
    ref = oracle.dequant_gather(codes_all, scales_all, S, world, bits, block)
    got = host16(full)
    nd = check_bf16(got[:world * S], ref, "gathered")
    assert nd == 0
    assert np.all(got[world * S:] == 0x5A5A)


@pytest.mark.parametrize("bits,block,S", [(4, 256, 15_560), (4, 128, 24_896), (4, 8, 1_000), (4, 16, 4_160),
                                          (8, 256, 15_560), (8, 64, 24_896), (8, 32, 1_000)])
def test_dequant_gather_arbitrary_payload(zs, bits, block, S):
    """Payloads no quantizer writes: every code value (the 4-bit -8 and the
    8-bit -128 included) under scales that are random, zero, negative, tiny
    (products round to bf16 subnormals), huge (products overflow to
    infinity), infinite and NaN of either sign. Shard lengths with and without
    16-byte-aligned per-rank code payloads (S a multiple of 32 at int4, of 16
    at int8), the two ways the kernel loads codes, each with a last block of
    the launch cut short."""
    import torch
    world = 3
    plan = zs.zs_shard_plan([world * S], world, 0, 1)
    assert plan.shard_numel == S
    rng = np.random.default_rng(block + S)
    nq = zs.zs_quant_code_bytes(plan, bits)
    ns = zs.zs_quant_num_scales(plan, block)
    assert (nq % 16 == 0) == (S % (128 // bits) == 0)
    codes_all = rng.integers(0, 256, world * nq, dtype=np.uint8)
    sc = (rng.standard_normal(world * ns) * 1e-3).astype(np.float32)
    special = np.array([0.0, -0.0, -1e-3, 1e-40, 2e-38, 3.0e38, -3.0e38, np.inf, -np.inf], np.float32)
    sc[:special.size] = special
    sc[special.size] = np.float32(np.nan)
    sc[special.size + 1] = np.frombuffer(np.uint32(0xFFC00001).tobytes(), np.float32)[0]  # negative NaN
    rng.shuffle(sc[:4 * special.size])
    full = torch.full((world * S + 64,), 0x5A5A, dtype=torch.int16, device="cuda")
    zs.zs_dequant_gather(plan, bits, block, torch.from_numpy(codes_all).cuda(), dev32(sc), full)
    ref = oracle.dequant_gather(codes_all, sc, S, world, bits, block)
    got = host16(full)
    assert check_bf16(got[:world * S], ref, "gathered") == 0
    assert np.all(got[world * S:] == 0x5A5A)


class QuantRun:
    """FLAT rank with the quantized fused step, several steps, against the oracle."""

    def __init__(self, zs, numels, world, rank, bits, block, steps, seed, replicas=1):
        import torch
        self.zs, self.bits, self.block = zs, bits, block
        self.plan = zs.zs_shard_plan(numels, world, rank, 1)
        T, S = self.plan.padded_numel, self.plan.shard_numel
        self.S, self.rank = S, rank
        real = sum(numels)
        lo = rank * S
        master = synth.cpu_f32(T, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02, real))[lo:lo + S].copy()
        self.mine = {t: [synth.cpu_bf16(T, 0, synth.spec(seed, synth.STREAM_CONTRIB + q, t, 1e-3, real))[lo:lo + S]
                         .copy() for q in range(world * replicas)] for t in range(1, steps + 1)}
        self.o = dict(g=np.zeros(S, np.uint16), master=master, m=np.zeros(S, np.float32),
                      v=np.zeros(S, np.float32), p=np.zeros(S, np.uint16))
        self.d = dict(g=dev16(np.zeros(S, np.uint16)), master=dev32(master), m=dev32(np.zeros(S, np.float32)),
                      v=dev32(np.zeros(S, np.float32)), p=dev16(np.zeros(S, np.uint16)))
        self.codes = _u8(zs.zs_quant_code_bytes(self.plan, bits))
        self.scales = _f32(zs.zs_quant_num_scales(self.plan, block))
        self.dc = {t: [dev16(c) for c in cs] for t, cs in self.mine.items()}
        torch.cuda.synchronize()

    def step(self, t, hp):
        zs, d, o = self.zs, self.d, self.o
        h = hp.at(t)
        zs.zs_fused_shard_step_quant(self.plan, h, self.dc[t], d["master"], d["m"], d["v"], self.bits, self.block,
                                     self.codes, self.scales, grad=d["g"], param=d["p"])
        oracle.shard_step(oracle.HParams(h.lr, h.beta1, h.beta2, h.eps, h.weight_decay, t), self.mine[t], o["g"],
                          o["master"], o["m"], o["v"], o["p"], None, self.rank)

    def check(self):
        o, d = self.o, self.d
        nd = check_bf16(host16(d["g"]), o["g"], "grad") + check_bf16(host16(d["p"]), o["p"], "param")
        for k in ("master", "m", "v"):
            nd += check_f32(host32(d[k]), o[k], k)
        assert nd == 0
        oq, osc = oracle.quantize(o["p"], self.bits, self.block)
        gq = _host8(self.codes)[:oq.size]
        assert np.array_equal(gq, oq), f"{(gq != oq).sum()} code bytes differ"
        _same_scales(host32(self.scales)[:osc.size], osc, "scales")


@pytest.mark.parametrize("bits,block,world,replicas", [(4, 256, 4, 1), (8, 64, 8, 1), (4, 32, 8, 8), (8, 256, 5, 1)])
def test_fused_step_quant(zs, bits, block, world, replicas):
    """reduce + AdamW + codes of the updated shard in one pass (8x8 = 64
    contributions takes the two-pass path: reduce, then AdamW + codes)."""
    run = QuantRun(zs, [300_007, 4_099], world, world - 1, bits, block, 2, 61 + bits, replicas)
    for t in (1, 2):
        run.step(t, _hp(zs))
        run.check()


def test_fused_quant_equals_quantize_of_param(zs):
    import torch
    run = QuantRun(zs, [65_536 * 3 + 40], 4, 1, 4, 128, 1, 5)
    run.step(1, _hp(zs))
    codes2, scales2 = _u8(run.codes.numel()), _f32(run.scales.numel())
    zs.zs_quantize_shard(run.plan, 4, 128, run.d["p"], codes2, scales2)
    torch.cuda.synchronize()
    assert torch.equal(codes2, run.codes)
    assert np.array_equal(host32(scales2).view(np.uint32), host32(run.scales).view(np.uint32))


def test_quant_round_trip_through_gather(zs):
    """Every rank's fused quantized step, then the gather of all payloads:
    the gathered buffer equals the dequantized oracle parameters."""
    import torch
    world, bits, block = 4, 8, 128
    numels = [77_777, 513]
    runs = [QuantRun(zs, numels, world, r, bits, block, 1, 9) for r in range(world)]
    for r in runs:
        r.step(1, _hp(zs))
    S = runs[0].S
    codes_all = torch.cat([r.codes[:zs.zs_quant_code_bytes(r.plan, bits)] for r in runs])
    scales_all = torch.cat([r.scales[:zs.zs_quant_num_scales(r.plan, block)] for r in runs])
    full = torch.zeros(world * S, dtype=torch.int16, device="cuda")
    zs.zs_dequant_gather(runs[0].plan, bits, block, codes_all, scales_all, full)
    ref = np.concatenate([oracle.dequantize(*oracle.quantize(r.o["p"], bits, block), S, bits, block) for r in runs])
    assert check_bf16(host16(full), ref, "gathered") == 0
    # every real element is within half a grid step of its exact bf16 parameter
    exact = oracle.bf16_to_f32(np.concatenate([r.o["p"] for r in runs])).astype(np.float64)
    got = oracle.bf16_to_f32(host16(full)).astype(np.float64)
    sc = np.concatenate([np.repeat(host32(r.scales)[:zs.zs_quant_num_scales(r.plan, block)], block)[:S]
                         for r in runs]).astype(np.float64)
    assert np.all(np.abs(got - exact) <= sc * 0.5 * (1 + 2.0**-20) + np.abs(got) * 2.0**-8)


def test_quant_errors(zs):
    import torch
    plan = zs.zs_shard_plan([4096], 4, 0)
    p = torch.zeros(1024, dtype=torch.int16, device="cuda")
    codes, scales = _u8(1024), _f32(1024)
    for bits, block in ((2, 64), (8, 4), (8, 512), (4, 48)):
        with pytest.raises(zs.ZsError):
            zs.zs_quantize_shard(plan, bits, block, p, codes, scales)
    pt = zs.zs_shard_plan([4096], 4, 0, 1, zs.ZS_LAYOUT_PER_TENSOR)
    with pytest.raises(zs.ZsError):
        zs.zs_quantize_shard(pt, 8, 64, p, codes, scales)
    torch.cuda.synchronize()
