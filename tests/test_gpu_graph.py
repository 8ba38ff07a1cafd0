"""The per-step entry points captured in a HIP graph.

The step calls only enqueue kernels on the caller's stream: no allocation, no
host synchronization and no memset nodes. A caller can therefore capture a
whole step once and replay it as one graph launch per step (worthwhile for
launch-bound shards such as the 1M-element one here, whose kernels run for a
few microseconds). Kernel arguments are fixed at capture, so a captured step
keeps the hyperparameters (step t included) it was captured with; the _dc
calls read the AdamW scalars from device memory instead, so a step captured
once can take each replay's own.

Each test captures a step on one copy of the state, then replays it several
times. Before every replay new gradients are copied into the captured
contribution buffers (ordinary eager work), and after it the same calls run
eagerly on a second copy of the state. Every replay must leave bit-identical
state on both copies, and the final state must match the oracle to the usual
bar (with zero non-identical elements).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_bf16, check_f32, dev16, dev32, host16, host32

pytestmark = pytest.mark.gpu

SENT = 0x5A5A
REPLAYS = 3


@pytest.fixture(scope="module")
def zs():
    import torch

    import fsdp_sharded_mixed_flatten_amd as m
    torch.cuda.init()
    return m


def _same(a, b, what):
    import torch
    assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                       b.view(torch.int32) if b.dtype == torch.float32 else b), what


def _capture(fn):
    """Captures fn() (which enqueues on the current stream) into a graph,
    after one eager warm-up of the same calls on throwaway state."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def _ora_hp(hp):
    return oracle.HParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_flat_step_in_graph(zs, fused):
    import torch
    numels, N, r, valid, seed = [1_000_003], 4, 1, 1_000_003, 9101
    plan = zs.zs_shard_plan(numels, N, r, 1)
    T, S = plan.padded_numel, plan.shard_numel
    lo = r * S
    hp = zs.AdamWHParams(lr=1e-3, weight_decay=0.1, step=3)
    bucket = 65_536  # the unfused form reduces in buckets: several launches per step
    master0 = synth.cpu_f32(T, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02, valid))[lo:lo + S].copy()

    def grads(k):
        return [synth.cpu_bf16(T, 0, synth.spec(seed, synth.STREAM_CONTRIB + q, k, 1e-3, valid))[lo:lo + S].copy()
                for q in range(N)]

    def state():
        return dict(master=dev32(master0), m=torch.zeros(S, device="cuda"), v=torch.zeros(S, device="cuda"),
                    g=torch.zeros(S, dtype=torch.int16, device="cuda"),
                    p=torch.zeros(S, dtype=torch.int16, device="cuda"), full=dev16(np.full(T, SENT, np.uint16)))

    contribs = [torch.zeros(S, dtype=torch.int16, device="cuda") for _ in range(N)]

    def step(d):
        if fused:
            zs.zs_fused_shard_step(plan, hp, contribs, d["master"], d["m"], d["v"], grad=d["g"], param=d["p"],
                                   full=d["full"])
        else:
            for off in range(0, S, bucket):
                zs.zs_reduce_shard(plan, contribs, d["g"], off, min(bucket, S - off))
            zs.zs_adamw_shard_step(plan, hp, d["g"], d["master"], d["m"], d["v"], d["p"])
            zs.zs_gather_params(plan, d["p"], d["full"])

    warm = state()
    step(warm)
    torch.cuda.synchronize()
    A, B = state(), state()
    graph = _capture(lambda: step(A))
    o = dict(g=np.zeros(S, np.uint16), master=master0.copy(), m=np.zeros(S, np.float32),
             v=np.zeros(S, np.float32), p=np.zeros(S, np.uint16), full=np.full(T, SENT, np.uint16))
    for k in range(1, REPLAYS + 1):
        gk = grads(k)
        for q in range(N):
            contribs[q].copy_(dev16(gk[q]))
        torch.cuda.synchronize()
        graph.replay()
        step(B)
        torch.cuda.synchronize()
        for key in A:
            _same(A[key], B[key], f"replay {k}: {key}")
        oracle.shard_step(_ora_hp(hp), gk, o["g"], o["master"], o["m"], o["v"], o["p"], o["full"], r)
    nd = check_f32(host32(A["master"]), o["master"], "master") + check_f32(host32(A["m"]), o["m"], "m")
    nd += check_f32(host32(A["v"]), o["v"], "v") + check_bf16(host16(A["g"]), o["g"], "grad")
    nd += check_bf16(host16(A["p"]), o["p"], "param")
    assert np.array_equal(host16(A["full"]), o["full"])
    assert nd == 0


def test_accumulation_clip_step_in_graph(zs):
    """G micro-steps of accumulation, the squared norm, the clip factor and the
    step from the accumulator: the whole sequence keeps its decisions on the
    device, so it captures as one graph."""
    import torch
    numels, N, r, valid, seed, G, max_norm = [1_000_003], 4, 2, 1_000_003, 5150, 2, 1e-4
    plan = zs.zs_shard_plan(numels, N, r, 1)
    T, S = plan.padded_numel, plan.shard_numel
    lo = r * S
    hp = zs.AdamWHParams(lr=1e-3, weight_decay=0.1, step=2)
    master0 = synth.cpu_f32(T, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02, valid))[lo:lo + S].copy()

    def grads(k, micro):
        return [synth.cpu_bf16(T, 0, synth.spec(seed, synth.STREAM_CONTRIB + q, 16 * k + micro, 1e-3,
                                                valid))[lo:lo + S].copy() for q in range(N)]

    contribs = [[torch.zeros(S, dtype=torch.int16, device="cuda") for _ in range(N)] for _ in range(G)]
    ws_bytes = zs.zs_grad_stats_workspace_bytes(plan)

    def state():
        return dict(acc=torch.zeros(S, device="cuda"), sumsq=torch.zeros(1, dtype=torch.float64, device="cuda"),
                    flag=torch.zeros(1, dtype=torch.int32, device="cuda"), scale=torch.zeros(1, device="cuda"),
                    skip=torch.zeros(1, dtype=torch.int32, device="cuda"), master=dev32(master0),
                    m=torch.zeros(S, device="cuda"), v=torch.zeros(S, device="cuda"),
                    p=torch.zeros(S, dtype=torch.int16, device="cuda"), full=dev16(np.full(T, SENT, np.uint16)),
                    ws=torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda"))

    def step(d):
        for k in range(G):
            zs.zs_accumulate_shard(plan, contribs[k], d["acc"], first=(k == 0))
        zs.zs_grad_stats(plan, d["acc"], float(G), d["sumsq"], d["flag"], d["ws"])
        zs.zs_clip_scale(d["sumsq"], d["flag"], max_norm, d["scale"], d["skip"])
        zs.zs_adamw_shard_step_accum(plan, hp, d["acc"], float(G), d["master"], d["m"], d["v"], scale=d["scale"],
                                     skip=d["skip"], param=d["p"], full=d["full"])

    warm = state()
    step(warm)
    torch.cuda.synchronize()
    A, B = state(), state()
    graph = _capture(lambda: step(A))
    om, ov, op = np.zeros(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.uint16)
    omaster = master0.copy()
    for k in range(1, REPLAYS + 1):
        gk = [grads(k, micro) for micro in range(G)]
        for micro in range(G):
            for q in range(N):
                contribs[micro][q].copy_(dev16(gk[micro][q]))
        torch.cuda.synchronize()
        graph.replay()
        step(B)
        torch.cuda.synchronize()
        for key in A:
            if key != "ws":
                _same(A[key], B[key], f"replay {k}: {key}")
        o_acc = np.zeros(S, np.float32)
        for micro in range(G):
            oracle.accumulate(gk[micro], o_acc, first=(micro == 0))
        s, f = oracle.grad_sumsq(o_acc, float(G))
        assert f == 0 and int(A["flag"].cpu()[0]) == 0 and int(A["skip"].cpu()[0]) == 0
        got = float(A["sumsq"].cpu()[0])
        assert abs(got - s) <= 1e-12 * s
        scale = float(A["scale"].cpu()[0])
        assert scale == oracle.clip_scale([got], max_norm) and scale < 1.0
        assert check_f32(host32(A["acc"]), o_acc, f"acc, replay {k}") == 0
        oracle.adamw_f32grad(_ora_hp(hp), o_acc, float(G), scale, False, omaster, om, ov, op)
    nd = check_f32(host32(A["master"]), omaster, "master") + check_f32(host32(A["m"]), om, "m")
    nd += check_f32(host32(A["v"]), ov, "v") + check_bf16(host16(A["p"]), op, "param")
    full_o = np.full(T, SENT, np.uint16)
    full_o[lo:lo + S] = op
    assert np.array_equal(host16(A["full"]), full_o)
    assert nd == 0


def test_multi_tensor_step_in_graph(zs):
    """The multi-tensor fused step: the table is bound once, outside the
    capture (binding copies and synchronizes), and the captured launch reads
    it on every replay."""
    import torch
    numels, N, r, seed = [4096 * 3, 512, 1000, 77, 8, 70_000], 4, 2, 31337
    hp = zs.AdamWHParams(lr=1e-3, weight_decay=0.1, step=1)
    plan = zs.zs_shard_plan(numels, N, r, 1, zs.ZS_LAYOUT_PER_TENSOR)
    oplan = oracle.plan_per_tensor(numels, N, r, 0)
    sizes = [pc.own_hi - pc.own_lo for pc in oplan.pieces]
    masters = [synth.cpu_f32(Si, pc.full_off, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02,
                                                         oplan.offsets[i] + numels[i]))
               for i, (Si, pc) in enumerate(zip(sizes, oplan.pieces))]

    def grads(k):
        return [[synth.cpu_bf16(Si, pc.full_off, synth.spec(seed, synth.STREAM_CONTRIB + q, k, 1e-3,
                                                            oplan.offsets[i] + numels[i]))
                 for i, (Si, pc) in enumerate(zip(sizes, oplan.pieces))] for q in range(N)]

    contribs = [[torch.zeros(Si, dtype=torch.int16, device="cuda") for Si in sizes] for _ in range(N)]

    def pieces():
        return [dict(grad=torch.zeros(Si, dtype=torch.int16, device="cuda"), master=dev32(masters[i]),
                     m=torch.zeros(Si, device="cuda"), v=torch.zeros(Si, device="cuda"),
                     param=torch.zeros(Si, dtype=torch.int16, device="cuda"),
                     full=dev16(np.full(oplan.padded[i], SENT, np.uint16))) for i, Si in enumerate(sizes)]

    nbytes = zs.zs_multi_workspace_bytes(plan, N)
    bound = []
    for _ in range(3):  # warm-up, graph, eager
        p = pieces()
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        zs.zs_multi_bind(plan, p, contribs, ws)
        bound.append((p, ws))
    zs.zs_fused_shard_step_multi(plan, hp, bound[0][1])
    torch.cuda.synchronize()
    (A, wsA), (B, wsB) = bound[1], bound[2]
    graph = _capture(lambda: zs.zs_fused_shard_step_multi(plan, hp, wsA))
    o = [dict(g=np.zeros(Si, np.uint16), master=masters[i].copy(), m=np.zeros(Si, np.float32),
              v=np.zeros(Si, np.float32), p=np.zeros(Si, np.uint16)) for i, Si in enumerate(sizes)]
    for k in range(1, REPLAYS + 1):
        gk = grads(k)
        for q in range(N):
            for i in range(len(sizes)):
                contribs[q][i].copy_(dev16(gk[q][i]))
        torch.cuda.synchronize()
        graph.replay()
        zs.zs_fused_shard_step_multi(plan, hp, wsB)
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            for key in A[i]:
                _same(A[i][key], B[i][key], f"replay {k}: piece {i} {key}")
            oi = o[i]
            oracle.reduce([gk[q][i] for q in range(N)], out=oi["g"])
            oracle.adamw(_ora_hp(hp), oi["g"], oi["master"], oi["m"], oi["v"], oi["p"])
    nd = 0
    for i, (oi, d) in enumerate(zip(o, A)):
        nd += check_bf16(host16(d["grad"]), oi["g"], f"grad[{i}]") + check_bf16(host16(d["param"]), oi["p"],
                                                                                  f"param[{i}]")
        nd += check_f32(host32(d["master"]), oi["master"], f"master[{i}]")
        nd += check_f32(host32(d["m"]), oi["m"], f"m[{i}]") + check_f32(host32(d["v"]), oi["v"], f"v[{i}]")
        full_o = np.full(oplan.padded[i], SENT, np.uint16)
        full_o[oplan.pieces[i].own_lo:oplan.pieces[i].own_hi] = oi["p"]
        assert np.array_equal(host16(d["full"]), full_o), f"full[{i}]"
    assert nd == 0


def _dev_coefs(zs, hps):
    import torch
    vals = [x for hp in hps for x in zs.zs_adamw_coefs_compute(hp).values()]
    return torch.tensor(vals, dtype=torch.float32, device="cuda")


def test_device_scalar_calls_equal_by_value(zs):
    """The _dc calls (AdamW scalars read from device memory) leave the same
    bytes as the by-value calls: fused step (one- and two-pass), AdamW, the
    step from the accumulator and the multi-tensor step with two groups."""
    import torch
    hp = zs.AdamWHParams(lr=2e-3, beta1=0.9, beta2=0.99, eps=1e-7, weight_decay=0.05, step=7)
    for N in (4, 64):
        numels = [30_011, 77]
        plan = zs.zs_shard_plan(numels, N, N - 1, 1)
        T, S = plan.padded_numel, plan.shard_numel
        rng = np.random.default_rng(N)
        cs = [dev16(oracle.f32_to_bf16((rng.standard_normal(S) * 1e-3).astype(np.float32))) for _ in range(N)]
        master0 = (rng.standard_normal(S) * 0.02).astype(np.float32)

        def state():
            return dict(master=dev32(master0), m=torch.zeros(S, device="cuda"), v=torch.zeros(S, device="cuda"),
                        g=torch.zeros(S, dtype=torch.int16, device="cuda"),
                        p=torch.zeros(S, dtype=torch.int16, device="cuda"),
                        full=dev16(np.full(T, SENT, np.uint16)), acc=dev32(master0 * 1e-2))

        a, b = state(), state()
        coefs = _dev_coefs(zs, [hp])
        zs.zs_fused_shard_step(plan, hp, cs, a["master"], a["m"], a["v"], grad=a["g"], param=a["p"], full=a["full"])
        zs.zs_fused_shard_step_dc(plan, coefs, cs, b["master"], b["m"], b["v"], grad=b["g"], param=b["p"],
                                  full=b["full"])
        zs.zs_adamw_shard_step(plan, hp.at(8), a["g"], a["master"], a["m"], a["v"], a["p"])
        coefs8 = _dev_coefs(zs, [hp.at(8)])
        zs.zs_adamw_shard_step_dc(plan, coefs8, b["g"], b["master"], b["m"], b["v"], b["p"])
        zs.zs_adamw_shard_step_accum(plan, hp.at(9), a["acc"], 3.0, a["master"], a["m"], a["v"], param=a["p"],
                                     full=a["full"])
        zs.zs_adamw_shard_step_accum_dc(plan, _dev_coefs(zs, [hp.at(9)]), b["acc"], 3.0, b["master"], b["m"],
                                        b["v"], param=b["p"], full=b["full"])
        torch.cuda.synchronize()
        for k in a:
            _same(a[k], b[k], f"N={N}: {k}")
    # multi-tensor with two hyperparameter groups
    numels, N, r = [4096 * 3, 512, 1000, 77], 4, 2
    plan = zs.zs_shard_plan_ex(numels, N, r, groups=[0, 1, 0, 1])
    oplan = oracle.plan_per_tensor(numels, N, r, 0)
    sizes = [pc.own_hi - pc.own_lo for pc in oplan.pieces]
    rng = np.random.default_rng(5)
    host = [dict(master=(rng.standard_normal(Si) * 0.02).astype(np.float32)) for Si in sizes]
    contribs = [[dev16(oracle.f32_to_bf16((rng.standard_normal(Si) * 1e-3).astype(np.float32))) for Si in sizes]
                for _ in range(N)]

    def pieces():
        return [dict(grad=torch.zeros(Si, dtype=torch.int16, device="cuda"), master=dev32(host[i]["master"]),
                     m=torch.zeros(Si, device="cuda"), v=torch.zeros(Si, device="cuda"),
                     param=torch.zeros(Si, dtype=torch.int16, device="cuda"),
                     full=dev16(np.full(oplan.padded[i], SENT, np.uint16))) for i, Si in enumerate(sizes)]

    pa, pb = pieces(), pieces()
    wsa = torch.zeros(zs.zs_multi_workspace_bytes(plan, N), dtype=torch.uint8, device="cuda")
    wsb = torch.zeros_like(wsa)
    zs.zs_multi_bind(plan, pa, contribs, wsa)
    zs.zs_multi_bind(plan, pb, contribs, wsb)
    hps = [hp, zs.AdamWHParams(lr=1e-3, weight_decay=0.0, step=7)]
    zs.zs_fused_shard_step_multi_groups(plan, hps, wsa)
    zs.zs_fused_shard_step_multi_dc(plan, _dev_coefs(zs, hps), 2, wsb)
    torch.cuda.synchronize()
    for i in range(len(sizes)):
        for k in pa[i]:
            _same(pa[i][k], pb[i][k], f"piece {i}: {k}")


def test_graph_replays_with_new_scalars(zs):
    """A training loop on a captured graph: captured once are a copy of the
    AdamW scalars from page-locked host memory into a device buffer and the
    fused step that reads them; before each replay the host writes the next
    step's scalars (t = 1, 2, 3, 4 and a learning-rate change) and new
    gradients. Every replay equals the eager by-value step with those
    hyperparameters, and the end state equals the oracle's."""
    import torch
    numels, N, r, valid, seed = [1_000_003], 4, 1, 1_000_003, 2718
    plan = zs.zs_shard_plan(numels, N, r, 1)
    T, S = plan.padded_numel, plan.shard_numel
    lo = r * S
    master0 = synth.cpu_f32(T, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02, valid))[lo:lo + S].copy()

    def grads(k):
        return [synth.cpu_bf16(T, 0, synth.spec(seed, synth.STREAM_CONTRIB + q, k, 1e-3, valid))[lo:lo + S].copy()
                for q in range(N)]

    def state():
        return dict(master=dev32(master0), m=torch.zeros(S, device="cuda"), v=torch.zeros(S, device="cuda"),
                    p=torch.zeros(S, dtype=torch.int16, device="cuda"), full=dev16(np.full(T, SENT, np.uint16)))

    contribs = [torch.zeros(S, dtype=torch.int16, device="cuda") for _ in range(N)]
    host_coefs = torch.zeros(9, dtype=torch.float32, pin_memory=True)
    dev_coefs = torch.zeros(9, dtype=torch.float32, device="cuda")
    A, B = state(), state()

    def step_dc(d):
        dev_coefs.copy_(host_coefs, non_blocking=True)
        zs.zs_fused_shard_step_dc(plan, dev_coefs, contribs, d["master"], d["m"], d["v"], param=d["p"],
                                  full=d["full"])

    warm = state()
    host_coefs.copy_(torch.tensor(zs.zs_adamw_coefs_compute(zs.AdamWHParams()).values()))
    step_dc(warm)
    torch.cuda.synchronize()
    graph = _capture(lambda: step_dc(A))
    o = dict(g=np.zeros(S, np.uint16), master=master0.copy(), m=np.zeros(S, np.float32), v=np.zeros(S, np.float32),
             p=np.zeros(S, np.uint16), full=np.full(T, SENT, np.uint16))
    schedule = [(1, 1e-3), (2, 1e-3), (3, 5e-4), (4, 2.5e-4)]
    for k, (t, lr) in enumerate(schedule, start=1):
        hp = zs.AdamWHParams(lr=lr, weight_decay=0.1, step=t)
        gk = grads(k)
        for q in range(N):
            contribs[q].copy_(dev16(gk[q]))
        host_coefs.copy_(torch.tensor(zs.zs_adamw_coefs_compute(hp).values()))
        torch.cuda.synchronize()
        graph.replay()
        zs.zs_fused_shard_step(plan, hp, contribs, B["master"], B["m"], B["v"], param=B["p"], full=B["full"])
        torch.cuda.synchronize()
        for key in A:
            _same(A[key], B[key], f"replay {k}: {key}")
        oracle.shard_step(oracle.HParams(lr, 0.9, 0.95, 1e-8, 0.1, t), gk, o["g"], o["master"], o["m"], o["v"],
                          o["p"], o["full"], r)
    nd = check_f32(host32(A["master"]), o["master"], "master") + check_f32(host32(A["m"]), o["m"], "m")
    nd += check_f32(host32(A["v"]), o["v"], "v") + check_bf16(host16(A["p"]), o["p"], "param")
    assert np.array_equal(host16(A["full"]), o["full"])
    assert nd == 0


def test_quantized_step_and_gather_in_graph(zs):
    """The quantized parameter gather captured whole: the fused step writes
    this rank's codes and scales straight into its slot of the all-ranks
    payload, and the dequantizing gather decodes every rank's slot into the
    gathered buffer. Before each replay the other ranks' payloads change (as
    a new all-gather would deliver them) together with the gradients."""
    import torch
    bits, B = 4, 64
    numels, N, r, seed = [1_048_573], 4, 2, 9404
    plan = zs.zs_shard_plan(numels, N, r, 1)
    T, S = plan.padded_numel, plan.shard_numel
    cb, nb = zs.zs_quant_code_bytes(plan, bits), zs.zs_quant_num_scales(plan, B)
    assert cb % 16 == 0 and (nb * 4) % 16 == 0  # every rank's slot starts 16-byte aligned
    lo = r * S
    hp = zs.AdamWHParams(lr=1e-3, weight_decay=0.1, step=2)
    master0 = synth.cpu_f32(T, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02, sum(numels)))[lo:lo + S].copy()
    rng = np.random.default_rng(seed)

    def grads(k):
        return [synth.cpu_bf16(T, 0, synth.spec(seed, synth.STREAM_CONTRIB + q, k, 1e-3, sum(numels)))[lo:lo + S]
                .copy() for q in range(N)]

    def state():
        return dict(master=dev32(master0), m=torch.zeros(S, device="cuda"), v=torch.zeros(S, device="cuda"),
                    g=torch.zeros(S, dtype=torch.int16, device="cuda"),
                    p=torch.zeros(S, dtype=torch.int16, device="cuda"),
                    codes=torch.zeros(N * cb, dtype=torch.uint8, device="cuda"),
                    scales=torch.zeros(N * nb, dtype=torch.float32, device="cuda"),
                    full=dev16(np.full(T, SENT, np.uint16)))

    contribs = [torch.zeros(S, dtype=torch.int16, device="cuda") for _ in range(N)]

    def step(d):
        zs.zs_fused_shard_step_quant(plan, hp, contribs, d["master"], d["m"], d["v"], bits, B,
                                     d["codes"][r * cb:(r + 1) * cb], d["scales"][r * nb:(r + 1) * nb],
                                     grad=d["g"], param=d["p"])
        zs.zs_dequant_gather(plan, bits, B, d["codes"], d["scales"], d["full"])

    warm = state()
    step(warm)
    torch.cuda.synchronize()
    A, Bst = state(), state()
    graph = _capture(lambda: step(A))
    o = dict(g=np.zeros(S, np.uint16), master=master0.copy(), m=np.zeros(S, np.float32),
             v=np.zeros(S, np.float32), p=np.zeros(S, np.uint16))
    for k in range(1, REPLAYS + 1):
        gk = grads(k)
        for q in range(N):
            contribs[q].copy_(dev16(gk[q]))
        codes_all = rng.integers(0, 256, N * cb, dtype=np.uint8)
        scales_all = (rng.random(N * nb) * 1e-2).astype(np.float32)
        for d in (A, Bst):  # the other ranks' slots; this rank's is rewritten by the step
            d["codes"].copy_(torch.from_numpy(codes_all).cuda())
            d["scales"].copy_(torch.from_numpy(scales_all).cuda())
        torch.cuda.synchronize()
        graph.replay()
        step(Bst)
        torch.cuda.synchronize()
        for key in A:
            _same(A[key], Bst[key], f"replay {k}: {key}")
        oracle.shard_step(_ora_hp(hp), gk, o["g"], o["master"], o["m"], o["v"], o["p"], None, r)
        q_own, s_own = oracle.quantize(o["p"], bits, B)
        codes_all[r * cb:(r + 1) * cb] = q_own
        scales_all[r * nb:(r + 1) * nb] = s_own
        ref_full = oracle.dequant_gather(codes_all, scales_all, S, N, bits, B)
        assert np.array_equal(A["codes"].cpu().numpy(), codes_all), f"replay {k}: codes"
        assert np.array_equal(A["scales"].cpu().numpy().view(np.uint32), scales_all.view(np.uint32)), \
            f"replay {k}: scales"
        assert check_bf16(host16(A["full"]), ref_full, f"replay {k}: full") == 0
    nd = check_f32(host32(A["master"]), o["master"], "master") + check_f32(host32(A["m"]), o["m"], "m")
    nd += check_f32(host32(A["v"]), o["v"], "v") + check_bf16(host16(A["g"]), o["g"], "grad")
    nd += check_bf16(host16(A["p"]), o["p"], "param")
    assert nd == 0
