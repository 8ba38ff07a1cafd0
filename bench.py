"""Benchmark of one rank's shard-local step (reduce + mixed-precision AdamW +
gather) on one MI355X.

A step is one pass of the whole path over the owned shard: the average of the
N bf16 gradient contributions, AdamW on the fp32 master/m/v state, and the
bf16 parameter write into the gathered buffer. Inputs are synthetic (seeded
generator, generated in HBM before the timed region); the other N-1 ranks'
contributions are local buffers on the one GPU.

Default workload: the Qwen2.5-3B shape (3,085,938,688 parameters, 434
tensors, 128-element tensor alignment) at N=4, rank 0 -- a 771,484,672-element
shard -- through the fused kernel, after one warm step. The fused steps of the
Llama-7B shape (N=8) and the Llama-70B shape (N=64) are timed as well and
reported under ``other_workloads``. Prints one JSON line. ``--gpus`` above 1
exits: this benchmark is one GPU's share by construction.
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E peak
KERNEL_SRC = os.path.join(ROOT, "fsdp_sharded_mixed_flatten_amd", "csrc", "zs_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

METRIC = "shard step: params updated/s + achieved HBM GB/s (% of MI355X peak)"


def kernel_hash():
    with open(KERNEL_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def fused_bytes_per_param(N, write_grad=False, write_param=False):
    # read: N bf16 contributions + fp32 master, m, v; write: fp32 master, m, v + bf16 slice of full
    return 2 * N + 12 + 12 + 2 + (2 if write_grad else 0) + (2 if write_param else 0)


def unfused_bytes_per_param(N):
    # reduce (2N read + 2 write) + AdamW (2 + 12 read, 12 + 2 write) + gather (2 + 2)
    return (2 * N + 2) + 28 + 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3b",
                    choices=["tiny", "qwen3b", "llama7b", "llama7b_wrap", "llama70b"])
    ap.add_argument("--also", default="llama7b,llama70b",
                    help="comma-separated FLAT workloads whose fused step is also timed and reported under "
                         "'other_workloads' ('none' skips them)")
    ap.add_argument("--no-unfused", action="store_true", help="skip the unfused path's timing")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-window", type=int, default=100_000_000,
                    help="owned elements of the CPU oracle's timed window")
    ap.add_argument("--arena-pad-kb", type=int, default=-1,
                    help="allocate the N contributions (and master/m/v) as rows of one buffer whose "
                         "rows start this many KiB apart beyond their length (-1: separate tensors)")
    ap.add_argument("--accum", type=int, default=4,
                    help="also time an optimizer step with this many accumulated micro-batches, global-norm "
                         "clipping and the non-finite skip (FLAT workloads; 0 skips it)")
    ap.add_argument("--clip", type=float, default=1.0, help="max norm of the --accum path")
    ap.add_argument("--quant", default="4:256",
                    help="BITS:BLOCK of the quantized-gather legs (fused step writing codes, and the "
                         "dequantizing gather of all ranks' payloads), FLAT workloads; 'none' skips them")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the CPU-offloaded optimizer step leg (FLAT workloads up to the 7B shape)")
    ap.add_argument("--offload-chunk", type=int, default=1 << 24, help="elements per offload pipeline chunk")
    ap.add_argument("--no-separate", action="store_true",
                    help="per-tensor workloads: skip the leg with one allocation per piece and array")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="also run a plain device copy of this many GiB (counter calibration)")
    return ap.parse_args()


def p99(xs):
    ys = sorted(xs)
    return ys[min(len(ys) - 1, int(round(0.99 * (len(ys) - 1))))]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Timer:
    """HIP events on torch's current stream (the stream the kernels run on)."""

    def __init__(self):
        import torch
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((s, e))

    def ms(self):
        self.torch.cuda.synchronize()
        return [s.elapsed_time(e) for s, e in self.pairs]


def rows(n_rows, S, dtype, pad_kb):
    """n_rows buffers of S elements: separate tensors (pad_kb < 0) or rows of
    one allocation whose starts are S*itemsize + pad_kb KiB apart."""
    import torch
    if pad_kb < 0:
        return [torch.empty(S, dtype=dtype, device="cuda") for _ in range(n_rows)]
    item = torch.empty(0, dtype=dtype).element_size()
    pitch = S + pad_kb * 1024 // item
    arena = torch.empty(n_rows * pitch, dtype=dtype, device="cuda")
    return [arena[r * pitch:r * pitch + S] for r in range(n_rows)]


def flat_setup(zs, synth, wl, pad_kb=-1):
    import torch
    plan = zs.zs_shard_plan(wl.numels, wl.world, wl.rank, wl.align, zs.ZS_LAYOUT_FLAT)
    S, T = plan.shard_numel, plan.padded_numel
    base, valid = wl.rank * S, sum(wl.numels)
    st = {}
    st["contribs"] = rows(wl.world, S, torch.int16, pad_kb)
    for q, c in enumerate(st["contribs"]):
        synth.gpu_bf16(c, base, wl.contrib_spec(q, 1, valid))
    st["master"], st["m"], st["v"] = rows(3, S, torch.float32, pad_kb)
    synth.gpu_f32(st["master"], base, wl.master_spec(valid))
    st["m"].zero_()
    st["v"].zero_()
    st["grad"] = torch.empty(S, dtype=torch.int16, device="cuda")
    st["param"] = torch.empty(S, dtype=torch.int16, device="cuda")
    free, _ = torch.cuda.mem_get_info()
    # the full gathered buffer (T elements) when it fits; rank 0 writes only [0, S)
    full_elems = T if free > T * 2 + (4 << 30) else (wl.rank + 1) * S
    st["full"] = torch.empty(full_elems, dtype=torch.int16, device="cuda")
    st["full_is_T"] = full_elems == T
    torch.cuda.synchronize()
    return plan, st


def per_tensor_setup(zs, synth, oracle, wl, packed=True):
    """PER_TENSOR pieces. packed: every piece's buffers are carved from one
    allocation per array at the plan's shard offset (the gathered tensors from
    one packed buffer at their flat offsets), contiguous as DeepSpeed's
    contiguous_gradients keeps them; otherwise one allocation per piece and
    array, as per-parameter tensors would be."""
    import torch
    plan = zs.zs_shard_plan(wl.numels, wl.world, wl.rank, 1, zs.ZS_LAYOUT_PER_TENSOR)
    op = oracle.plan_per_tensor(wl.numels, wl.world, wl.rank)
    S = plan.shard_numel
    if packed:
        arena = {k: torch.empty(S, dtype=dt, device="cuda") for k, dt in
                 (("grad", torch.int16), ("master", torch.float32), ("m", torch.float32), ("v", torch.float32),
                  ("param", torch.int16))}
        arena["m"].zero_()
        arena["v"].zero_()
        carena = [torch.empty(S, dtype=torch.int16, device="cuda") for _ in range(wl.world)]
        full_arena = torch.empty(op.T, dtype=torch.int16, device="cuda")
    pieces, contribs = [], [[] for _ in range(wl.world)]
    for i, pc in enumerate(op.pieces):
        Si = pc.own_hi - pc.own_lo
        valid = op.offsets[i] + wl.numels[i]
        if packed:
            lo = pc.shard_off
            d = {k: arena[k][lo:lo + Si] for k in arena}
            d["full"] = full_arena[op.offsets[i]:op.offsets[i] + op.padded[i]]
        else:
            d = dict(grad=torch.empty(Si, dtype=torch.int16, device="cuda"),
                     master=torch.empty(Si, dtype=torch.float32, device="cuda"),
                     m=torch.zeros(Si, dtype=torch.float32, device="cuda"),
                     v=torch.zeros(Si, dtype=torch.float32, device="cuda"),
                     param=torch.empty(Si, dtype=torch.int16, device="cuda"),
                     full=torch.empty(op.padded[i], dtype=torch.int16, device="cuda"))
        synth.gpu_f32(d["master"], pc.full_off, wl.master_spec(valid))
        pieces.append(d)
        for q in range(wl.world):
            c = carena[q][pc.shard_off:pc.shard_off + Si] if packed else torch.empty(Si, dtype=torch.int16,
                                                                                      device="cuda")
            synth.gpu_bf16(c, pc.full_off, wl.contrib_spec(q, 1, valid))
            contribs[q].append(c)
    ws = torch.zeros(zs.zs_multi_workspace_bytes(plan, wl.world), dtype=torch.uint8, device="cuda")
    zs.zs_multi_bind(plan, pieces, contribs, ws)
    ws_fused = torch.zeros_like(ws)
    zs.zs_multi_bind(plan, [dict(pc, param=None, grad=None) for pc in pieces], contribs, ws_fused)
    torch.cuda.synchronize()
    return plan, dict(pieces=pieces, contribs=contribs, ws=ws, ws_fused=ws_fused)


GRAPH_MAX_ELEMS = 1 << 24  # shards up to this size are launch-bound: also time their steps from a HIP graph


def graph_time(torch, fn, steps_per_graph, replays):
    """fn(t, None) for t = 1 .. steps_per_graph captured once into one HIP
    graph (PyTorch's CUDAGraph drives HIP graphs on ROCm) and replayed
    `replays` times back to back; returns device ms per step from one event
    pair around the replays. Kernel arguments are fixed at capture, so every
    replay repeats the same step counts on the evolving state."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for t in range(1, steps_per_graph + 1):
            fn(t, None)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / (replays * steps_per_graph)


def time_loop(fn, warmup, steps):
    """Runs fn(t, timer) for `warmup` untimed steps, then `steps` timed steps
    launched back to back. Returns (wall ms per step, bracketed by device
    synchronization; device ms per step from one HIP event pair on the
    stream the kernels run on; per-step event durations of a second,
    separately timed pass, for the median and P99)."""
    import torch
    for i in range(warmup):
        fn(i + 1, None)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        fn(warmup + i + 1, None)
    stop.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    dev_ms = start.elapsed_time(stop) / steps
    timer = Timer()
    for i in range(steps):
        fn(warmup + steps + i + 1, timer)
    return wall_ms, dev_ms, timer.ms()


def cpu_baseline(oracle, synth, wl, S, window, fused_bpp):
    """The oracle's shard step timed on this host over a window of the same workload."""
    import numpy as np
    n = min(window, S)
    base, valid = wl.rank * S, sum(wl.numels)
    contribs = [synth.cpu_bf16(n, base, wl.contrib_spec(q, 1, valid)) for q in range(wl.world)]
    master = synth.cpu_f32(n, base, wl.master_spec(valid))
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    g, p = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    full = np.zeros(n, np.uint16)  # the window's slice of the gathered buffer (rank 0: offset 0)
    threads = max(1, min(16, os.cpu_count() or 1))
    hp = oracle.HParams(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, 1)
    secs = oracle.time_shard_step(hp, contribs, g, master, m, v, p, full, threads, 6)
    med = statistics.median(secs[1:])
    secs1 = oracle.time_shard_step(hp, contribs, g, master, m, v, p, full, 1, 1)
    cpu_seconds = threads * sum(secs) + secs1[0]
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu_model)
    except OSError:
        pass
    return {"value": n / med, "unit": "params/s", "cores": threads, "kind": "oracle",
            "host_cpu": cpu_model, "host_logical_cpus": os.cpu_count(),
            "sample": f"{n:,}-element window of the {wl.name} shard (N={wl.world}), "
                      f"median of 5 timed passes after 1 warm-up, {threads} threads, plus one "
                      f"single-thread pass; {cpu_seconds:.1f} core-seconds of oracle work",
            "core_seconds": cpu_seconds,
            "gbps_algorithmic": n * fused_bpp / med / 1e9,
            "single_thread_params_per_s": n / secs1[0]}


def extra_fused_leg(zs, synth, torch, name, args):
    """The fused step of another FLAT workload, timed like the main one."""
    wl = synth.workloads()[name]
    N = wl.world
    hp0 = zs.AdamWHParams(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, 1)
    log(f"[bench] also: workload={wl.name} N={N} rank={wl.rank}")
    try:
        plan, st = flat_setup(zs, synth, wl)
    except torch.cuda.OutOfMemoryError as e:
        torch.cuda.empty_cache()
        return {"skipped": f"device memory: {str(e).splitlines()[0]}"}
    S = plan.shard_numel
    write_grad = N >= 64
    grad_out = st["grad"] if write_grad else None

    def fused(t, timer):
        e = timer.start() if timer else None
        zs.zs_fused_shard_step(plan, hp0.at(t), st["contribs"], st["master"], st["m"], st["v"], grad=grad_out,
                               full=st["full"])
        if timer:
            timer.stop(e)

    wall, kern, ev = time_loop(fused, args.warmup, args.steps)
    bpp = fused_bytes_per_param(N, write_grad=write_grad)
    kname = "k_reduce+k_adamw" if write_grad else "k_fused"
    achieved = S * bpp / (kern / 1e3) / 1e9
    out = {"workload": f"{wl.name}_n{N}_fused", "world_size": N, "shard_elems": S, "ms_per_step": wall,
           "kernel_ms_mean": kern, "kernel_ms_median": statistics.median(ev), "kernel_ms_p99": p99(ev),
           "params_per_s": S / (wall / 1e3), "bytes_per_param": bpp,
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBPS, "traffic": read_traffic(kname, wl.name), "kernel": kname,
                        "algorithmic_bytes_per_launch": S * bpp}}
    del st, plan
    torch.cuda.empty_cache()
    return out


def offload_leg(zs, torch, plan, st, hp0, S, args, fused):
    """ZeRO-Offload step: device grad shard -> pinned host, host AdamW on
    pinned fp32 state, bf16 parameters -> the gathered buffer; pipelined in
    chunks. Times whole steps (host arithmetic included)."""
    threads = max(1, min(16, os.cpu_count() or 1))
    try:
        t0 = time.perf_counter()
        hm = torch.empty(S, dtype=torch.float32, pin_memory=True)
        hm.copy_(st["master"].cpu())
        hmm = torch.zeros(S, dtype=torch.float32, pin_memory=True)
        hv = torch.zeros(S, dtype=torch.float32, pin_memory=True)
        gh = torch.empty(S, dtype=torch.int16, pin_memory=True)
        ph = torch.empty(S, dtype=torch.int16, pin_memory=True)
        alloc_s = time.perf_counter() - t0
    except RuntimeError as e:
        return {"skipped": f"pinned host buffers: {e}"}
    zs.zs_reduce_shard(plan, st["contribs"], st["grad"])

    def step(t, timer):
        e = timer.start() if timer else None
        zs.zs_offload_adamw_step(plan, hp0.at(t), st["grad"], hm, hmm, hv, gh, ph, full_dev=st["full"],
                                 chunk_elems=args.offload_chunk, n_threads=threads)
        if timer:
            timer.stop(e)

    wall, dev, ev = time_loop(step, 1, 3)
    host_bpp, pcie_bpp = 28, 4
    out = {"ms_per_step": wall, "events_ms_median": statistics.median(ev), "host_threads": threads,
           "chunk_elems": args.offload_chunk, "host_bytes_per_param": host_bpp, "pcie_bytes_per_param": pcie_bpp,
           "host_gbps": S * host_bpp / (wall / 1e3) / 1e9, "pcie_gbps": S * pcie_bpp / (wall / 1e3) / 1e9,
           "slowdown_vs_fused_gpu_step": wall / fused["ms_per_step"], "pinned_alloc_s": alloc_s}
    del hm, hmm, hv, gh, ph
    return out


def read_traffic(kernel_name, workload):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        data = json.load(open(TRAFFIC_FILE))
    except ValueError:
        return None
    rec = data.get(f"{workload}:{kernel_name}")
    if not rec or rec.get("kernel_src_sha256_16") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the step; --gpus {args.gpus} is not supported: "
              f"every rank runs the same kernels on its own shard, so one GPU at its real shard shape is "
              f"the measurement (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch

    import fsdp_sharded_mixed_flatten_amd as zs
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    wl = synth.workloads()[args.workload]
    N = wl.world
    hp0 = zs.AdamWHParams(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, 1)
    log(f"[bench] workload={wl.name} N={N} rank={wl.rank} layout={wl.layout}")
    result_paths = {}

    if args.calib_copy_gib > 0:
        n = int(args.calib_copy_gib * 2**30) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {n * 4:,} bytes read and written per launch, 3 launches")
        del a, b

    if wl.layout == "flat":
        plan, st = flat_setup(zs, synth, wl, args.arena_pad_kb)
        S = plan.shard_numel
        log(f"[bench] S={S:,} T={plan.padded_numel:,} gathered buffer {'full' if st['full_is_T'] else 'owned slice'}")

        # At large N the library runs the fused step as a reduce into the
        # grad shard followed by AdamW + gather, which needs the grad buffer
        # (part of the persistent 16 B/param state); its write is counted.
        write_grad = N >= 64
        grad_out = st["grad"] if write_grad else None

        def fused(t, timer):
            e = timer.start() if timer else None
            zs.zs_fused_shard_step(plan, hp0.at(t), st["contribs"], st["master"], st["m"], st["v"],
                                   grad=grad_out, full=st["full"])
            if timer:
                timer.stop(e)

        wall_ms, kern_ms, ev = time_loop(fused, args.warmup, args.steps)
        bpp = fused_bytes_per_param(N, write_grad=write_grad)
        result_paths["fused"] = {"ms_per_step": wall_ms, "kernel_ms_mean": kern_ms,
                                 "kernel_ms_median": statistics.median(ev), "kernel_ms_p99": p99(ev),
                                 "bytes_per_param": bpp, "launches_per_step": 2 if write_grad else 1,
                                 "kernel": "k_reduce+k_adamw" if write_grad else "k_fused"}
        main_path = "fused"
        graphable = {"fused": fused}
        if not args.no_unfused:
            B = wl.bucket_elems or S

            def unfused(t, timer):
                e = timer.start() if timer else None
                for off in range(0, S, B):
                    zs.zs_reduce_shard(plan, st["contribs"], st["grad"], off, min(B, S - off))
                zs.zs_adamw_shard_step(plan, hp0.at(t), st["grad"], st["master"], st["m"], st["v"],
                                       st["param"])
                zs.zs_gather_params(plan, st["param"], st["full"])
                if timer:
                    timer.stop(e)

            u_wall, u_dev, u_ev = time_loop(unfused, 1, max(3, args.steps // 2))
            graphable["unfused"] = unfused
            result_paths["unfused"] = {"ms_per_step": u_wall, "device_ms_per_step": u_dev,
                                       "events_ms_median": statistics.median(u_ev),
                                       "bytes_per_param": unfused_bytes_per_param(N),
                                       "launches_per_step": (S + B - 1) // B + 2,
                                       "reduce_buckets": (S + B - 1) // B}
            if B < S:
                # the fused step bucket by bucket, as it would run behind a bucketed exchange
                def fused_buckets(t, timer):
                    e = timer.start() if timer else None
                    for off in range(0, S, B):
                        zs.zs_fused_shard_step_bucket(plan, hp0.at(t), st["contribs"], st["master"], st["m"],
                                                      st["v"], off, min(B, S - off), grad=grad_out, full=st["full"])
                    if timer:
                        timer.stop(e)

                b_wall, b_dev, b_ev = time_loop(fused_buckets, 1, max(3, args.steps // 2))
                result_paths["fused_bucketed"] = {"ms_per_step": b_wall, "device_ms_per_step": b_dev,
                                                  "events_ms_median": statistics.median(b_ev),
                                                  "bytes_per_param": bpp,
                                                  "gbps": S * bpp / (b_dev / 1e3) / 1e9,
                                                  "buckets": (S + B - 1) // B}
        if args.quant != "none":
            bits, qblock = (int(x) for x in args.quant.split(":"))
            nq, ns = zs.zs_quant_code_bytes(plan, bits), zs.zs_quant_num_scales(plan, qblock)
            codes = torch.empty(nq, dtype=torch.uint8, device="cuda")
            scales = torch.empty(ns, dtype=torch.float32, device="cuda")

            def fused_q(t, timer):
                e = timer.start() if timer else None
                zs.zs_fused_shard_step_quant(plan, hp0.at(t), st["contribs"], st["master"], st["m"], st["v"],
                                             bits, qblock, codes, scales, grad=grad_out)
                if timer:
                    timer.stop(e)

            q_wall, q_dev, q_ev = time_loop(fused_q, 1, max(3, args.steps // 2))
            q_bpp = fused_bytes_per_param(N, write_grad=write_grad) - 2 + bits / 8 + 4 / qblock
            result_paths["fused_quant"] = {"bits": bits, "block": qblock, "ms_per_step": q_wall,
                                           "device_ms_per_step": q_dev, "events_ms_median": statistics.median(q_ev),
                                           "bytes_per_param": q_bpp, "gbps": S * q_bpp / (q_dev / 1e3) / 1e9,
                                           "payload_bytes": nq + 4 * ns,
                                           "bf16_slice_bytes": 2 * S}
            T = plan.padded_numel
            free, _ = torch.cuda.mem_get_info()
            if st["full_is_T"] and free > N * (nq + 4 * ns) + (2 << 30):
                # every rank's payload (copies of this rank's stand in for the others)
                codes_all = codes.repeat(N)
                scales_all = scales.repeat(N)

                def dequant(t, timer):
                    e = timer.start() if timer else None
                    zs.zs_dequant_gather(plan, bits, qblock, codes_all, scales_all, st["full"])
                    if timer:
                        timer.stop(e)

                d_wall, d_dev, d_ev = time_loop(dequant, 1, max(3, args.steps // 2))
                d_bpe = bits / 8 + 4 / qblock + 2
                result_paths["dequant_gather"] = {"bits": bits, "block": qblock, "gathered_elems": T,
                                                  "ms_per_step": d_wall, "device_ms_per_step": d_dev,
                                                  "events_ms_median": statistics.median(d_ev),
                                                  "bytes_per_gathered_elem": d_bpe,
                                                  "gbps": T * d_bpe / (d_dev / 1e3) / 1e9}
                del codes_all, scales_all
            else:
                result_paths["dequant_gather"] = {"skipped": "the gathered buffer and all payloads do not fit "
                                                             "beside the resident contributions"}
            del codes, scales
        if not args.no_offload and S <= 1_000_000_000:
            result_paths["offload"] = offload_leg(zs, torch, plan, st, hp0, S, args, result_paths["fused"])
        if args.accum > 0:
            G, B = args.accum, wl.bucket_elems or S
            acc = torch.empty(S, dtype=torch.float32, device="cuda")
            sumsq = torch.zeros(N, dtype=torch.float64, device="cuda")
            flags = torch.zeros(N, dtype=torch.int32, device="cuda")
            scale = torch.zeros(1, dtype=torch.float32, device="cuda")
            skip = torch.zeros(1, dtype=torch.int32, device="cuda")
            ws = torch.zeros(zs.zs_grad_stats_workspace_bytes(plan), dtype=torch.uint8, device="cuda")

            def accum_step(t, timer):
                e = timer.start() if timer else None
                for k in range(G):  # each micro-step's contributions (resident inputs reused)
                    for off in range(0, S, B):
                        zs.zs_accumulate_shard(plan, st["contribs"], acc, off, min(B, S - off), first=(k == 0))
                zs.zs_grad_stats(plan, acc, float(G), sumsq[0:1], flags[0:1], ws)
                # the other ranks' squared norms arrive by an all-reduce in a
                # multi-GPU job; copies of this rank's stand in for them here
                sumsq[1:].copy_(sumsq[0:1].expand(N - 1))
                flags[1:].copy_(flags[0:1].expand(N - 1))
                zs.zs_clip_scale(sumsq, flags, args.clip, scale, skip)
                zs.zs_adamw_shard_step_accum(plan, hp0.at(t), acc, float(G), st["master"], st["m"], st["v"],
                                             scale=scale, skip=skip, full=st["full"])
                if timer:
                    timer.stop(e)

            a_wall, a_dev, a_ev = time_loop(accum_step, 1, max(3, args.steps // 2))
            graphable["accum_clip"] = accum_step
            a_bytes = G * (2 * N + 8) - 4 + 4 + 30  # micro-steps (first one does not read acc), stats, AdamW
            result_paths["accum_clip"] = {"micro_steps": G, "max_norm": args.clip, "ms_per_step": a_wall,
                                          "device_ms_per_step": a_dev, "events_ms_median": statistics.median(a_ev),
                                          "bytes_per_param": a_bytes,
                                          "gbps": S * a_bytes / (a_dev / 1e3) / 1e9}
        if S <= GRAPH_MAX_ELEMS:
            # launch-bound: the same steps replayed from a HIP graph, 20 per graph
            for name, fn in graphable.items():
                g_ms = graph_time(torch, fn, 20, max(5, args.steps // 20))
                result_paths[name]["graph_ms_per_step"] = g_ms
                result_paths[name]["graph_speedup_over_eager"] = result_paths[name]["ms_per_step"] / g_ms
    else:
        import oracle
        plan, st = per_tensor_setup(zs, synth, oracle, wl)
        S = plan.shard_numel
        log(f"[bench] per-tensor plan: {plan.num_tensors} pieces, S={S:,}")

        def fused(t, timer):
            e = timer.start() if timer else None
            zs.zs_fused_shard_step_multi(plan, hp0.at(t), st["ws_fused"])
            if timer:
                timer.stop(e)

        wall_ms, kern_ms, ev = time_loop(fused, args.warmup, args.steps)
        bpp = fused_bytes_per_param(N)
        result_paths["fused_multi"] = {"ms_per_step": wall_ms, "kernel_ms_mean": kern_ms,
                                       "kernel_ms_median": statistics.median(ev),
                                       "kernel_ms_p99": p99(ev), "bytes_per_param": bpp,
                                       "launches_per_step": 1, "kernel": "k_multi"}
        main_path = "fused_multi"
        if not args.no_unfused:
            def unfused(t, timer):
                e = timer.start() if timer else None
                zs.zs_reduce_shard_multi(plan, st["ws"])
                zs.zs_adamw_shard_step_multi(plan, hp0.at(t), st["ws"])
                zs.zs_gather_params_multi(plan, st["ws"])
                if timer:
                    timer.stop(e)

            u_wall, u_dev, u_ev = time_loop(unfused, 1, max(3, args.steps // 2))
            result_paths["unfused_multi"] = {"ms_per_step": u_wall, "device_ms_per_step": u_dev,
                                             "events_ms_median": statistics.median(u_ev),
                                             "bytes_per_param": unfused_bytes_per_param(N),
                                             "launches_per_step": 3}
        if not args.no_separate:
            del st
            torch.cuda.empty_cache()
            plan2, st2 = per_tensor_setup(zs, synth, oracle, wl, packed=False)

            def fused_sep(t, timer):
                e = timer.start() if timer else None
                zs.zs_fused_shard_step_multi(plan2, hp0.at(t), st2["ws_fused"])
                if timer:
                    timer.stop(e)

            s_wall, s_dev, s_ev = time_loop(fused_sep, 1, max(3, args.steps // 2))
            result_paths["fused_multi_separate_allocations"] = {
                "ms_per_step": s_wall, "device_ms_per_step": s_dev, "events_ms_median": statistics.median(s_ev),
                "bytes_per_param": bpp, "gbps": S * bpp / (s_dev / 1e3) / 1e9}
            del st2

    params_per_s = S / (wall_ms / 1e3)
    achieved = S * bpp / (kern_ms / 1e3) / 1e9
    step_gbps = S * bpp / (wall_ms / 1e3) / 1e9
    kname = result_paths[main_path]["kernel"]
    traffic = read_traffic(kname, wl.name)
    gathered = "full" if wl.layout != "flat" or st.get("full_is_T") else "owned slice"
    st = None
    torch.cuda.empty_cache()
    others = {}
    for name in ([] if args.also == "none" else [x for x in args.also.split(",") if x and x != wl.name]):
        if synth.workloads()[name].layout != "flat":
            continue
        others[name] = extra_fused_leg(zs, synth, torch, name, args)
    cpu = None
    if not args.no_cpu:
        import oracle
        log(f"[bench] CPU oracle baseline on a {min(args.cpu_window, S):,}-element window")
        cpu = cpu_baseline(oracle, synth, wl, S, args.cpu_window, bpp)
    out = {
        "metric": METRIC,
        "value": params_per_s,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded counter-based generator; model shapes only, no weights)",
        "config": {"workload": f"{wl.name}_n{N}_{main_path}", "world_size": N, "rank": wl.rank,
                   "layout": wl.layout, "shard_elems": S, "bytes_per_param": bpp,
                   "gathered_buffer": gathered,
                   **({"piece_buffers": "carved from one allocation per array at the plan's offsets"}
                      if wl.layout != "flat" else {})},
        "hbm_gbps": step_gbps,
        "pct_of_peak": 100.0 * step_gbps / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": kname, "algorithmic_bytes_per_launch": S * bpp},
        "cpu_baseline": cpu,
        "paths": result_paths,
        "other_workloads": others,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
