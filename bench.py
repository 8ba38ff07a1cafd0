"""Benchmark of one rank's shard-local step (reduce + mixed-precision AdamW +
gather) on one MI355X.

A step is one pass of the whole path over the owned shard: the average of the
N bf16 gradient contributions, AdamW on the fp32 master/m/v state, and the
bf16 parameter write into the gathered buffer. Inputs are synthetic (seeded
generator, generated in HBM before the timed region); the other N-1 ranks'
contributions are local buffers on the one GPU.

Default workload: the Llama-70B shape (70,553,706,496 parameters, 723
tensors) at N=64, rank 0 -- a 1,102,401,664-element shard with 141 GB of
contributions -- through the fused entry point, which at this world size runs
the reduce into the grad shard and then AdamW writing the gathered slice. The
step is timed on several independently allocated buffer sets (the median is
reported), and once more with HIP events around each of its two kernels for
the roofline of the dominant one. Also timed and reported under
``other_workloads``: the Qwen2.5-3B shape (N=4), the Llama-7B shape (N=8,
median over buffer sets allocated side by side), the same 7B shard stepped in
34 buckets of 25M elements, and the 7B shape wrapped per tensor (291 pieces,
multi-tensor apply; packed arenas and one allocation per piece). Prints one
JSON line. ``--gpus`` above 1 exits: this benchmark is one GPU's share by
construction.
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
KERNEL_SRCS = ([os.path.join(ROOT, "fsdp_sharded_mixed_flatten_amd", "csrc", f) for f in ("zs_kernels.hip", "zs_internal.h")]
               + [os.path.join(ROOT, "include", "zs.h")])
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

METRIC = "shard step: params updated/s + achieved HBM GB/s (% of MI355X peak)"
GRAPH_MAX_ELEMS = 1 << 24  # shards up to this size are launch-bound: also time their steps from a HIP graph


# ---------------------------------------------------------------- algorithmic bytes per owned element


def reduce_bpp(N):
    return 2 * N + 2  # N bf16 contributions read, the bf16 average written


def adamw_bpp():
    return 2 + 12 + 12 + 2  # bf16 grad + fp32 master/m/v read; fp32 master/m/v + one bf16 parameter written


def fused_bpp(N, write_grad=False, write_param=False):
    # read: N bf16 contributions + fp32 master, m, v; write: fp32 master, m, v + bf16 slice of full
    return 2 * N + 12 + 12 + 2 + (2 if write_grad else 0) + (2 if write_param else 0)


def unfused_bpp(N):
    return reduce_bpp(N) + adamw_bpp() + 4  # + gather (2 read + 2 write)


def code_text(src):
    """C++ source without its comments, whitespace runs collapsed: what the
    compiler sees of it (string and character literals kept as written)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_hash():
    """Hash of the kernels' code (the kernel source, its internal header and
    the public header whose constants they use; comments and layout
    excluded): counter-measured traffic stays valid across comment edits and
    is dropped by any change to the code."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama70b",
                    choices=["tiny", "qwen3b", "llama7b", "llama7b_bucketed", "llama7b_wrap", "llama70b"])
    ap.add_argument("--also", default="qwen3b,llama7b,llama7b_bucketed,llama7b_wrap",
                    help="comma-separated workloads also timed and reported under 'other_workloads' "
                         "('none' skips them)")
    ap.add_argument("--placements", type=int, default=3,
                    help="independently allocated buffer sets the fused step is timed on (median reported)")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only the fused step of each workload (no unfused, quantized, accumulation "
                         "or offload legs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-window", type=int, default=25_000_000,
                    help="owned elements of the CPU oracle's timed window")
    ap.add_argument("--accum", type=int, default=4,
                    help="micro-batches of the accumulation + clipping leg (0 skips it)")
    ap.add_argument("--clip", type=float, default=1.0, help="max norm of the accumulation leg")
    ap.add_argument("--quant", default="4:256",
                    help="BITS:BLOCK of the quantized-gather legs; 'none' skips them")
    ap.add_argument("--offload-chunk", type=int, default=1 << 24, help="elements per offload pipeline chunk")
    ap.add_argument("--world", type=int, default=0,
                    help="cut the --workload shape for this world size (1..256) instead of its own; "
                         "the other workloads are then not run")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="also run a plain device copy of this many GiB (counter calibration)")
    return ap.parse_args()


def p99(xs):
    ys = sorted(xs)
    return ys[min(len(ys) - 1, int(round(0.99 * (len(ys) - 1))))]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Timer:
    """HIP event pairs on torch's current stream, the stream the library's
    kernels are launched on (every call below passes no stream, so the
    binding uses torch.cuda.current_stream())."""

    def __init__(self):
        import torch
        self.torch = torch
        self.pairs = {}

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s, key="step"):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.setdefault(key, []).append((s, e))

    def ms(self, key="step"):
        self.torch.cuda.synchronize()
        return [s.elapsed_time(e) for s, e in self.pairs.get(key, [])]


def time_loop(fn, warmup, steps):
    """fn(t, timer) for `warmup` untimed steps, then `steps` timed steps
    launched back to back. Returns (wall ms per step bracketed by device
    synchronization, device ms per step from one HIP event pair around the
    timed steps, the Timer of a second pass whose fn calls record per-step
    or per-kernel event pairs)."""
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
    torch.cuda.synchronize()
    return wall_ms, dev_ms, timer


def graph_time(torch, fn, steps_per_graph, replays):
    """fn(t, None) for t = 1 .. steps_per_graph captured once into one HIP
    graph (PyTorch's CUDAGraph drives HIP graphs on ROCm) and replayed
    `replays` times back to back; device ms per step."""
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


def read_traffic(kernel_name, workload):
    """Counter-measured HBM bytes per launch (profiles/traffic.json), or None
    once the kernels' code (kernel_hash) has changed since the counters were
    taken."""
    if workload is None or not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except ValueError:
        return None
    rec = data.get(f"{workload}:{kernel_name}")
    if not rec or rec.get("kernel_code_sha256_16") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def roofline(kernel, workload, units, bpp, launch_ms):
    achieved = units * bpp / (launch_ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": read_traffic(kernel, workload), "kernel": kernel,
            "bytes_per_param": bpp, "algorithmic_bytes_per_launch": units * bpp, "launch_ms": launch_ms}


def release():
    import gc

    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- buffer sets


def flat_buffers(zs, synth, wl, plan, full="auto"):
    """One FLAT buffer set: N contributions, fp32 master/m/v, bf16 grad and
    param shards, and the gathered buffer (all T elements when it fits, else
    the owned slice; rank 0 writes [0, S) of either)."""
    import torch
    S, T = plan.shard_numel, plan.padded_numel
    base, valid = wl.rank * S, sum(wl.numels)
    st = {"contribs": [torch.empty(S, dtype=torch.int16, device="cuda") for _ in range(wl.world)]}
    for q, c in enumerate(st["contribs"]):
        synth.gpu_bf16(c, base, wl.contrib_spec(q, 1, valid))
    st["master"], st["m"], st["v"] = (torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(3))
    synth.gpu_f32(st["master"], base, wl.master_spec(valid))
    st["m"].zero_()
    st["v"].zero_()
    st["grad"] = torch.empty(S, dtype=torch.int16, device="cuda")
    st["param"] = torch.empty(S, dtype=torch.int16, device="cuda")
    free, _ = torch.cuda.mem_get_info()
    if full == "auto":
        full = "T" if free > T * 2 + (4 << 30) else "slice"
    full_elems = T if full == "T" else (wl.rank + 1) * S
    st["full"] = torch.empty(full_elems, dtype=torch.int16, device="cuda")
    st["full_is_T"] = full_elems == T
    st["full_own"] = st["full"][wl.rank * S:(wl.rank + 1) * S]
    torch.cuda.synchronize()
    return st


def per_tensor_buffers(zs, synth, wl, plan, packed=True):
    """PER_TENSOR pieces laid out from the library's plan (zs_plan_tensor).
    packed: every piece's buffers are carved from one allocation per array
    at the piece's shard offset (the gathered tensors from one packed buffer
    at their offsets), contiguous as DeepSpeed's contiguous_gradients keeps
    them; otherwise one allocation per piece and array, as per-parameter
    tensors are."""
    import torch
    S, T = plan.shard_numel, plan.padded_numel
    infos = [plan.tensor(i) for i in range(plan.num_tensors)]
    if packed:
        arena = {k: torch.empty(S, dtype=dt, device="cuda") for k, dt in
                 (("grad", torch.int16), ("master", torch.float32), ("m", torch.float32), ("v", torch.float32),
                  ("param", torch.int16))}
        arena["m"].zero_()
        arena["v"].zero_()
        carena = [torch.empty(S, dtype=torch.int16, device="cuda") for _ in range(wl.world)]
        full_arena = torch.empty(T, dtype=torch.int16, device="cuda")
    pieces, contribs = [], [[] for _ in range(wl.world)]
    for info in infos:
        Si = info.own_hi - info.own_lo
        full_off = info.flat_off + info.own_lo  # packed global index of the piece's first element
        valid = info.flat_off + info.numel     # global indices past the tensor's end are padding
        if packed:
            lo = info.shard_off
            d = {k: arena[k][lo:lo + Si] for k in arena}
            d["full"] = full_arena[info.flat_off:info.flat_off + info.padded_numel]
        else:
            d = dict(grad=torch.empty(Si, dtype=torch.int16, device="cuda"),
                     master=torch.empty(Si, dtype=torch.float32, device="cuda"),
                     m=torch.zeros(Si, dtype=torch.float32, device="cuda"),
                     v=torch.zeros(Si, dtype=torch.float32, device="cuda"),
                     param=torch.empty(Si, dtype=torch.int16, device="cuda"),
                     full=torch.empty(info.padded_numel, dtype=torch.int16, device="cuda"))
        synth.gpu_f32(d["master"], full_off, wl.master_spec(valid))
        pieces.append(d)
        for q in range(wl.world):
            c = (carena[q][info.shard_off:info.shard_off + Si] if packed
                 else torch.empty(Si, dtype=torch.int16, device="cuda"))
            synth.gpu_bf16(c, full_off, wl.contrib_spec(q, 1, valid))
            contribs[q].append(c)
    ws = torch.zeros(zs.zs_multi_workspace_bytes(plan, wl.world), dtype=torch.uint8, device="cuda")
    zs.zs_multi_bind(plan, pieces, contribs, ws)
    ws_fused = torch.zeros_like(ws)
    zs.zs_multi_bind(plan, [dict(pc, param=None, grad=None) for pc in pieces], contribs, ws_fused)
    torch.cuda.synchronize()
    return dict(pieces=pieces, contribs=contribs, ws=ws, ws_fused=ws_fused)


def unbind(zs, st):
    for k in ("ws", "ws_fused"):
        if st.get(k) is not None:
            zs.zs_multi_unbind(st[k])


# ---------------------------------------------------------------- legs


def fused_step_fn(zs, plan, hp0, st, N):
    """The fused entry point as a caller runs it: from
    zs.FUSED_TWO_PASS_MIN_CONTRIBS contributions on with the grad shard given
    (part of the persistent 16 B/param state), which selects the reduce +
    AdamW/gather two-pass form; one kernel otherwise."""
    grad = st["grad"] if N >= zs.FUSED_TWO_PASS_MIN_CONTRIBS else None

    def step(t, timer):
        e = timer.start() if timer else None
        zs.zs_fused_shard_step(plan, hp0.at(t), st["contribs"], st["master"], st["m"], st["v"], grad=grad,
                               full=st["full"])
        if timer:
            timer.stop(e)
    return step


def split_kernels_fn(zs, plan, hp0, st):
    """The two kernels of the two-pass fused step issued as their own calls,
    so each gets its own event pair: the reduce into the grad shard (the
    kernel k_reduce), then AdamW writing the owned slice of the gathered
    buffer (k_adamw). Same kernels, same bytes as the fused entry point."""

    def step(t, timer):
        e = timer.start() if timer else None
        zs.zs_reduce_shard(plan, st["contribs"], st["grad"])
        if timer:
            timer.stop(e, "reduce")
            e = timer.start()
        zs.zs_adamw_shard_step(plan, hp0.at(t), st["grad"], st["master"], st["m"], st["v"], st["full_own"])
        if timer:
            timer.stop(e, "adamw")
    return step


def flat_workload(zs, synth, torch, wl, args, primary):
    """The fused step of a FLAT workload on `args.placements` buffer sets
    (sequentially reallocated, or side by side when they fit), plus, for the
    primary workload, the extra legs."""
    N = wl.world
    plan = zs.zs_shard_plan(wl.numels, wl.world, wl.rank, wl.align, zs.ZS_LAYOUT_FLAT)
    S, T = plan.shard_numel, plan.padded_numel
    hp0 = zs.AdamWHParams(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, 1)
    two_pass = N >= zs.FUSED_TWO_PASS_MIN_CONTRIBS
    bpp = fused_bpp(N, write_grad=two_pass)
    log(f"[bench] workload={wl.name} N={N} rank={wl.rank} S={S:,} T={T:,}")
    free, _ = torch.cuda.mem_get_info()
    set_bytes = S * (2 * N + 16) + T * 2
    side_by_side = args.placements > 1 and free > args.placements * set_bytes + (8 << 30)
    sets, results = [], []
    P = max(1, args.placements)
    for k in range(P):
        st = flat_buffers(zs, synth, wl, plan)
        fn = fused_step_fn(zs, plan, hp0, st, N)
        wall, dev, timer = time_loop(fn, args.warmup, args.steps)
        ev = timer.ms()
        res = {"ms_per_step": wall, "device_ms_per_step": dev, "events_ms_median": statistics.median(ev),
               "events_ms_p99": p99(ev), "full_buffer": "T" if st["full_is_T"] else "owned slice"}
        if two_pass:
            split = split_kernels_fn(zs, plan, hp0, st)
            wall2, dev2, t2 = time_loop(split, 1, args.steps)
            r_ms, a_ms = t2.ms("reduce"), t2.ms("adamw")
            res["reduce_ms_mean"] = statistics.fmean(r_ms)
            res["adamw_ms_mean"] = statistics.fmean(a_ms)
            res["split_device_ms_per_step"] = dev2
            del split
        del fn
        results.append(res)
        log(f"[bench]   buffer set {k}: {wall:.3f} ms/step" +
            (f" (reduce {res['reduce_ms_mean']:.3f} + adamw {res['adamw_ms_mean']:.3f} ms)" if two_pass else ""))
        if side_by_side or k == P - 1:
            sets.append(st)
        else:
            st = None
            release()
        st = None
    # the reported buffer set: the one at the median step time
    order = sorted(range(len(results)), key=lambda i: results[i]["ms_per_step"])
    med = results[order[len(order) // 2]]
    wall = med["ms_per_step"]
    out = {"workload": f"{wl.name}_n{N}_fused", "world_size": N, "rank": wl.rank, "layout": "flat",
           "shard_elems": S, "padded_elems": T, "bytes_per_param": bpp, "ms_per_step": wall,
           "params_per_s": S / (wall / 1e3), "placements": [r["ms_per_step"] for r in results],
           "placement_spread": (max(r["ms_per_step"] for r in results) / min(r["ms_per_step"] for r in results))
           if results else None, "buffer_sets": "side by side" if side_by_side else "reallocated in turn",
           "median_set": med}
    if two_pass:
        # dominant kernel: the N-way reduce (2N+2 bytes per owned element)
        out["roofline"] = roofline("k_reduce", traffic_key(wl), S, reduce_bpp(N), med["reduce_ms_mean"])
        out["kernels"] = {"k_reduce": {"ms": med["reduce_ms_mean"], "bytes_per_param": reduce_bpp(N),
                                       "gbps": S * reduce_bpp(N) / med["reduce_ms_mean"] / 1e6},
                          "k_adamw": {"ms": med["adamw_ms_mean"], "bytes_per_param": adamw_bpp(),
                                      "gbps": S * adamw_bpp() / med["adamw_ms_mean"] / 1e6,
                                      "note": "also reads the 2-byte grad shard the reduce wrote"}}
    else:
        out["roofline"] = roofline("k_fused", traffic_key(wl), S, bpp, med["device_ms_per_step"])
    # the whole step against the minimum the method moves: 2N+26 B per owned
    # element (plus the grad shard written by the two-pass form, which the ledger keeps)
    step_ms = med["device_ms_per_step"]
    out["step_roofline"] = {"min_bytes_per_param": fused_bpp(N), "bytes_per_param_counted": bpp,
                            "frac_at_min_bytes": S * fused_bpp(N) / (step_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
                            "frac_counted": S * bpp / (step_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
                            "step_ms": step_ms}
    # extra legs on the median buffer set (side by side) or the last one
    st = sets[order[len(order) // 2]] if side_by_side else sets[-1]
    paths = {}
    if (primary or wl.name == "llama7b") and not args.no_extra:
        paths = flat_extra_legs(zs, synth, torch, wl, plan, hp0, st, args, out)
    out["paths"] = paths
    sets.clear()
    st = None
    release()
    return out


def flat_extra_legs(zs, synth, torch, wl, plan, hp0, st, args, head):
    """Unfused, quantized, accumulation + clipping and offload legs on one buffer set."""
    N, S, T = wl.world, plan.shard_numel, plan.padded_numel
    two_pass = N >= zs.FUSED_TWO_PASS_MIN_CONTRIBS
    grad_out = st["grad"] if two_pass else None
    paths, graphable = {}, {"fused": fused_step_fn(zs, plan, hp0, st, N)}
    B = wl.bucket_elems or S

    def unfused(t, timer):
        e = timer.start() if timer else None
        for off in range(0, S, B):
            zs.zs_reduce_shard(plan, st["contribs"], st["grad"], off, min(B, S - off))
        zs.zs_adamw_shard_step(plan, hp0.at(t), st["grad"], st["master"], st["m"], st["v"], st["param"])
        zs.zs_gather_params(plan, st["param"], st["full"])
        if timer:
            timer.stop(e)

    u_wall, u_dev, u_t = time_loop(unfused, 1, max(3, args.steps // 2))
    graphable["unfused"] = unfused
    paths["unfused"] = {"ms_per_step": u_wall, "device_ms_per_step": u_dev,
                        "events_ms_median": statistics.median(u_t.ms()), "bytes_per_param": unfused_bpp(N),
                        "gbps": S * unfused_bpp(N) / u_dev / 1e6,
                        "launches_per_step": (S + B - 1) // B + 2, "reduce_buckets": (S + B - 1) // B}
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

        q_wall, q_dev, q_t = time_loop(fused_q, 1, max(3, args.steps // 2))
        q_bpp = fused_bpp(N, write_grad=two_pass) - 2 + bits / 8 + 4 / qblock
        paths["fused_quant"] = {"bits": bits, "block": qblock, "ms_per_step": q_wall, "device_ms_per_step": q_dev,
                                "events_ms_median": statistics.median(q_t.ms()), "bytes_per_param": q_bpp,
                                "gbps": S * q_bpp / q_dev / 1e6, "payload_bytes": nq + 4 * ns,
                                "bf16_slice_bytes": 2 * S}
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

            d_wall, d_dev, d_t = time_loop(dequant, 1, max(3, args.steps // 2))
            d_bpe = bits / 8 + 4 / qblock + 2
            paths["dequant_gather"] = {"bits": bits, "block": qblock, "gathered_elems": T, "ms_per_step": d_wall,
                                       "device_ms_per_step": d_dev, "events_ms_median": statistics.median(d_t.ms()),
                                       "bytes_per_gathered_elem": d_bpe,
                                       "roofline": roofline("k_dequant", traffic_key(wl), T, d_bpe, d_dev)}
            del codes_all, scales_all
        else:
            paths["dequant_gather"] = {"skipped": "the gathered buffer and all payloads do not fit beside the "
                                                  "resident contributions"}
        del codes, scales
    if S <= 1_000_000_000:
        paths["offload"] = offload_leg(zs, torch, plan, st, hp0, S, args, head["ms_per_step"])
    if args.accum > 0:
        G = args.accum
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

        a_wall, a_dev, a_t = time_loop(accum_step, 1, max(3, args.steps // 2))
        graphable["accum_clip"] = accum_step
        a_bytes = G * (2 * N + 8) - 4 + 4 + 30  # micro-steps (the first one does not read acc), stats, AdamW
        paths["accum_clip"] = {"micro_steps": G, "max_norm": args.clip, "ms_per_step": a_wall,
                               "device_ms_per_step": a_dev, "events_ms_median": statistics.median(a_t.ms()),
                               "bytes_per_param": a_bytes, "gbps": S * a_bytes / a_dev / 1e6}
    if S <= GRAPH_MAX_ELEMS:
        # launch-bound: the same steps replayed from a HIP graph, 20 per graph
        for name, fn in graphable.items():
            g_ms = graph_time(torch, fn, 20, max(5, args.steps // 20))
            rec = paths.setdefault(name, {"ms_per_step": head["ms_per_step"]})
            rec["graph_ms_per_step"] = g_ms
            rec["graph_speedup_over_eager"] = rec["ms_per_step"] / g_ms
    return paths


def offload_leg(zs, torch, plan, st, hp0, S, args, fused_ms):
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

    wall, dev, t = time_loop(step, 1, 3)
    host_bpp, pcie_bpp = 28, 4
    out = {"ms_per_step": wall, "events_ms_median": statistics.median(t.ms()), "host_threads": threads,
           "chunk_elems": args.offload_chunk, "host_bytes_per_param": host_bpp, "pcie_bytes_per_param": pcie_bpp,
           "host_gbps": S * host_bpp / (wall / 1e3) / 1e9, "pcie_gbps": S * pcie_bpp / (wall / 1e3) / 1e9,
           "slowdown_vs_fused_gpu_step": wall / fused_ms, "pinned_alloc_s": alloc_s}
    del hm, hmm, hv, gh, ph
    return out


def bucketed_workload(zs, synth, torch, wl, args):
    """The Llama-7B shard stepped bucket by bucket (25M owned elements per
    call: 33 full buckets and one of 17,301,952), as the step would run
    behind a bucketed reduce-scatter: the fused step per bucket, and the
    unfused path with the reduce per bucket."""
    N = wl.world
    plan = zs.zs_shard_plan(wl.numels, wl.world, wl.rank, wl.align, zs.ZS_LAYOUT_FLAT)
    S = plan.shard_numel
    B = wl.bucket_elems
    nb = (S + B - 1) // B
    hp0 = zs.AdamWHParams(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, 1)
    log(f"[bench] workload={wl.name}_bucketed N={N} S={S:,} buckets={nb}")
    st = flat_buffers(zs, synth, wl, plan)

    def fused_buckets(t, timer):
        e = timer.start() if timer else None
        for off in range(0, S, B):
            zs.zs_fused_shard_step_bucket(plan, hp0.at(t), st["contribs"], st["master"], st["m"], st["v"], off,
                                          min(B, S - off), full=st["full"])
        if timer:
            timer.stop(e)

    def unfused(t, timer):
        e = timer.start() if timer else None
        for off in range(0, S, B):
            zs.zs_reduce_shard(plan, st["contribs"], st["grad"], off, min(B, S - off))
        zs.zs_adamw_shard_step(plan, hp0.at(t), st["grad"], st["master"], st["m"], st["v"], st["param"])
        zs.zs_gather_params(plan, st["param"], st["full"])
        if timer:
            timer.stop(e)

    wall, dev, t = time_loop(fused_buckets, args.warmup, args.steps)
    ev = t.ms()
    bpp = fused_bpp(N)
    u_wall, u_dev, u_t = time_loop(unfused, 1, max(3, args.steps // 2))
    out = {"workload": f"{wl.name}_n{N}_fused_bucketed", "world_size": N, "rank": wl.rank, "layout": "flat",
           "shard_elems": S, "bucket_elems": B, "buckets": nb, "bytes_per_param": bpp, "ms_per_step": wall,
           "device_ms_per_step": dev, "events_ms_median": statistics.median(ev), "events_ms_p99": p99(ev),
           "params_per_s": S / (wall / 1e3),
           # the step's kernels are the per-bucket launches of k_fused; their
           # average launch covers S / buckets elements
           "roofline": roofline("k_fused", traffic_key(wl, "_bucketed"), S / nb, bpp, dev / nb),
           "paths": {"unfused_bucketed_reduce": {"ms_per_step": u_wall, "device_ms_per_step": u_dev,
                                                 "events_ms_median": statistics.median(u_t.ms()),
                                                 "bytes_per_param": unfused_bpp(N),
                                                 "gbps": S * unfused_bpp(N) / u_dev / 1e6,
                                                 "launches_per_step": nb + 2}}}
    st = None
    release()
    return out


def wrap_workload(zs, synth, torch, wl, args):
    """The Llama-7B shape wrapped per tensor (291 pieces, 65 of them 512-element
    norm pieces), each sharded on its own; the fused multi-tensor step over
    packed arenas and over one allocation per piece and array, and the
    unfused multi-tensor calls."""
    N = wl.world
    plan = zs.zs_shard_plan(wl.numels, wl.world, wl.rank, 1, zs.ZS_LAYOUT_PER_TENSOR)
    S = plan.shard_numel
    hp0 = zs.AdamWHParams(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, 1)
    bpp = fused_bpp(N)
    log(f"[bench] workload={wl.name} N={N} pieces={plan.num_tensors} S={S:,}")
    out = {"workload": f"{wl.name}_n{N}_fused_multi", "world_size": N, "rank": wl.rank, "layout": "per_tensor",
           "pieces": plan.num_tensors, "shard_elems": S, "bytes_per_param": bpp, "paths": {}}
    for packed in (True, False):
        st = per_tensor_buffers(zs, synth, wl, plan, packed=packed)

        def fused(t, timer):
            e = timer.start() if timer else None
            zs.zs_fused_shard_step_multi(plan, hp0.at(t), st["ws_fused"])
            if timer:
                timer.stop(e)

        wall, dev, t = time_loop(fused, args.warmup, args.steps)
        ev = t.ms()
        rec = {"ms_per_step": wall, "device_ms_per_step": dev, "events_ms_median": statistics.median(ev),
               "events_ms_p99": p99(ev), "params_per_s": S / (wall / 1e3),
               "roofline": roofline("k_multi", traffic_key(wl, "" if packed else "_separate"), S, bpp, dev)}
        if packed:
            def unfused(t, timer):
                e = timer.start() if timer else None
                zs.zs_reduce_shard_multi(plan, st["ws"])
                zs.zs_adamw_shard_step_multi(plan, hp0.at(t), st["ws"])
                zs.zs_gather_params_multi(plan, st["ws"])
                if timer:
                    timer.stop(e)

            u_wall, u_dev, u_t = time_loop(unfused, 1, max(3, args.steps // 2))
            out["paths"]["unfused_multi"] = {"ms_per_step": u_wall, "device_ms_per_step": u_dev,
                                             "events_ms_median": statistics.median(u_t.ms()),
                                             "bytes_per_param": unfused_bpp(N),
                                             "gbps": S * unfused_bpp(N) / u_dev / 1e6, "launches_per_step": 3}
            out.update(ms_per_step=wall, params_per_s=S / (wall / 1e3), roofline=rec["roofline"],
                       piece_buffers="carved from one allocation per array at the plan's offsets")
            out["paths"]["fused_multi_packed"] = rec
        else:
            rec["piece_buffers"] = "one allocation per piece and array"
            out["paths"]["fused_multi_separate_allocations"] = rec
        unbind(zs, st)
        fused = unfused = st = None
        release()
    return out


def cpu_baseline(oracle, synth, wl, S, window, bpp):
    """The oracle's shard step timed on this host over a window of the same
    workload (its first `window` owned elements, the same N contributions)."""
    import numpy as np
    n = min(window, S)
    threads = max(1, min(16, os.cpu_count() or 1))
    base, valid = wl.rank * S, sum(wl.numels)
    t0 = time.perf_counter()
    contribs = [synth.cpu_bf16(n, base, wl.contrib_spec(q, 1, valid), threads=threads) for q in range(wl.world)]
    master = synth.cpu_f32(n, base, wl.master_spec(valid), threads=threads)
    gen_s = time.perf_counter() - t0
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    g, p = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    full = np.zeros(n, np.uint16)  # the window's slice of the gathered buffer (rank 0: offset 0)
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
            "sample": f"the first {n:,} owned elements of the {wl.name} shard with all N={wl.world} "
                      f"contributions, median of 5 timed passes after 1 warm-up on {threads} threads, plus one "
                      f"single-thread pass; {cpu_seconds:.1f} core-seconds of oracle work "
                      f"(inputs generated on the host in {gen_s:.1f} s, untimed)",
            "core_seconds": cpu_seconds, "gbps_algorithmic": n * bpp / med / 1e9,
            "single_thread_params_per_s": n / secs1[0]}


def workload(synth, name, world=0):
    """The named workload, cut for `world` ranks when that is nonzero."""
    import dataclasses
    wl = synth.workloads()["llama7b" if name == "llama7b_bucketed" else name]
    if not world or world == wl.world:
        return wl
    return dataclasses.replace(wl, world=world, extra=dict(wl.extra, resized=True))


def traffic_key(wl, suffix=""):
    """The key of the workload's counter-measured traffic; None for a shape
    cut for another world size, which the counters were not taken on."""
    return None if wl.extra.get("resized") else wl.name + suffix


def run_workload(zs, synth, torch, name, args, primary):
    wl = workload(synth, name, args.world if primary else 0)
    try:
        if name == "llama7b_bucketed":
            return bucketed_workload(zs, synth, torch, wl, args)
        if wl.layout == "per_tensor":
            return wrap_workload(zs, synth, torch, wl, args)
        return flat_workload(zs, synth, torch, wl, args, primary)
    except torch.cuda.OutOfMemoryError as e:
        release()
        return {"workload": name, "skipped": f"device memory: {str(e).splitlines()[0]}"}


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

    if args.calib_copy_gib > 0:
        n = int(args.calib_copy_gib * 2**30) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {n * 4:,} bytes read and written per launch, 3 launches")
        del a, b

    if args.world:
        if not 1 <= args.world <= zs.ZS_MAX_CONTRIBS:
            print(f"--world {args.world} is outside 1..{zs.ZS_MAX_CONTRIBS}", file=sys.stderr)
            sys.exit(2)
        args.also = "none"
    head = run_workload(zs, synth, torch, args.workload, args, primary=True)
    if "skipped" in head:
        print(json.dumps({"metric": METRIC, "error": head["skipped"]}), flush=True)
        sys.exit(1)
    others = {}
    for name in ([] if args.also == "none" else [x for x in args.also.split(",") if x and x != args.workload]):
        others[name] = run_workload(zs, synth, torch, name, args, primary=False)
    cpu = None
    if not args.no_cpu:
        import oracle
        wl = workload(synth, args.workload, args.world)
        log(f"[bench] CPU oracle baseline on a {min(args.cpu_window, head['shard_elems']):,}-element window, "
            f"N={wl.world}")
        cpu = cpu_baseline(oracle, synth, wl, head["shard_elems"], args.cpu_window, fused_bpp(wl.world))
    config = {k: head[k] for k in ("workload", "world_size", "rank", "layout", "shard_elems", "bytes_per_param")
              if k in head}
    for k in ("buffer_sets", "bucket_elems", "buckets", "pieces", "piece_buffers"):
        if k in head:
            config[k] = head[k]
    if "median_set" in head:
        config["gathered_buffer"] = head["median_set"]["full_buffer"]
    wall = head["ms_per_step"]
    S = head["shard_elems"]
    out = {
        "metric": METRIC,
        "value": S / (wall / 1e3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded counter-based generator; model shapes only, no weights)",
        "config": config,
        "hbm_gbps": S * head["bytes_per_param"] / wall / 1e6,
        "pct_of_peak": 100.0 * S * head["bytes_per_param"] / wall / 1e6 / HBM_PEAK_GBPS,
        "roofline": head["roofline"],
        "step_roofline": head.get("step_roofline"),
        "cpu_baseline": cpu,
        "placements_ms": head.get("placements"),
        "kernels": head.get("kernels"),
        "paths": head.get("paths"),
        "other_workloads": others,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
