"""The C ABI used from a plain C11 program (``tests/c_abi/zs_c_step.c``): no
Python and no torch in that process. The CPU tests check that the public
header is valid pedantic C11 and C++17 on its own and that the program links and loads
the in-tree library; the GPU test runs three steps through the program (the
fused call, the unfused calls, and the fused call with device-resident
scalars), over FLAT plans and over a PER_TENSOR plan through the multi-tensor
calls, and compares every output byte with the oracle."""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

from gpu_util import check_bf16, check_f32

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "c_abi")
EXE = os.path.join(HERE, "_build", "zs_c_step")

needs_gcc = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


def _exe():
    if not os.path.exists(EXE):
        import importlib.util
        spec = importlib.util.spec_from_file_location("zs_c_build", os.path.join(HERE, "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return EXE


@needs_gcc
@pytest.mark.parametrize("lang", ["c11", "c++17"])
def test_header_is_pedantic(tmp_path, lang):
    src = tmp_path / ("h.c" if lang == "c11" else "h.cpp")
    src.write_text('#include "zs.h"\nint main(void) { zs_status s = ZS_OK; return (int)s; }\n')
    cc = "gcc" if lang == "c11" else "g++"
    res = subprocess.run([cc, f"-std={lang}", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                          f"-I{os.path.join(ROOT, 'include')}", str(src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


@needs_gcc
def test_program_links_the_library():
    import fsdp_sharded_mixed_flatten_amd as zs
    res = subprocess.run([_exe()], capture_output=True, text=True, timeout=60)
    assert res.returncode == 2, res.stderr
    assert f"library {zs.zs_version()}" in res.stderr


CASES = [
    # numels, world, rank, align, layout
    ([4093, 77, 1000], 4, 3, 8, "flat"),        # the last rank owns every padding gap
    ([1_000_003], 8, 5, 1, "flat"),             # one ragged tensor, several tiles
    ([70_000, 3, 4_608], 64, 17, 128, "flat"),  # the two-pass form of the fused call
    ([300_007, 64], 24, 23, 8, "flat"),         # the runtime rank loop (three groups of 8)
    ([4093, 77, 1000, 65_536, 5], 8, 6, 1, "per_tensor"),  # multi-tensor pieces with per-tensor padding
    ([4093, 77, 1000, 65_536, 5], 52, 40, 1, "per_tensor"),  # the two-launch multi-tensor step
]


@pytest.mark.gpu
@pytest.mark.parametrize("numels,world,rank,align,layout", CASES,
                         ids=["n4", "n8", "n64", "n24", "per_tensor_n8", "per_tensor_n52"])
def test_c_program_matches_oracle(tmp_path, ora, syn, numels, world, rank, align, layout):
    from oracle.plan import plan_flat, plan_per_tensor
    steps = 3
    flat = layout == "flat"
    plan = plan_flat(numels, world, rank, align) if flat else plan_per_tensor(numels, world, rank)
    T, S = plan.T, plan.S
    pad = np.frombuffer(bytes(plan.padding_mask_full()), dtype=np.uint8).astype(bool)
    # owned positions of the packed gathered buffer, in shard order
    own = (np.arange(rank * S, rank * S + S) if flat else
           np.concatenate([np.arange(pc.full_off, pc.full_off + pc.own_hi - pc.own_lo) for pc in plan.pieces]))
    assert own.size == S
    seed = 4242 + world
    hp = (1e-3, 0.9, 0.95, 1e-8, 0.1)
    master0 = syn.cpu_f32(T, 0, syn.spec(seed, syn.STREAM_MASTER, 0, 0.02))
    master0[pad] = 0
    contribs = []  # [step][rank] owned elements in shard order
    for t in range(1, steps + 1):
        row = []
        for q in range(world):
            c = syn.cpu_bf16(T, 0, syn.spec(seed, syn.STREAM_CONTRIB + q, t, 1e-3))
            c[pad] = 0
            row.append(c[own].copy())
        contribs.append(row)

    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(struct.pack("<7q", len(numels), world, rank, align, steps, S, 0 if flat else 1))
        f.write(struct.pack(f"<{len(numels)}q", *numels))
        f.write(struct.pack("<5d", *hp))
        for row in contribs:
            for c in row:
                f.write(c.astype("<u2").tobytes())
        f.write(master0[own].astype("<f4").tobytes())
    print(f"[c-abi] {layout} world={world} rank={rank} T={T} S={S}", flush=True)
    res = subprocess.run([_exe(), str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, f"rc={res.returncode}\nstdout:\n{res.stdout}\nstderr:\n{res.stderr}"
    assert "expected error:" in res.stdout and "rank" in res.stdout, res.stdout

    raw = out.read_bytes()
    t_out, s_out = struct.unpack_from("<2q", raw, 0)
    assert (t_out, s_out) == (T, S)
    pos = 16

    def take(dtype, n):
        nonlocal pos
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=pos).copy()
        pos += a.nbytes
        return a

    got = {k: take("<f4", S) for k in ("master", "m", "v")}
    got.update(grad=take("<u2", S), param=take("<u2", S), full=take("<u2", T))
    assert pos == len(raw)

    g = np.zeros(S, np.uint16)
    mst = master0[own].copy()
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    p = np.zeros(S, np.uint16)
    full = np.full(T, 0x5A5A, np.uint16)
    for t in range(1, steps + 1):
        ohp = ora.HParams(*hp, t)
        if flat:
            ora.shard_step(ohp, contribs[t - 1], g, mst, m, v, p, full, rank)
        else:
            # the pieces are views into the shard arrays, and the gathered
            # tensors views into the packed buffer
            sl = [slice(pc.shard_off, pc.shard_off + (pc.own_hi - pc.own_lo)) for pc in plan.pieces]
            ora.plan_step(plan, ohp, [[c[k] for c in contribs[t - 1]] for k in sl],
                          [(g[k], mst[k], m[k], v[k], p[k]) for k in sl],
                          [full[o:o + n] for o, n in zip(plan.offsets, plan.padded)])

    nd = check_f32(got["master"], mst, "master") + check_f32(got["m"], m, "m") + check_f32(got["v"], v, "v")
    nd += check_bf16(got["grad"], g, "grad") + check_bf16(got["param"], p, "param")
    nd += check_bf16(got["full"], full, "full")
    assert nd == 0, f"{nd} elements not bit-identical"
