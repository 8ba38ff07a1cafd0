"""Builds the shard-step library libzs.so for gfx950, in-tree.

Host code (plan, validation, the host AdamW of the offloaded step) is C++17;
kernels and the offload pipeline are HIP compiled for gfx950. Everything is
built with contraction off (the element arithmetic must round operation by
operation); HIP code also with packed-fp32 instruction generation disabled.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libzs.so")
BUILD = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-ffp-contract=off", "-Wall", "-Wextra", f"-I{INCLUDE}"]
HIP_ONLY = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{err}")
    if err.strip() and verbose:
        print(err)


def build(verbose=False, out=None):
    """Builds libzs.so (or ``out``)."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    api_o = os.path.join(BUILD, "zs_api.o")
    _run(["g++", *COMMON, "-c", os.path.join(CSRC, "zs_api.cpp"), "-o", api_o], verbose)
    objs.append(api_o)
    host_o = os.path.join(BUILD, "zs_host_adamw.o")
    # host AdamW: same one-rounding-per-operation rule; -fno-math-errno lets
    # sqrtf become the (correctly rounded) vector instruction
    _run(["g++", *COMMON, "-fno-math-errno", "-pthread", "-c", os.path.join(CSRC, "zs_host_adamw.cpp"), "-o",
          host_o], verbose)
    objs.append(host_o)
    for name in ("zs_kernels", "zs_offload"):
        o = os.path.join(BUILD, f"{name}.o")
        _run([HIPCC, *COMMON, *HIP_ONLY, "-c", os.path.join(CSRC, f"{name}.hip"), "-o", o], verbose)
        objs.append(o)
    target = out or LIB
    tmp = target + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp, *objs], verbose)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
