"""Builds ``zs_c_step`` (a plain C11 program that runs shard steps through
the C ABI alone, with the HIP runtime's C API for memory and the stream) into
``tests/c_abi/_build/``. It links the in-tree ``libzs.so`` through a relative
run path, so the binary keeps working wherever the repository is copied."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "fsdp_sharded_mixed_flatten_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "_build", "zs_c_step")


def build(verbose=False):
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-D__HIP_PLATFORM_AMD__",  # selects the AMD runtime in the HIP headers
           f"-I{os.path.join(ROOT, 'include')}", "-isystem", os.path.join(ROCM, "include"),
           os.path.join(HERE, "zs_c_step.c"), "-o", EXE + ".tmp",
           f"-L{PKG}", "-lzs", "-Wl,-rpath,$ORIGIN/../../../fsdp_sharded_mixed_flatten_amd",
           f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
