"""Builds the synthetic-input generator: host build with gcc, GPU build with hipcc."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_cpu(verbose=False):
    out = os.path.join(HERE, "libsynth_cpu.so")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-Wall",
           "-o", out + ".tmp", os.path.join(HERE, "synth_cpu.c")]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build_gpu(verbose=False):
    out = os.path.join(HERE, "libsynth_gpu.so")
    cmd = ["hipcc", *HIP_FLAGS, "-o", out + ".tmp", os.path.join(HERE, "synth_gpu.hip")]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(verbose=False):
    return [build_cpu(verbose), build_gpu(verbose)]


if __name__ == "__main__":
    build(verbose=True)
