"""Builds the oracle's C part into oracle/libzs_oracle.so with gcc.

-O2 without fast-math and with -ffp-contract=off: every fp32 operation in the
oracle is rounded on its own, in source order.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zs_oracle.c")
LIB = os.path.join(HERE, "libzs_oracle.so")


def build(verbose=False):
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
