"""Compile the oracle (plain C, fp64, OpenMP) into ``oracle/libngv_oracle.so``.

Test infrastructure only. ``-ffp-contract=off`` keeps every product and sum
rounded as written (no fused multiply-add), so the oracle's rounding follows
its source.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ngv_oracle.c")
LIB = os.path.join(HERE, "libngv_oracle.so")


def build_oracle(verbose=False):
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-fvisibility=hidden", "-Wall", "-Wextra", "-Wno-unused-parameter",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build_oracle(verbose=True)
    sys.exit(0)
