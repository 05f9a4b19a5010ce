"""Builds the CPU oracle shared library with gcc (host only, no HIP).

Test infrastructure: see the header of moe_ep_oracle.c.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_ep_oracle.c")
LIB = os.path.join(HERE, "liboracle_moe_ep.so")

CFLAGS = ["-O2", "-std=c99", "-Wall", "-Wextra", "-ffp-contract=off",
          "-fno-fast-math", "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
