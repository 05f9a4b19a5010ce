"""Builds libmoe_ep.so (the HIP kernels and the C ABI) for gfx950 in-tree,
and beside it libmoe_ep_probe.so (the HBM stream probes of
`bench.py --probe stream`; measurement tooling, not part of the path).

    python -m combine_topk_ids_dest_amd.build [-v]
"""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_ep.so")
PROBE_SRC = os.path.join(PKG, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(PKG, "libmoe_ep_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # products are rounded to fp32 before they are added: no contraction
    "-ffp-contract=off",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(srcs, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _compile(sources(), LIB, verbose)
    _compile([PROBE_SRC], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
