"""Builds tests/c_abi/moe_ep_path: the whole path through the C ABI alone
(moe_ep_path.c, plain C99 compiled by gcc, linked against libmoe_ep.so and
the HIP runtime, no torch). Needs the library built first; __graft_entry__
build() runs this after it."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "combine_topk_ids_dest_amd")
SRC = os.path.join(HERE, "moe_ep_path.c")
EXE = os.path.join(HERE, "moe_ep_path")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    if not os.path.exists(os.path.join(PKG, "libmoe_ep.so")):
        raise RuntimeError("libmoe_ep.so is not built: run the package build first")
    tmp = EXE + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", PKG, "-lmoe_ep", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../combine_topk_ids_dest_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
