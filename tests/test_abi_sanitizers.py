"""The host code of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer.

libmoe_ep.so is rebuilt with both sanitizers on its host code only (hipcc,
each flag after -Xarch_host; the gfx950 device code is built as usual) and
the ABI tests (symbols, capacities, workspace sizes, status strings and the
argument checks of every entry point, none of which launches a kernel) run
against it in a child process with clang's sanitizer runtime preloaded."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


def _asan_runtime():
    if not os.path.exists(CLANG):
        return None
    res = subprocess.run([CLANG, "--print-resource-dir"], capture_output=True,
                         text=True).stdout.strip()
    p = os.path.join(res, "lib", "linux", "libclang_rt.asan-x86_64.so")
    return p if os.path.exists(p) else None


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if not os.path.exists(HIPCC) or rt is None:
        pytest.skip("hipcc or clang's sanitizer runtime is not installed")
    from combine_topk_ids_dest_amd import build as hip_build
    lib = str(tmp_path / "libmoe_ep_sanitized.so")
    flags = [f for f in hip_build.FLAGS if f != "-O3"] + ["-O1", "-g"]
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer"):
        flags += ["-Xarch_host", f]
    subprocess.run([HIPCC, *flags, "-shared-libsan", "-I", hip_build.INCLUDE,
                    "-I", hip_build.CSRC, *hip_build.sources(), "-o", lib],
                   check=True, capture_output=True)
    driver = ("import sys, pytest\n"
              "from combine_topk_ids_dest_amd import binding\n"
              f"binding.LIB_PATH = {lib!r}\n"
              f"rc = pytest.main([{os.path.join(HERE, 'test_abi.py')!r}, '-q', '-s', '-x',"
              " '-m', 'not gpu', '-p', 'no:cacheprovider'])\n"
              "loaded = [l.split()[-1] for l in open('/proc/self/maps') if 'moe_ep' in l]\n"
              f"assert {lib!r} in loaded, loaded\n"
              "sys.exit(rc)\n")
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               PYTHONPATH=os.pathsep.join([ROOT, HERE]))
    r = subprocess.run([sys.executable, "-c", driver], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    if r.returncode != 0 or "passed" not in r.stdout or "Sanitizer" in r.stderr:
        at = [i for i in (r.stderr.find("ERROR: AddressSanitizer"),
                          r.stderr.find("runtime error")) if i >= 0]
        report = r.stderr[min(at):min(at) + 3000] if at else r.stderr[-3000:]
        pytest.fail("the ABI tests failed on the sanitized library:\n" + r.stdout[-2000:]
                    + "\n" + report, pytrace=False)
