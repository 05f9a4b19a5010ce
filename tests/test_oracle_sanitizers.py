"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The C oracle is rebuilt with both sanitizers (host code, gcc, the same
floating-point flags as its normal build) and the oracle's pin tests run
against that build in a child process with the sanitizer runtimes preloaded
(oracle.use_library routes every call through it). An out-of-bounds or
use-after-free access, a signed overflow, a bad shift or a misaligned access
anywhere the pins reach aborts the child and fails this test."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PIN_FILES = ["test_oracle_pins.py", "test_oracle_fp8.py", "test_oracle_fp4.py",
             "test_oracle_sanitize.py"]


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    lib = tmp_path / "liboracle_moe_ep_sanitized.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-Wall", "-Wextra", "-ffp-contract=off",
                    "-fno-fast-math", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    "-o", str(lib), os.path.join(ROOT, "oracle", "moe_ep_oracle.c"), "-lm"],
                   check=True)
    files = [os.path.join(HERE, f) for f in PIN_FILES]
    driver = ("import sys, pytest, oracle\n"
              f"with oracle.use_library({str(lib)!r}):\n"
              f"    sys.exit(pytest.main({files!r} + ['-q', '-s', '-x', '-m', 'not gpu',"
              " '-p', 'no:cacheprovider']))\n")
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               PYTHONPATH=os.pathsep.join([ROOT, HERE]))
    r = subprocess.run([sys.executable, "-c", driver], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    if r.returncode != 0 or "passed" not in r.stdout or "Sanitizer" in r.stderr:
        # the sanitizer's report from its first line (its stack runs on into
        # the interpreter's frames)
        at = [i for i in (r.stderr.find("ERROR: AddressSanitizer"),
                          r.stderr.find("runtime error")) if i >= 0]
        report = r.stderr[min(at):min(at) + 3000] if at else r.stderr[-3000:]
        pytest.fail("the pins failed on the sanitized oracle:\n" + r.stdout[-2000:] + "\n"
                    + report, pytrace=False)
