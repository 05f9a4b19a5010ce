"""CPU: the plain-C program of tests/c_abi builds against the header and the
library with -Wall -Wextra -Werror, checks its arguments, and reports a
status from the library's host checks by name (moe_ep_capacities rejects
E % W != 0 before any device call)."""
import subprocess

import numpy as np

import workloads as wl
from c_abi_io import program as _exe, write_inputs


def test_usage_without_arguments():
    r = subprocess.run([_exe()], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr


def test_library_status_reaches_the_caller(tmp_path):
    w = wl.WORKLOADS[1]
    inp = tmp_path / "in.bin"
    write_inputs(inp, w, [], [], header=(w.T, w.H, 9, w.K, 4, w.cap))   # E % W != 0
    r = subprocess.run([_exe(), str(inp), str(tmp_path / "out.bin")],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 1
    assert "moe_ep_capacities" in r.stderr and "invalid" in r.stderr.lower()
    assert not (tmp_path / "out.bin").exists()
