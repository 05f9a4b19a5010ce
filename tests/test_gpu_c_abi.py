"""GPU: the path through the C ABI alone. tests/c_abi/moe_ep_path (plain
C99, the HIP runtime for memory and copies, no torch and no Python) runs
the packs, the receive sides and combine reduces, and the unpacks for W
logical ranks with identity experts (an expert's output rows are its
batched input rows). Its counts, token slots, expert_num_tokens, error
flags and combined rows must be the oracle's, bit for bit."""
import subprocess

import numpy as np
import pytest

import oracle
import workloads as wl
from parity import say
from c_abi_io import program, read_outputs, write_inputs

pytestmark = pytest.mark.gpu

W1 = wl.WORKLOADS[1]
CASES = {
    "tiny": W1,
    "one_tile": W1.scaled(W=8, E=64, K=6, T=200, cap=220, H=128, pad_frac=0.05),
    "several_tiles": W1.scaled(W=4, E=32, K=4, T=700, cap=700, H=64),
    "w1": W1.scaled(W=1, E=8, K=2, T=90, cap=96, H=64),
    "empty": W1.scaled(T=0, cap=16),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_c_program_runs_the_path(name, tmp_path):
    exe = program()
    w = CASES[name]
    srcs = [wl.routing(w, s, 31) for s in range(w.W)]
    hid = [wl.hidden_bf16(w, s, 31) for s in range(w.W)]
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    write_inputs(inp, w, srcs, hid)
    say(f"[c abi] {name}: T={w.T} H={w.H} E={w.E} K={w.K} W={w.W} cap={w.cap}")
    r = subprocess.run([exe, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    got = read_outputs(outp, w)

    def identity(dest, batch):
        b = batch["b"][0]
        return b.view(np.uint16).reshape(w.e_local, b.shape[1], w.H)

    ref = oracle.run_path([s[0] for s in srcs], [s[1] for s in srcs],
                          [[h.view(np.uint8).reshape(w.T, 2 * w.H)] for h in hid],
                          w.E, w.W, w.cap, identity)
    for s in range(w.W):
        assert np.array_equal(got["send_cnt"][s], ref["packs"][s]["send_cnt"]), f"send_cnt {s}"
        assert np.array_equal(got["token_slot"][s], ref["packs"][s]["token_slot"]), f"slots {s}"
        assert np.array_equal(got["out"][s], ref["outs"][s].reshape(w.T, w.H)), f"out {s}"
    for r_ in range(w.W):
        assert np.array_equal(got["expert_num_tokens"][r_],
                              ref["batches"][r_]["expert_num_tokens"]), f"expert_num_tokens {r_}"
    err = 0
    for p in ref["packs"]:
        err |= p["err"]
    for b in ref["batches"]:
        err |= b["err"]
    assert got["err"] == err
