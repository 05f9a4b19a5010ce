"""GPU parity on seeded random shapes: world sizes, local expert counts and
hidden sizes that are not powers of two, K above and below e_local, cap
above T, partial padding, skewed routing, and every form of the path
(plain, fp32 combine, fp8 and fp4 quantize-on-pack, fused local combine),
each with the receive side's own scan and, in every other group of five
cases, with the senders' per-expert ranks, compared element by element
with the oracle. A second set takes the senders' ranks over wider shapes:
up to 16 picks per token (the form's limit), up to about 1,500 tokens
(several routing tiles) and up to 4,096 experts."""
import numpy as np
import pytest

import workloads as wl
from parity import run_full_parity, say

pytestmark = pytest.mark.gpu

N_CASES = 60


def _case(i):
    rng = np.random.default_rng(9000 + i)
    W = int(rng.choice([1, 2, 3, 5, 8, 13, 32, 64]))
    e_local = int(rng.choice([1, 2, 3, 5, 8, 12, 32, 100]))
    while W * e_local > 1024:
        e_local = max(1, e_local // 2)
    E = W * e_local
    K = int(rng.integers(1, min(E, 10) + 1))
    T = int(rng.integers(0, 400))
    cap = T + int(rng.integers(0, 50))
    mode = ["plain", "f32", "fp8", "fp4", "fused"][i % 5]
    ranked = (i // 5) % 2 == 1
    # bf16 rows are 16-byte multiples (H % 8); the quantised rows need more
    H = int(rng.choice([32, 96, 256, 544, 1024])) if mode in ("fp8", "fp4") \
        else int(rng.choice([8, 24, 64, 120, 256, 1000]))
    if mode == "fp8":
        H = H // 32 * 32
    routing = "zipf" if rng.random() < 0.4 else "uniform"
    w = wl.WORKLOADS[1].scaled(T=T, H=H, E=E, K=K, W=W, cap=cap, routing=routing,
                               zipf_s=1.1 if routing == "zipf" else 0.0,
                               pad_frac=float(rng.choice([0.0, 0.05, 0.3])))
    return w, mode, ranked


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_parity(i):
    w, mode, ranked = _case(i)
    say(f"[random {i}] {mode}{' ranked' if ranked else ''} T={w.T} H={w.H} E={w.E} K={w.K} "
        f"W={w.W} cap={w.cap} {w.routing} pad={w.pad_frac}")
    kw = {"ranked": ranked}
    if mode == "f32":
        kw["f32"] = True
    elif mode == "fp8":
        kw["fp8_group"] = 32 if w.H % 64 else 64
    elif mode == "fp4":
        kw["fp4"] = True
    elif mode == "fused":
        kw["fused_local"] = True
    run_full_parity(w, salt=100 + i, **kw)


N_WIDE = 16


def _wide_case(i):
    rng = np.random.default_rng(77000 + i)
    while True:
        W = int(rng.choice([1, 2, 3, 5, 8, 13, 32, 64]))
        e_local = int(rng.choice([1, 2, 3, 5, 8, 12, 32, 100, 300]))
        E = W * e_local
        if E > 4096:
            continue
        K = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.integers(0, 1500))
        cap = T + int(rng.integers(0, 50))
        mode = ["plain", "fused", "fp8", "fp4"][i % 4]
        H = int(rng.choice([32, 96, 256])) if mode in ("fp8", "fp4") \
            else int(rng.choice([8, 24, 64, 120, 256]))
        # keep the send and expert-batch buffers small
        if W * W * max(cap, 1) * 2 * H > (1 << 30) or E * W * max(cap, 1) * 2 * H > (1 << 31):
            continue
        routing = "zipf" if rng.random() < 0.4 else "uniform"
        w = wl.WORKLOADS[1].scaled(T=T, H=H, E=E, K=K, W=W, cap=cap, routing=routing,
                                   zipf_s=1.1 if routing == "zipf" else 0.0,
                                   pad_frac=float(rng.choice([0.0, 0.05, 0.3])))
        return w, mode


@pytest.mark.parametrize("i", range(N_WIDE))
def test_random_wide_ranked_parity(i):
    w, mode = _wide_case(i)
    say(f"[random wide {i}] {mode} ranked T={w.T} H={w.H} E={w.E} K={w.K} W={w.W} "
        f"cap={w.cap} {w.routing} pad={w.pad_frac}")
    kw = {"ranked": True}
    if mode == "fp8":
        kw["fp8_group"] = 32 if w.H % 64 else 64
    elif mode == "fp4":
        kw["fp4"] = True
    elif mode == "fused":
        kw["fused_local"] = True
    run_full_parity(w, salt=500 + i, **kw)
