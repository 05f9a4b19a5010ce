#!/usr/bin/env python3
"""Throughput of the MoE expert-parallel dispatch/combine layout transform on
one MI355X.

A step is one pass of the whole path over W logical ranks with synthetic,
seeded inputs already resident in HBM: W dispatch packs, then for every
destination the expert batch and the combine reduce, then W combine
unpacks. The ranks are spread over --lanes HIP streams (2, or 1 for a tiny
step), so the kernels of one rank overlap those of another, as they would on
W GPUs; each phase waits for the previous one on every stream. `value` is
tokens/s over all W*T tokens of a step; effective GB/s
uses the algorithmic byte model (what the method must read and write, from
the run's actual counts):

  pack (source s)      8*T*K + T_routed*P + U*P + U*slots*8 + 4*W
  batch (dest r)       4*W + S*slots*4 + S*P + R*P + 4*e_local
  reduce (dest r)      R*Hb + S*slots*8 + S*Hb
  unpack (source s)    U*Hb + T*Hb

with P = payload bytes per token row, Hb = combine row bytes, U = slots a
source sends, S = slots a destination receives, R = expert rows it batches.
With --fused-local the local slice (source s = destination r, S_own slots
with R_own expert rows) leaves the reduce and enters the fused unpack:

  reduce_peers (dest r)   (R - R_own)*Hb + (S - S_own)*(slots*8 + Hb)
  unpack_fused (source s) (U - S_own)*Hb + R_own*Hb + S_own*slots*8 + T*Hb

With the sender-ranked receive side (--receive ranked, and --receive auto
when T <= 256) the pack also writes each used slot's ranks and the counts
per expert, and the receive side reads those instead of scanning:

  pack (source s)      ... + U*slots*4 + 4*E
  batch (dest r)       4*W + S*slots*8 + 4*E + S*P + R*P + 4*e_local

Besides the contract fields the line carries: per-call times (a separate
pass with HIP events around each call; averages, which the roofline uses,
and medians), the whole step with every call on one stream, the time per
rank share, the critical-path rate (T over the slowest rank's share, which
sets the pace under skewed routing), the dispatch and combine split, the
same calls timed cold (each after a 1 GiB device write that evicts the
256 MB last-level cache) together with whole cold steps over the lanes,
and the rate of the runtime's own 1 GiB device copy in the same session as
a second roofline. The roofline object is that of the call with the most
kernel time among the calls that move rows (the receive plan moves index
data only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]
                       [--receive auto|scan|ranked] [--fp8-group G | --fp4] [--fused-local]
"""
import argparse
import gc
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine tokens/s and effective HBM GB/s (% of peak), 1 MI355X"
PEAK_HBM_GBPS = 8000.0
# Calls timed one by one in the per-call pass, with the kernel that moves
# the rows in each (moe_ep_expert_batch is timed as its two halves).
KERNEL_OF_CALL = {
    "pack": "pack_copy_kernel",
    "batch": "batch_copy_kernel",
    "batch_plan": "batch_local_kernel",
    "batch_copy": "batch_copy_kernel",
    "reduce": "combine_reduce_kernel",
    "unpack": "combine_unpack_kernel",
    "reduce_peers": "combine_reduce_kernel",
    "unpack_fused": "combine_unpack_fused_kernel",
}
ABI_OF_CALL = {
    "pack": "moe_ep_dispatch_pack",
    "batch": "moe_ep_expert_batch_ranked",
    "batch_plan": "moe_ep_expert_batch_plan",
    "batch_copy": "moe_ep_expert_batch_copy",
    "reduce": "moe_ep_combine_reduce",
    "unpack": "moe_ep_combine_unpack",
    "reduce_peers": "moe_ep_combine_reduce_peers",
    "unpack_fused": "moe_ep_combine_unpack_fused",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The source file of each kernel; with the shared header and the build
# flags it determines the kernel's code.
KERNEL_SOURCE = {
    "route_local_kernel": "route.hip",
    "column_scan_kernel": "route.hip",
    "pack_copy_kernel": "pack.hip",
    "batch_local_kernel": "batch.hip",
    "batch_copy_kernel": "batch.hip",
    "sanitize_ids_kernel": "batch.hip",
    "combine_reduce_kernel": "combine.hip",
    "combine_unpack_kernel": "combine.hip",
    "combine_unpack_fused_kernel": "combine.hip",
}


def source_digest(kernel: str) -> str:
    """sha256 over the kernel's source file, the shared header and the build
    script: a counter summary taken from an older build of the kernel no
    longer describes it."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "combine_topk_ids_dest_amd")
    for f in (os.path.join(pkg, "csrc", KERNEL_SOURCE[kernel]),
              os.path.join(pkg, "csrc", "common.h"), os.path.join(pkg, "build.py")):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<kernel>.<workload>.pmc.txt, or None when it is absent or was
    taken on other sources of the kernel."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_digest(kernel):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# Largest batch per source for which --receive auto takes the sender-ranked
# receive side: one routing tile, where the pack counts the ranks itself
# (measured faster there: decode 0.94 against 1.02 ms per step, tiny 0.132
# against 0.139 ms; at the larger shapes within -2 % to +1 %).
RANKED_MAX_T = 256


# The sender-ranked form's limits (the library returns EINVAL beyond them).
RANKED_MAX_K = 16
RANKED_MAX_E = 4096


def roofline_call(total_ms):
    """The call whose HBM roofline the line reports: the one with the most
    kernel time among the calls that move rows. The receive plan moves index
    data only (it is latency bound), so it is not a candidate."""
    moving = {k: t for k, t in total_ms.items() if k != "batch_plan"} or total_ms
    return max(moving, key=moving.get)


def receive_ranked(receive: str, T: int, K: int = 1, E: int = 1) -> bool:
    """Whether the step uses the sender-ranked receive side (--receive):
    always for "ranked"; for "auto" when the batch is one routing tile and
    the shape is within the form's limits."""
    if receive == "ranked":
        return True
    return receive == "auto" and T <= RANKED_MAX_T and K <= RANKED_MAX_K and E <= RANKED_MAX_E


def mode_suffix(args) -> str:
    """The part of a counter summary's name that tells the dispatch format
    and the receive form: the counters of one form do not describe another."""
    s = ""
    if args.fp8_group:
        s += f"_fp8_g{args.fp8_group}"
    if args.fp4:
        s += "_fp4"
    if args.fused_local:
        s += "_fused_local"
    if args.ranked:
        s += "_ranked"
    return s


def byte_model(w, row_bytes, slots, send_cnt, ent, routed, send_row_bytes=None,
               r_own=None, ranked=False):
    """Algorithmic bytes per call kind (lists over ranks). row_bytes: the
    source rows a pack reads; send_row_bytes: the rows that travel (the
    same unless the pack quantises); r_own[s]: expert rows of rank s's
    local slice (for the fused combine). ranked: the packs also write each
    used slot's per-expert ranks and the counts per expert, and the receive
    side ("batch") reads those instead of scanning."""
    import numpy as np
    P_src = int(sum(row_bytes))
    P = int(sum(send_row_bytes if send_row_bytes is not None else row_bytes))
    Hb = w.H * 2
    U = send_cnt.sum(axis=1)            # per source
    S = send_cnt.sum(axis=0)            # per destination
    R = ent.sum(axis=1)                 # per destination
    pack = [8 * w.T * w.K + int(routed[s]) * P_src + int(U[s]) * P + int(U[s]) * slots * 8
            + 4 * w.W for s in range(w.W)]
    batch_plan = [4 * w.W + int(S[r]) * slots * 4 + 4 * w.e_local for r in range(w.W)]
    batch_copy = [int(S[r]) * P + int(R[r]) * P for r in range(w.W)]
    reduce = [int(R[r]) * Hb + int(S[r]) * slots * 8 + int(S[r]) * Hb for r in range(w.W)]
    unpack = [int(U[s]) * Hb + w.T * Hb for s in range(w.W)]
    out = {"pack": pack, "batch_plan": batch_plan, "batch_copy": batch_copy,
           "reduce": reduce, "unpack": unpack, "U": U, "S": S, "R": R}
    if ranked:
        out["pack"] = [pack[s] + int(U[s]) * slots * 4 + 4 * w.E for s in range(w.W)]
        out["batch"] = [4 * w.W + int(S[r]) * slots * 8 + 4 * w.E + int(S[r]) * P
                        + int(R[r]) * P + 4 * w.e_local for r in range(w.W)]
    if r_own is not None:
        S_own = [int(send_cnt[s, s]) for s in range(w.W)]
        out["reduce_peers"] = [(int(R[r]) - int(r_own[r])) * Hb
                               + (int(S[r]) - S_own[r]) * (slots * 8 + Hb)
                               for r in range(w.W)]
        out["unpack_fused"] = [(int(U[s]) - S_own[s]) * Hb + int(r_own[s]) * Hb
                               + S_own[s] * slots * 8 + w.T * Hb for s in range(w.W)]
    return out


# Device memory the lanes' expert-batch and expert-output buffers may take
# together.
LANE_MEMORY_BYTES = 160 << 30
# Two lanes measured fastest at every shape with more than one lane's worth
# of work: with the ranks over 1, 2, 3 and 4 streams the DS-V3 step took
# 3.30, 3.24, 3.40 and 3.38 ms, Mixtral 1.39, 1.35, - and 1.38 ms, decode
# 1.40, 0.98, 0.99 and 1.12 ms.
AUTO_LANES = 2
AUTO_LANES_MIN_BYTES = 16 << 20


def lanes_that_fit(w, row_bytes, fp8_group, fp4, want: int) -> int:
    """Lanes to use: at most `want` and W, and no more than fit their
    [e_local, W*cap, row] expert-batch and [e_local, W*cap, H] bf16
    expert-output buffers in LANE_MEMORY_BYTES."""
    from combine_topk_ids_dest_amd import binding
    rows = list(row_bytes)
    if fp4:
        rows = [w.H // 2, binding.fp4_scale_pitch(w.H)] + rows[1:]
    elif fp8_group:
        rows = [w.H, 4 * binding.scale_pitch(w.H, fp8_group)] + rows[1:]
    per_lane = w.e_local * w.W * w.cap * (sum(rows) + 2 * w.H)
    return max(1, min(want, w.W, LANE_MEMORY_BYTES // max(per_lane, 1)))


def auto_lanes(w, row_bytes, fp8_group=None, fp4=False) -> int:
    """The lanes of --lanes auto."""
    want = AUTO_LANES if w.W * w.T * sum(row_bytes) >= AUTO_LANES_MIN_BYTES else 1
    return lanes_that_fit(w, row_bytes, fp8_group, fp4, want)


def cpu_baseline(w, srcs, pls, shares: int):
    """The CPU oracle, as it stands, timed on this host: `shares` logical-rank
    shares (pack of a source, batch and reduce of a destination, unpack of a
    source), single-threaded."""
    import numpy as np
    import oracle
    K = w.K
    t_setup = time.perf_counter()
    packs = [oracle.dispatch_pack(srcs[s][0], srcs[s][1], w.E, w.W, w.cap, pls[s])
             for s in range(w.W)]
    log(f"[cpu_baseline] oracle packs of {w.W} sources for the sample: "
        f"{time.perf_counter() - t_setup:.1f} s")
    times = []
    nbytes = 0
    for i in range(shares):
        s = r = i % w.W
        t0 = time.perf_counter()
        p = oracle.dispatch_pack(srcs[s][0], srcs[s][1], w.E, w.W, w.cap, pls[s])
        t1 = time.perf_counter()
        cnt = np.ascontiguousarray(np.stack([q["send_cnt"][r] for q in packs]))
        eloc = np.ascontiguousarray(np.stack([q["send_eloc"][r] for q in packs]))
        wts = np.ascontiguousarray(np.stack([q["send_w"][r] for q in packs]))
        recv = [oracle.stack_ranks([q["send"][j][r] for q in packs])
                for j in range(len(pls[0]))]
        t2 = time.perf_counter()
        b = oracle.expert_batch(cnt, eloc, w.W, w.e_local, K, w.cap, recv)
        t3 = time.perf_counter()
        Y = b["b"][0].view(np.uint16).reshape(w.e_local, -1, w.H)    # identity experts
        ret = oracle.combine_reduce(Y, cnt, eloc, wts, b["recv_row"], w.W,
                                    w.e_local, K, w.cap)["ret"]
        t4 = time.perf_counter()
        rows = int(p["send_cnt"].max(initial=0))
        a1 = pls[s][0].view(np.uint16).reshape(w.T, w.H)
        back = np.empty((w.W, rows, w.H), np.uint16)
        for d in range(w.W):
            back[d] = a1[:rows] if rows <= w.T else 0
        t5 = time.perf_counter()
        oracle.combine_unpack(back, p["token_slot"])
        t6 = time.perf_counter()
        times.append((t1 - t0) + (t3 - t2) + (t4 - t3) + (t6 - t5))
        P = sum(x.shape[1] for x in pls[s])
        U = int(p["send_cnt"].sum())
        S = int(cnt.sum())
        R = int(b["expert_num_tokens"].sum())
        routed = int((srcs[s][0] >= 0).any(axis=1).sum())
        slots = p["slots"]
        nbytes += (8 * w.T * K + routed * P + U * P + U * slots * 8 + S * slots * 4 + S * P
                   + R * P + R * w.H * 2 + S * slots * 8 + S * w.H * 2 + U * w.H * 2
                   + w.T * w.H * 2)
        del b, ret, back
    total = sum(times)
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": shares * w.T / total,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{shares} logical-rank share(s) of {w.name}: pack of a source, batch and "
                   f"reduce of a destination (identity experts), unpack of a source; "
                   f"{total:.2f} s on 1 of {os.cpu_count()} host threads ({model})"),
        "gbps": nbytes / total / 1e9,
    }


def copy_rate(steps: int) -> float:
    """GB/s (read + write) of the runtime's plain device copy of 1 GiB."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    del a, b
    return 2 * n / dt / 1e9


def probe_copy(steps: int):
    """A plain device copy of known size, for scaling HBM counters."""
    n = 1 << 30
    gbps = copy_rate(steps)
    print(json.dumps({"probe": "copy", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "ms": 2 * n / gbps / 1e6,
                      "gbps": gbps}), flush=True)


def probe_stream(steps: int):
    """HBM streams of 16-byte accesses in the read/write proportions of the
    path's copy kernels (libmoe_ep_probe.so, built with the library): one
    JSON line per stream with its rate over `steps` timed launches. These
    are the practical ceilings the copy kernels are compared with."""
    import ctypes
    import torch
    from combine_topk_ids_dest_amd import build as hb
    if not os.path.exists(hb.PROBE_LIB):
        raise SystemExit(f"{hb.PROBE_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(hb.PROBE_LIB)
    f = lib.moe_ep_probe_stream
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    n = 1 << 31                                    # 2 GiB per buffer
    dev = torch.device("cuda")
    a = torch.full((n,), 1, dtype=torch.uint8, device=dev)
    a2 = torch.full((n,), 2, dtype=torch.uint8, device=dev)
    d = torch.empty(n, dtype=torch.uint8, device=dev)
    d2 = torch.empty(n, dtype=torch.uint8, device=dev)
    grid = 256 * 8
    sink = torch.zeros(grid, dtype=torch.int32, device=dev)
    chunk = 256 * 4 * 16
    st = torch.cuda.current_stream()
    # name, read main, extra read (fraction of n), write main, extra write
    shapes = [("read", True, 0.0, False, 0.0), ("write", False, 0.0, True, 0.0),
              ("copy_1_1", True, 0.0, True, 0.0),
              ("copy_1_1.5 (batch_copy)", True, 0.0, True, 0.5),
              ("copy_5_3 (combine_reduce)", True, 2.0 / 3.0, True, 0.0),
              ("copy_1_2", True, 0.0, True, 1.0)]
    for nt in (1, 0):
        for name, rd, xr, wr, xw in shapes:
            base = n
            er = int(base * xr) // chunk * chunk
            ew = int(base * xw) // chunk * chunk
            args = (a.data_ptr() if rd else None, a2.data_ptr() if er else None, base, er,
                    d.data_ptr() if wr else None, d2.data_ptr() if ew else None, ew,
                    sink.data_ptr(), grid, nt, nt, ctypes.c_void_p(st.cuda_stream))
            assert f(*args) == 0
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(steps):
                f(*args)
            e1.record(st)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            moved = (base if rd else 0) + er + (base if wr else 0) + ew
            print(json.dumps({"probe": "stream", "shape": name, "nontemporal": bool(nt),
                              "bytes_per_launch": moved, "ms": round(ms, 4),
                              "gbps": round(moved / (ms / 1e3) / 1e9, 1)}), flush=True)
    del a, a2, d, d2


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2,
                    help="1 tiny, 2 dsv3_prefill, 3 mixtral_zipf, 4 decode, 5 multi_payload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the pass with the last-level cache evicted before each call "
                         "(profiles then see the warm calls only)")
    ap.add_argument("--cpu-shares", type=int, default=8,
                    help="logical-rank shares the CPU oracle is timed on")
    ap.add_argument("--probe", choices=["copy", "stream"], default=None,
                    help="copy: torch's 1 GiB device copy (the counter scale); stream: HBM "
                         "streams in the copy kernels' read/write proportions")
    ap.add_argument("--graph", action="store_true",
                    help="capture the step in HIP graphs (one per phase and lane when the "
                         "ranks are spread over several lanes) and time their replays")
    ap.add_argument("--fused-local", action="store_true",
                    help="combine each rank's local slice with the fused unpack "
                         "(moe_ep_combine_reduce_peers + moe_ep_combine_unpack_fused)")
    ap.add_argument("--fp4", action="store_true",
                    help="quantize-on-pack: send the bf16 hidden row as 4-bit e2m1 "
                         "codes with one e4m3 scale per 16 columns")
    ap.add_argument("--lanes", default="auto",
                    help="HIP streams the logical ranks are spread over, so one rank's "
                         "kernels overlap another's (each lane holds its own workspace, "
                         "expert-batch and expert-output buffers; capped by LANE_MEMORY_BYTES; with --graph one "
                         "graph per phase and lane); "
                         "1 runs the ranks one after another; auto: AUTO_LANES, or 1 when a "
                         "step's source rows are under AUTO_LANES_MIN_BYTES (the joins "
                         "between streams then cost more than the overlap gains)")
    ap.add_argument("--no-contiguous", action="store_true",
                    help="allocate every buffer from torch's caching allocator instead of "
                         "physically contiguous blocks for the large ones")
    ap.add_argument("--receive", choices=["auto", "scan", "ranked"], default="auto",
                    help="how the receive side finds each pick's expert row: scan (the "
                         "receiver's own scan, moe_ep_expert_batch) or ranked (the packs "
                         "also write per-expert ranks, moe_ep_expert_batch_ranked); auto: "
                         "ranked when a source's batch is one routing tile "
                         f"(T <= {RANKED_MAX_T}, where the pack counts the ranks itself), "
                         "else scan")
    ap.add_argument("--ranked", action="store_true", help="same as --receive ranked")
    ap.add_argument("--fp8-group", type=int, default=None,
                    help="quantize-on-pack: send the bf16 hidden row as fp8 e4m3 "
                         "with one scale per this many columns")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the W expert-parallel ranks are logical "
              "partitions on a single device, so --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as wl
    from combine_topk_ids_dest_amd import binding
    from combine_topk_ids_dest_amd.emulate import LogicalEP

    binding.load()                      # the HIP library or nothing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.probe == "copy":
        probe_copy(max(args.steps, 1))
        return
    if args.probe == "stream":
        probe_stream(max(args.steps, 1))
        return

    w = wl.WORKLOADS[args.workload]
    if args.ranked:
        args.receive = "ranked"
    args.ranked = receive_ranked(args.receive, w.T, w.K, w.E)
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    srcs = [wl.routing(w, s) for s in range(w.W)]
    pls = [wl.payloads(w, s, ids=srcs[s][0], wts=srcs[s][1]) for s in range(w.W)]
    row_bytes = [p.shape[1] for p in pls[0]]
    if args.fp4 and args.fp8_group:
        print("--fp4 and --fp8-group exclude each other", file=sys.stderr)
        sys.exit(2)
    if args.lanes == "auto":
        lanes = auto_lanes(w, row_bytes, args.fp8_group, args.fp4)
    else:
        lanes = lanes_that_fit(w, row_bytes, args.fp8_group, args.fp4, int(args.lanes))
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, row_bytes, torch.bfloat16, dev,
                   quant_group=args.fp8_group, quant_fp4=args.fp4, lanes=lanes,
                   contiguous=not args.no_contiguous, ranked=args.ranked)
    streams = [torch.cuda.Stream() for _ in range(lanes)] if lanes > 1 else None
    for s in range(w.W):
        ep.set_source(s, srcs[s][0], srcs[s][1], pls[s])
    wl.expert_outputs_device(ep.Y, seed=1000 + w.wid)
    ep.share_expert_outputs()
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: inputs generated and resident in "
        f"{time.perf_counter() - t_gen:.1f} s")

    fused = args.fused_local
    for _ in range(args.warmup):
        ep.step(fused_local=fused, streams=streams)
    torch.cuda.synchronize()

    # Timed region: K whole steps, nothing else enqueued between them.
    stream = torch.cuda.current_stream()
    def run_step():
        ep.step(fused_local=fused, streams=streams)

    if args.graph and lanes > 1:
        # one graph per (phase, lane), replayed on the lanes' streams
        ep.capture_lane_graphs(fused_local=fused)
        ep.step_graphs(streams)
        run_step = lambda: ep.step_graphs(streams)
    elif args.graph:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            ep.step(fused_local=fused, streams=streams)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            ep.step(fused_local=fused, streams=streams)
        torch.cuda.synchronize()
        graph.replay()
        run_step = graph.replay
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert int(ep.err.item()) == 0, "device reported data errors"
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # Per-call durations: K more steps with a pair of HIP events around every
    # call, all on one stream, the one the library launches on (torch's
    # current stream), one call after another whatever the lanes. The events
    # add a few microseconds between calls, so these steps are timed
    # separately from the region above.
    k_red, k_unp = ("reduce_peers", "unpack_fused") if fused else ("reduce", "unpack")
    recv_kinds = ["batch"] if args.ranked else ["batch_plan", "batch_copy"]
    recv_calls = [ep.batch] if args.ranked else [ep.batch_plan, ep.batch_copy]
    kinds = (["pack"] * w.W + (recv_kinds + [k_red]) * w.W + [k_unp] * w.W)
    red_call = ep.reduce_peers if fused else ep.reduce
    unp_call = ep.unpack_fused if fused else ep.unpack
    # rank each call belongs to (source for pack/unpack, destination else)
    rank_of = (list(range(w.W)) + [r for r in range(w.W) for _ in range(len(recv_kinds) + 1)]
               + list(range(w.W)))

    def timed_pass(flush=None):
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in kinds] for _ in range(args.steps)]

        def one(k, i, fn, x):
            if flush is not None:
                flush.fill_(k & 0xFF)          # evict the last-level cache first
            ev[k][i][0].record(stream); fn(x); ev[k][i][1].record(stream)

        for k in range(args.steps):
            i = 0
            for s in range(w.W):
                one(k, i, ep.pack, s); i += 1
            for r in range(w.W):
                for fn in recv_calls:
                    one(k, i, fn, r); i += 1
                one(k, i, red_call, r); i += 1
            for s in range(w.W):
                one(k, i, unp_call, s); i += 1
        torch.cuda.synchronize()
        return [[ev[k][i][0].elapsed_time(ev[k][i][1]) for i in range(len(kinds))]
                for k in range(args.steps)]

    times = timed_pass()
    calls = ["pack"] + recv_kinds + [k_red, k_unp]
    per_kind = {k: [] for k in calls}
    for k in range(args.steps):
        for i, kind in enumerate(kinds):
            per_kind[kind].append(times[k][i])
    # Under skewed routing the slowest rank share sets the pace of a real
    # expert-parallel step: per step, the largest per-rank sum of its calls.
    worst_share_ms = float(np.median([
        max(sum(t for t, rk in zip(times[k], rank_of) if rk == r) for r in range(w.W))
        for k in range(args.steps)]))
    dispatch_ms = float(np.median([sum(t for t, kd in zip(times[k], kinds)
                                        if kd in ("pack", "batch", "batch_plan",
                                                  "batch_copy"))
                                    for k in range(args.steps)]))
    combine_ms = float(np.median([sum(t for t, kd in zip(times[k], kinds)
                                       if kd in (k_red, k_unp))
                                   for k in range(args.steps)]))
    # The same calls with the 256 MB last-level cache flushed before each
    # one (a 1 GiB device write), so no call finds its inputs cached; and
    # whole steps over the lanes, each after such a flush.
    cold_info = None
    if not args.no_cold:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold = timed_pass(flush)
        cold_calls = {kd: [cold[k][i] for k in range(args.steps)
                           for i, x in enumerate(kinds) if x == kd] for kd in calls}
        cold_avg_us = {kd: float(np.mean(v)) * 1e3 for kd, v in cold_calls.items()}
        cold_med_us = {kd: float(np.median(v)) * 1e3 for kd, v in cold_calls.items()}
        cold_step_ms = float(np.mean([sum(c) for c in cold]))
        cold_steps = []
        for k in range(args.steps):
            a, b = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            flush.fill_(k & 0xFF)
            a.record(stream)
            ep.step(fused_local=fused, streams=streams)
            b.record(stream)
            cold_steps.append((a, b))
        torch.cuda.synchronize()
        cold_lanes_ms = float(np.median([a.elapsed_time(b) for a, b in cold_steps]))
        del flush

    # The whole step with every call on one stream (the lanes' buffers, no
    # overlap between ranks), timed like the headline region.
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        ep.step(fused_local=fused)
    torch.cuda.synchronize()
    one_stream_ms = (time.perf_counter() - t2) * 1e3 / args.steps

    send_cnt = ep.send_cnt.cpu().numpy().astype(np.int64)
    ent = ep.expert_num_tokens.cpu().numpy().astype(np.int64)
    routed = [int((srcs[s][0] >= 0).any(axis=1).sum()) for s in range(w.W)]
    r_own = None
    if fused:
        r_own = [int((ep.recv_row[s, s, :int(send_cnt[s, s])] >= 0).sum().item())
                 for s in range(w.W)]
    bm = byte_model(w, row_bytes, ep.slots, send_cnt, ent, routed, ep.send_row_bytes,
                    r_own, ranked=args.ranked)
    step_bytes = sum(sum(bm[k]) for k in calls)
    gbps = step_bytes / (ms_per_step / 1e3) / 1e9
    tokens = w.W * w.T
    value = tokens / (ms_per_step / 1e3)

    # the runtime's own 1 GiB device copy in this session, as a second roofline
    copy_gbps = copy_rate(10)
    if not args.no_cold:
        cold_info = {
            "note": "each call timed after a 1 GiB device write that evicts the last-level "
                    "cache; step_over_lanes: whole steps as the timed region runs them, "
                    "each after such a write (median)",
            "per_call_avg_us": {k: round(v, 2) for k, v in cold_avg_us.items()},
            "per_call_median_us": {k: round(v, 2) for k, v in cold_med_us.items()},
            "tokens_per_s": round(tokens / (cold_step_ms / 1e3), 1),
            "effective_gbps": round(step_bytes / (cold_step_ms / 1e3) / 1e9, 1),
            "step_over_lanes_ms": round(cold_lanes_ms, 4),
            "step_over_lanes_tokens_per_s": round(tokens / (cold_lanes_ms / 1e3), 1),
            "step_over_lanes_frac_of_peak_hbm": round(
                step_bytes / (cold_lanes_ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)}

    avg_us = {k: float(np.mean(v)) * 1e3 for k, v in per_kind.items()}
    med_us = {k: float(np.median(v)) * 1e3 for k, v in per_kind.items()}
    total_ms = {k: float(np.sum(v)) for k, v in per_kind.items()}
    dom = roofline_call(total_ms)
    bytes_per_launch = float(np.mean(bm[dom]))
    achieved = bytes_per_launch / (avg_us[dom] * 1e-6) / 1e9
    traffic = read_traffic(KERNEL_OF_CALL[dom], w.name + mode_suffix(args))
    roofline = {
        "bound": "hbm",
        "kernel": KERNEL_OF_CALL[dom],
        "call": ABI_OF_CALL[dom],
        "achieved": round(achieved, 1),
        "peak": PEAK_HBM_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_HBM_GBPS, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": int(bytes_per_launch),
        "avg_launch_us": round(avg_us[dom], 2),
        "median_launch_us": round(med_us[dom], 2),
    }

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "T": w.T, "H": w.H, "E": w.E, "K": w.K,
            "W": w.W, "cap": w.cap, "routing": w.routing
            + (f" s={w.zipf_s}" if w.routing == "zipf" else ""),
            "padding_rows": w.n_pad, "payload_bytes_per_row": int(sum(ep.send_row_bytes)),
            "dispatch_format": (f"fp8_e4m3_g{args.fp8_group}" if args.fp8_group
                                else "fp4_e2m1_e4m3_g16" if args.fp4 else "as_given"),
            "combine_accumulation": "fp32",
            "launch": "hip_graph" if args.graph else "eager",
            "lanes": lanes,
            "large_buffers": ("physically_contiguous" if ep.contiguous_bytes
                              else "caching_allocator"),
            "local_slice_combine": "fused" if fused else "reduce_then_unpack",
            "receive_rows": ("sender_ranks" if args.ranked else "receive_scan"),
            "parallelism": f"1 GPU, {w.W} logical expert-parallel ranks",
        },
        "effective_gbps": round(gbps, 1),
        "frac_of_peak_hbm": round(gbps / PEAK_HBM_GBPS, 4),
        "copy_reference_gbps": round(copy_gbps, 1),
        "frac_of_copy_reference": round(gbps / copy_gbps, 4),
        "algorithmic_bytes_per_step": int(step_bytes),
        "per_call_avg_us": {k: round(v, 2) for k, v in avg_us.items()},
        "per_call_median_us": {k: round(v, 2) for k, v in med_us.items()},
        "per_call_gbps": {k: round(float(np.sum(bm[k])) / (total_ms[k] / args.steps / 1e3) / 1e9, 1)
                          for k in calls},
        "per_call_note": "per-call times come from a separate pass with HIP events around each call",
        "one_stream_ms_per_step": round(one_stream_ms, 4),
        "one_stream_tokens_per_s": round(tokens / (one_stream_ms / 1e3), 1),
        "per_rank_share_us": round(ms_per_step * 1e3 / w.W, 2),
        "critical_path_tokens_per_s": round(w.T / (worst_share_ms / 1e3), 1),
        "dispatch_ms_per_step": round(dispatch_ms, 4),
        "combine_ms_per_step": round(combine_ms, 4),
        "cold": cold_info,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    log(f"[bench] {w.name}: {ms_per_step:.3f} ms/step, {value / 1e6:.2f} M tokens/s, "
        f"{gbps:.0f} GB/s ({100 * gbps / PEAK_HBM_GBPS:.1f} % of peak); per call us "
        f"{result['per_call_avg_us']}")

    if not args.no_cpu_baseline:
        del ep
        gc.collect()
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(w, srcs, pls, args.cpu_shares)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
