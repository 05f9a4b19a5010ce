"""CPU oracle for the MoE expert-parallel dispatch/combine layout transform.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package. The product path (the
HIP library and its Python binding) never imports, links or calls it.

The arithmetic lives in moe_ep_oracle.c (plain single-threaded C, built by
gcc); this module only marshals numpy arrays into it. The method is the one
stated on the vLLM API documentation page
"vllm.model_executor.layers.fused_moe.prepare_finalize.alltoall_batched"
(AllToAllBatchedPrepareAndFinalize: capacities, prepare, finalize); each C
function cites the step it follows.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(hand-derived worked examples, brute force over micro shapes against a
set-based formulation, closed forms and invariants). None is unpinned.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

from . import build as _build

ERR_ID_RANGE = 1
ERR_PICKS = 2
ERR_ELOC = 4
ERR_ROWCAP = 8
ERR_CNT = 16

BF16 = 0
F32 = 1

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def load(rebuild: bool = False):
    """Loads liboracle_moe_ep.so, building it with gcc when it is absent."""
    global _lib
    if _lib is not None and not rebuild:
        return _lib
    if (rebuild or not os.path.exists(_build.LIB)
            or os.path.getmtime(_build.SRC) > os.path.getmtime(_build.LIB)):
        _build.build()
    _lib = _open(_build.LIB)
    return _lib


class use_library:
    """Context manager: route every call of this module through another
    build of moe_ep_oracle.c (the mutation tests build planted-mistake
    copies on the CPU and check that the pins reject them)."""

    def __init__(self, path: str):
        self.path = path
        self.saved = None

    def __enter__(self):
        global _lib
        self.saved = load()
        _lib = _open(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _open(path: str):
    lib = ctypes.CDLL(path)
    lib.oracle_capacities.argtypes = [_I32, _I32, _I32, _I64, _P, _P, _P]
    lib.oracle_capacities.restype = ctypes.c_int
    lib.oracle_dispatch_pack.argtypes = [
        _P, _P, _I64, _I32, _I32, _I32, _I64, _I32,
        _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_dispatch_pack.restype = ctypes.c_uint32
    lib.oracle_expert_batch.argtypes = [
        _P, _I64, _P, _I64, _I32, _I32, _I32, _I64, _I32,
        _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_expert_batch.restype = ctypes.c_uint32
    lib.oracle_combine_reduce.argtypes = [
        _P, _I64, _I64, _I32, _I64, _P, _I64, _P, _P, _I64, _P,
        _I32, _I32, _I32, _I64, _P, _I64, _I64]
    lib.oracle_combine_reduce.restype = ctypes.c_uint32
    lib.oracle_combine_unpack.argtypes = [
        _P, _I64, _I64, _I32, _I64, _P, _I64, _I32, _P, _I64]
    lib.oracle_combine_unpack.restype = None
    lib.oracle_pick_ranks.argtypes = [_P, _P, _I32, _I32, _I32, _I64, _P, _P]
    lib.oracle_pick_ranks.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [ctypes.c_float]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_round_bf16_bits.argtypes = [ctypes.c_uint32]
    lib.oracle_round_bf16_bits.restype = ctypes.c_uint16
    lib.oracle_sanitize_expert_ids.argtypes = [
        _P, _I64, _P, _I64, _I32, _I32, _I32, _I64, _I32, _P, _I64]
    lib.oracle_sanitize_expert_ids.restype = ctypes.c_uint32
    lib.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_e4m3.restype = ctypes.c_uint8
    lib.oracle_quantize_fp8.argtypes = [_P, _I64, _I64, _I64, _I32, _P, _I64, _P, _I64]
    lib.oracle_quantize_fp8.restype = None
    lib.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_e2m1.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_e2m1.restype = ctypes.c_uint8
    lib.oracle_quantize_fp4.argtypes = [_P, _I64, _I64, _I64, _P, _I64, _P, _I64]
    lib.oracle_quantize_fp4.restype = None
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _ptr_array(arrs: Sequence[np.ndarray]):
    return (ctypes.c_void_p * max(1, len(arrs)))(*[_ptr(a) for a in arrs])


def _i64_array(vals: Sequence[int]):
    return (ctypes.c_int64 * max(1, len(vals)))(*[int(v) for v in vals])


def _inner_contiguous(a: np.ndarray, name: str, ndim: int):
    if a.ndim != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {a.shape}")
    exp = a.itemsize
    if a.size == 0:
        return
    for ax in range(ndim - 1, 0, -1):
        if a.shape[ax] > 1 and a.strides[ax] != exp:
            raise ValueError(f"{name}: inner dims must be dense")
        exp *= a.shape[ax]


def capacities(K: int, E: int, W: int, max_num_tokens: int):
    """(cap, slots, expert_cap) as capacities() defines them."""
    cap = ctypes.c_int64()
    slots = ctypes.c_int32()
    ecap = ctypes.c_int64()
    rc = load().oracle_capacities(K, E, W, max_num_tokens, ctypes.byref(cap),
                                  ctypes.byref(slots), ctypes.byref(ecap))
    if rc:
        raise ValueError("invalid capacities arguments")
    return cap.value, slots.value, ecap.value


def round_bf16(x: float) -> int:
    return int(load().oracle_round_bf16(ctypes.c_float(x)))


def round_bf16_bits(u: int) -> int:
    """bf16 bits of the binary32 word u (passed as an integer, so NaN
    payloads and signaling NaNs arrive unchanged)."""
    return int(load().oracle_round_bf16_bits(ctypes.c_uint32(u)))


def f32_to_e4m3(x: float) -> int:
    return int(load().oracle_f32_to_e4m3(ctypes.c_float(x)))


def quantize_fp8(hidden_bits: np.ndarray, group: int = 128):
    """fp8 e4m3 codes uint8 [T, H] and fp32 scales [T, H/group] of bf16 rows
    (uint16 bit patterns [T, H], dense rows)."""
    x = np.ascontiguousarray(hidden_bits, dtype=np.uint16)
    T, H = x.shape
    G = -(-H // group)
    q = np.empty((T, H), np.uint8)
    sc = np.empty((T, G), np.float32)
    load().oracle_quantize_fp8(_ptr(x), T, H, H, group, _ptr(q), H, _ptr(sc), G)
    return q, sc


def dispatch_pack_fp8(topk_ids: np.ndarray, topk_weights: np.ndarray, E: int,
                      W: int, max_num_tokens: int, hidden_bits: np.ndarray,
                      group: int = 128, payloads: Sequence[np.ndarray] = (),
                      fill: int = 0) -> dict:
    """Quantize-on-pack: every token row is quantised once (quantize_fp8),
    then the codes, the scales (rows padded with +0.0 to a multiple of 4
    floats) and the further payloads are packed like any payload
    (dispatch_pack). send[0] holds the codes, send[1] the scales as bytes."""
    q, sc = quantize_fp8(hidden_bits, group)
    T, G = sc.shape
    # scale rows padded with +0.0 to a multiple of 4 floats (16-byte rows)
    Gp = (G + 3) // 4 * 4
    scp = np.zeros((T, Gp), np.float32)
    scp[:, :G] = sc
    pl = [q, scp.view(np.uint8).reshape(T, Gp * 4)] + list(payloads)
    r = dispatch_pack(topk_ids, topk_weights, E, W, max_num_tokens, pl, fill)
    r.update(q=q, scales=sc)
    return r


def e4m3_to_f32(code: int) -> float:
    return float(load().oracle_e4m3_to_f32(ctypes.c_uint8(code)))


def f32_to_e2m1(x: float) -> int:
    return int(load().oracle_f32_to_e2m1(ctypes.c_float(x)))


def fp4_scale_pitch(H: int) -> int:
    """Bytes of a 4-bit row's scale row: H/16, padded to a multiple of 16."""
    return (H // 16 + 15) // 16 * 16


def quantize_fp4(hidden_bits: np.ndarray):
    """4-bit e2m1 codes uint8 [T, H/2] (two per byte, even column low) and
    e4m3 scale codes uint8 [T, H/16] of bf16 rows (uint16 [T, H], H a
    multiple of 16)."""
    x = np.ascontiguousarray(hidden_bits, dtype=np.uint16)
    T, H = x.shape
    if H % 16:
        raise ValueError("H must be a multiple of 16")
    q = np.empty((T, H // 2), np.uint8)
    sc = np.empty((T, H // 16), np.uint8)
    load().oracle_quantize_fp4(_ptr(x), T, H, H, _ptr(q), H // 2, _ptr(sc), H // 16)
    return q, sc


def dispatch_pack_fp4(topk_ids: np.ndarray, topk_weights: np.ndarray, E: int,
                      W: int, max_num_tokens: int, hidden_bits: np.ndarray,
                      payloads: Sequence[np.ndarray] = (), fill: int = 0) -> dict:
    """4-bit quantize-on-pack: every token row is quantised once
    (quantize_fp4), then the codes, the scale codes (rows padded with 0x00,
    +0.0 in e4m3, to a multiple of 16 bytes) and the further payloads are
    packed like any payload (dispatch_pack)."""
    q, sc = quantize_fp4(hidden_bits)
    T, nb = sc.shape
    scp = np.zeros((T, fp4_scale_pitch(nb * 16)), np.uint8)
    scp[:, :nb] = sc
    r = dispatch_pack(topk_ids, topk_weights, E, W, max_num_tokens,
                      [q, scp] + list(payloads), fill)
    r.update(q=q, scales=sc)
    return r


def dispatch_pack(topk_ids: np.ndarray, topk_weights: np.ndarray, E: int,
                  W: int, max_num_tokens: int,
                  payloads: Sequence[np.ndarray] = (),
                  fill: int = 0) -> dict:
    """Send side of one source rank.

    payloads: 2-D arrays [T, row] of any dtype with dense rows (row stride
    may exceed the row). Returns send_cnt [W], send_eloc / send_w
    [W, cap, slots], token_slot [T, W], send (one uint8 [W, rows, row_bytes]
    array per payload with rows = max(send_cnt), the valid prefix of the
    [W, cap, row] layout; tails filled with `fill`) and err.
    """
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    wts = np.ascontiguousarray(topk_weights, dtype=np.float32)
    T, K = ids.shape
    cap, slots, _ = capacities(K, E, W, max_num_tokens)
    send_cnt = np.zeros(W, np.int32)
    send_eloc = np.full((W, cap, slots), -7, np.int32)
    send_w = np.full((W, cap, slots), np.nan, np.float32)
    token_slot = np.full((T, W), -7, np.int32)
    rows = 0
    if len(payloads):
        # the counts alone first, to size the send rows to the valid prefix
        rows = int(dispatch_pack(ids, wts, E, W, max_num_tokens)["send_cnt"].max(initial=0))
    srcs, rbytes, sstr, dsts = [], [], [], []
    for p in payloads:
        if p.ndim != 2 or p.shape[0] != T:
            raise ValueError("payloads must be [T, row]")
        if T > 0 and p.shape[1] > 1 and p.strides[1] != p.itemsize:
            raise ValueError("payload rows must be dense")
        rb = p.shape[1] * p.itemsize
        srcs.append(p)
        sstr.append(p.strides[0])
        rbytes.append(rb)
        dsts.append(np.full((W, rows, rb), fill, np.uint8))
    err = load().oracle_dispatch_pack(
        _ptr(ids), _ptr(wts), T, K, E, W, max_num_tokens, len(srcs),
        _ptr_array(srcs), _i64_array(sstr), _i64_array(rbytes),
        _ptr_array(dsts), _i64_array([rows * rb for rb in rbytes]),
        _i64_array(rbytes),
        _ptr(send_cnt), _ptr(send_eloc), _ptr(send_w), _ptr(token_slot))
    if err == 0xFFFFFFFF:
        raise ValueError("oracle_dispatch_pack rejected its arguments")
    return dict(send_cnt=send_cnt, send_eloc=send_eloc, send_w=send_w,
                token_slot=token_slot, send=dsts, err=int(err),
                cap=cap, slots=slots)


def pick_ranks(send_cnt: np.ndarray, send_eloc: np.ndarray, e_local: int) -> dict:
    """Send-side ranks of one source's pack outputs (send_cnt [W], send_eloc
    [W, cap, slots]): send_rank [W, cap, slots] (-1 for unused columns;
    slots past the count are -9, never written) and send_ecnt
    [W, e_local]."""
    cnt = np.ascontiguousarray(send_cnt, dtype=np.int32)
    eloc = np.ascontiguousarray(send_eloc, dtype=np.int32)
    W, cap, slots = eloc.shape
    rank = np.full(eloc.shape, -9, np.int32)
    ecnt = np.empty((W, e_local), np.int32)
    rc = load().oracle_pick_ranks(_ptr(cnt), _ptr(eloc), W, e_local, slots, cap,
                                  _ptr(rank), _ptr(ecnt))
    if rc:
        raise ValueError("oracle_pick_ranks: bad sizes")
    return {"send_rank": rank, "send_ecnt": ecnt}


def expert_batch(recv_cnt: np.ndarray, recv_eloc: np.ndarray, W: int,
                 e_local: int, K: int, max_num_tokens: int,
                 recv_payloads: Sequence[np.ndarray] = (),
                 fill: int = 0) -> dict:
    """Receive side of one destination rank.

    recv_cnt: int32 [W] (any stride). recv_eloc: int32 [W, cap, slots]
    (rank stride free, inner dense). recv_payloads: uint8 [W, rows, row]
    (rank stride free, inner dense, rows >= every received count). Returns expert_num_tokens [e_local],
    recv_row [W, cap, slots], b (uint8 [e_local, rows, row] per payload,
    rows = the largest expert_num_tokens, i.e. the valid prefix of the
    [e_local, W*cap, row] layout) and err.
    """
    cap, slots, ecap = capacities(K, e_local * W, W, max_num_tokens)
    if recv_cnt.dtype != np.int32 or recv_eloc.dtype != np.int32:
        raise ValueError("counts and local expert ids are int32")
    if recv_cnt.shape != (W,):
        raise ValueError("recv_cnt must be [W]")
    _inner_contiguous(recv_eloc, "recv_eloc", 3)
    if recv_eloc.shape != (W, cap, slots):
        raise ValueError(f"recv_eloc must be {(W, cap, slots)}")
    ent = np.zeros(e_local, np.int32)
    recv_row = np.full((W, cap, slots), -7, np.int32)
    nrows = 0
    if len(recv_payloads):
        # the counts alone first, to size the batched rows to the valid prefix
        nrows = int(expert_batch(recv_cnt, recv_eloc, W, e_local, K,
                                 max_num_tokens)["expert_num_tokens"].max(initial=0))
    srcs, rstr, rowstr, rbytes, dsts = [], [], [], [], []
    for p in recv_payloads:
        _inner_contiguous(p, "recv payload", 3)
        if p.shape[0] != W or p.shape[1] < int(np.clip(recv_cnt, 0, cap).max(initial=0)):
            raise ValueError("recv payloads must be [W, rows >= counts, row]")
        rb = p.shape[2] * p.itemsize
        srcs.append(p)
        rstr.append(p.strides[0])
        rowstr.append(rb)
        rbytes.append(rb)
        dsts.append(np.full((e_local, nrows, rb), fill, np.uint8))
    err = load().oracle_expert_batch(
        _ptr(recv_cnt), recv_cnt.strides[0] // 4,
        _ptr(recv_eloc), recv_eloc.strides[0] // 4,
        W, e_local, K, max_num_tokens, len(srcs),
        _ptr_array(srcs), _i64_array(rstr), _i64_array(rowstr),
        _i64_array(rbytes), _ptr_array(dsts),
        _i64_array([nrows * rb for rb in rbytes]), _i64_array(rbytes),
        _ptr(ent), _ptr(recv_row))
    if err == 0xFFFFFFFF:
        raise ValueError("oracle_expert_batch rejected its arguments")
    return dict(expert_num_tokens=ent, recv_row=recv_row, b=dsts,
                err=int(err), cap=cap, slots=slots, expert_cap=ecap)


def sanitize_expert_ids(recv_cnt: np.ndarray, recv_eloc: np.ndarray, W: int,
                        e_local: int, K: int, max_num_tokens: int,
                        invalid_id: int) -> dict:
    """The received local ids [W, cap, slots] with every entry that is not a
    valid pick set to invalid_id (all entries written)."""
    cap, slots, _ = capacities(K, e_local * W, W, max_num_tokens)
    _inner_contiguous(recv_eloc, "recv_eloc", 3)
    if recv_eloc.shape != (W, cap, slots):
        raise ValueError(f"recv_eloc must be {(W, cap, slots)}")
    out = np.full((W, cap, slots), -7, np.int32)
    err = load().oracle_sanitize_expert_ids(
        _ptr(recv_cnt), recv_cnt.strides[0] // 4, _ptr(recv_eloc),
        recv_eloc.strides[0] // 4, W, e_local, K, max_num_tokens, invalid_id,
        _ptr(out), cap * slots)
    if err == 0xFFFFFFFF:
        raise ValueError("oracle_sanitize_expert_ids rejected its arguments")
    return dict(ids=out, err=int(err))


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise ValueError("combine data must be bf16 bits (uint16) or float32")


def combine_reduce(Y: np.ndarray, recv_cnt: np.ndarray, recv_eloc: np.ndarray,
                   recv_w: np.ndarray, recv_row: np.ndarray, W: int,
                   e_local: int, K: int, max_num_tokens: int,
                   fill=None) -> dict:
    """Weighted reduce on one destination rank.

    Y: [e_local, rows, H] (bf16 bits as uint16, or float32), strides free
    on the two outer axes, last axis dense. recv_eloc / recv_w share one
    rank stride. Returns ret [W, rows, H] (same dtype as Y; rows = the
    largest received count, the valid prefix of the [W, cap, H] layout;
    rows past a source's count hold `fill`) and err.
    """
    dt = _dtype_code(Y)
    cap, slots, _ = capacities(K, e_local * W, W, max_num_tokens)
    if Y.ndim != 3 or Y.shape[0] != e_local or (Y.size and Y.strides[2] != Y.itemsize):
        raise ValueError("Y must be [e_local, rows, H] with dense rows")
    if Y.size == 0:                      # nothing can be read from it
        Y = np.zeros((e_local, 1, Y.shape[2]), Y.dtype)
    if recv_eloc.strides != recv_w.strides:
        raise ValueError("recv_eloc and recv_w must share strides")
    _inner_contiguous(recv_eloc, "recv_eloc", 3)
    H = Y.shape[2]
    if fill is None:
        fill = 0xFFFF if dt == BF16 else np.nan
    rows = int(np.clip(recv_cnt, 0, cap).max(initial=0))
    ret = np.full((W, rows, H), fill, Y.dtype)
    rr = np.ascontiguousarray(recv_row, dtype=np.int32)
    err = load().oracle_combine_reduce(
        _ptr(Y), Y.strides[0] // Y.itemsize, Y.strides[1] // Y.itemsize, dt, H,
        _ptr(recv_cnt), recv_cnt.strides[0] // 4,
        _ptr(recv_eloc), _ptr(recv_w), recv_eloc.strides[0] // 4, _ptr(rr),
        W, e_local, K, max_num_tokens, _ptr(ret), rows * H, H)
    if err == 0xFFFFFFFF:
        raise ValueError("oracle_combine_reduce rejected its arguments")
    return dict(ret=ret, err=int(err))


def combine_unpack(back: np.ndarray, token_slot: np.ndarray) -> np.ndarray:
    """Per-token sum of the returned partials of one source rank.

    back: [W, rows, H] (bf16 bits uint16 or float32), rank stride free, rows
    dense, rows past every slot in token_slot. token_slot: int32 [T, W]. Returns out [T, H], every row written.
    """
    dt = _dtype_code(back)
    if back.ndim != 3 or (back.size and back.strides[2] != back.itemsize):
        raise ValueError("back must be [W, rows, H] with dense rows")
    if back.size == 0:                   # no slot can be read from it
        back = np.zeros((back.shape[0], 1, back.shape[2]), back.dtype)
    ts = np.ascontiguousarray(token_slot, dtype=np.int32)
    T, W = ts.shape
    if back.shape[0] != W:
        raise ValueError("back and token_slot disagree on W")
    H = back.shape[2]
    out = np.empty((T, H), back.dtype)
    load().oracle_combine_unpack(
        _ptr(back), back.strides[0] // back.itemsize,
        back.strides[1] // back.itemsize, dt, H, _ptr(ts), T, W, _ptr(out), H)
    return out


# --------------------------------------------------------------------------
# Whole-path helpers over W logical ranks (the exchange is an index swap).
# --------------------------------------------------------------------------

def stack_ranks(blocks: Sequence[np.ndarray], fill=0, min_rows: int = 0) -> np.ndarray:
    """[n_i, ...] blocks of W ranks -> [W, max(n_i, min_rows), ...], padded
    with fill."""
    rows = max([b.shape[0] for b in blocks] + [min_rows])
    out = np.full((len(blocks), rows) + blocks[0].shape[1:], fill, blocks[0].dtype)
    for i, b in enumerate(blocks):
        out[i, :b.shape[0]] = b
    return out


def run_path(srcs_ids: List[np.ndarray], srcs_wts: List[np.ndarray],
             srcs_payloads: List[List[np.ndarray]], E: int, W: int,
             max_num_tokens: int, expert_out_fn=None,
             combine_dtype: str = "bf16") -> dict:
    """Runs pack for every source, batch for every destination, then (when
    expert_out_fn is given) reduce for every destination and unpack for
    every source.

    expert_out_fn(dest, batch_result) -> Y [e_local, rows, H] returns the
    expert outputs of a destination; the exchange of step a5 is
    recv_r[s] = send_s[r] and of step a9 back_s[d] = ret_d[s].
    """
    K = srcs_ids[0].shape[1]
    e_local = E // W
    packs = [dispatch_pack(srcs_ids[s], srcs_wts[s], E, W, max_num_tokens,
                           srcs_payloads[s]) for s in range(W)]
    n_pl = len(srcs_payloads[0])
    send_cnt = np.stack([p["send_cnt"] for p in packs])          # [src, dst]
    send_eloc = np.stack([p["send_eloc"] for p in packs])        # [src,dst,cap,slots]
    send_w = np.stack([p["send_w"] for p in packs])
    batches = []
    for r in range(W):
        recv_pl = [stack_ranks([packs[s]["send"][p][r] for s in range(W)])
                   for p in range(n_pl)]
        batches.append(expert_batch(
            np.ascontiguousarray(send_cnt[:, r]),
            np.ascontiguousarray(send_eloc[:, r]), W, e_local, K,
            max_num_tokens, recv_pl))
    res = dict(packs=packs, batches=batches, send_cnt=send_cnt,
               send_eloc=send_eloc, send_w=send_w)
    if expert_out_fn is None:
        return res
    rets = []
    for r in range(W):
        Y = expert_out_fn(r, batches[r])
        rets.append(combine_reduce(
            Y, np.ascontiguousarray(send_cnt[:, r]),
            np.ascontiguousarray(send_eloc[:, r]),
            np.ascontiguousarray(send_w[:, r]), batches[r]["recv_row"],
            W, e_local, K, max_num_tokens)["ret"])
    outs = []
    for s in range(W):
        back = stack_ranks([rets[d][s] for d in range(W)])
        outs.append(combine_unpack(back, packs[s]["token_slot"]))
    res.update(rets=rets, outs=outs)
    return res
