"""Python binding of libmoe_ep.so: the same names as the C ABI
(include/moe_ep.h), argument marshalling only.

Tensors are torch device tensors; this module reads their data pointers,
element strides and the current HIP stream, checks that the layouts are the
ones the C ABI describes, and calls the library. Every step of the path runs
in the library's HIP kernels. If the library is missing this module raises;
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_ep.so")

OK, EINVAL, ECAP, EDTYPE, EALIGN, EWORKSPACE, EHIP, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
NOALLOC_SCRATCH_BYTES = 8 << 20
BF16, F32 = 0, 1
ERR_ID_RANGE, ERR_PICKS, ERR_ELOC, ERR_ROWCAP, ERR_CNT = 1, 2, 4, 8, 16
MAX_PAYLOADS = 8

EXPORTED = (
    "moe_ep_capacities",
    "moe_ep_workspace_bytes",
    "moe_ep_status_string",
    "moe_ep_dispatch_pack",
    "moe_ep_dispatch_pack_fp8",
    "moe_ep_expert_batch",
    "moe_ep_expert_batch_plan",
    "moe_ep_expert_batch_copy",
    "moe_ep_sanitize_expert_ids",
    "moe_ep_dispatch_pack_fp4",
    "moe_ep_combine_reduce",
    "moe_ep_combine_unpack",
    "moe_ep_combine_reduce_peers",
    "moe_ep_combine_unpack_fused",
    "moe_ep_dispatch_pack_noalloc",
    "moe_ep_expert_batch_ranked",
)


class MoeEpPayload(ctypes.Structure):
    _fields_ = [
        ("src", ctypes.c_void_p),
        ("src_stride", ctypes.c_int64),
        ("dst", ctypes.c_void_p),
        ("dst_stride", ctypes.c_int64),
        ("row_bytes", ctypes.c_int64),
    ]


class MoeEpError(RuntimeError):
    def __init__(self, name: str, status: int, text: str):
        super().__init__(f"{name}: {text} (status {status})")
        self.status = status


_lib = None
_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads libmoe_ep.so; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with `python -m combine_topk_ids_dest_amd.build`")
    lib = ctypes.CDLL(p)
    lib.moe_ep_capacities.argtypes = [_I32, _I32, _I32, _I64, _P, _P, _P]
    lib.moe_ep_workspace_bytes.argtypes = [_I64, _I32, _I32, _I32, _I64, _P]
    lib.moe_ep_status_string.argtypes = [ctypes.c_int]
    lib.moe_ep_status_string.restype = ctypes.c_char_p
    lib.moe_ep_dispatch_pack.argtypes = [
        _P, _P, _I64, _I32, _I32, _I32, _I64, _P, _I32,
        _P, _P, _P, _I64, _P, _P, _P, _P, _P, _SZ, _P]
    lib.moe_ep_dispatch_pack_noalloc.argtypes = [
        _P, _P, _I64, _I32, _I32, _I32, _I64, _P, _I32,
        _P, _P, _P, _I64, _P, _P, _P, _P, _P]
    lib.moe_ep_dispatch_pack_fp8.argtypes = [
        _P, _P, _I64, _I32, _I32, _I32, _I64, _P, _I64, _I64, _I32,
        _P, _I64, _P, _I64, _P, _I32, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _SZ, _P]
    lib.moe_ep_expert_batch_ranked.argtypes = [
        _P, _I64, _P, _P, _I64, _P, _I64, _I32, _I32, _I32, _I64, _P, _I32,
        _P, _P, _P, _P]
    lib.moe_ep_expert_batch.argtypes = [
        _P, _I64, _P, _I64, _I32, _I32, _I32, _I64, _P, _I32,
        _P, _P, _P, _P, _SZ, _P]
    lib.moe_ep_expert_batch_plan.argtypes = [
        _P, _I64, _P, _I64, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _SZ, _P]
    lib.moe_ep_expert_batch_copy.argtypes = [
        _P, _I64, _P, _I64, _I32, _I32, _I32, _I64, _P, _I32, _P, _P, _P, _SZ, _P]
    lib.moe_ep_dispatch_pack_fp4.argtypes = [
        _P, _P, _I64, _I32, _I32, _I32, _I64, _P, _I64, _I64, _P, _I64, _P, _I64,
        _P, _I32, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _SZ, _P]
    lib.moe_ep_sanitize_expert_ids.argtypes = [
        _P, _I64, _P, _I64, _I32, _I32, _I32, _I64, _I32, _P, _I64, _P, _P]
    lib.moe_ep_combine_reduce.argtypes = [
        _P, _I64, _I32, _I64, _P, _I64, _P, _P, _I64, _P,
        _I32, _I32, _I32, _I64, _P, _I64, _P]
    lib.moe_ep_combine_unpack.argtypes = [
        _P, _I64, _I32, _I64, _P, _I64, _I32, _I64, _P, _P]
    lib.moe_ep_combine_reduce_peers.argtypes = [
        _P, _I64, _I32, _I64, _P, _I64, _P, _P, _I64, _P,
        _I32, _I32, _I32, _I64, _I32, _P, _I64, _P]
    lib.moe_ep_combine_unpack_fused.argtypes = [
        _P, _I64, _I32, _I64, _P, _I64, _I32, _I64, _I32, _P, _I64, _P, _P, _P,
        _I32, _I32, _P, _P]
    for name in EXPORTED:
        if name != "moe_ep_status_string":
            getattr(lib, name).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_ep_status_string(int(status)).decode()


def _check(name: str, status: int):
    if status != OK:
        raise MoeEpError(name, status, status_string(status))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dense_from(t: torch.Tensor, first: int, name: str):
    """Checks that dims >= first of t are dense (row-major, no gaps)."""
    exp = 1
    for ax in range(t.dim() - 1, first - 1, -1):
        if t.size(ax) > 1 and t.stride(ax) != exp:
            raise ValueError(f"{name}: dims from {first} on must be dense")
        exp *= t.size(ax)


def _row_bytes(t: torch.Tensor, first: int) -> int:
    n = 1
    for s in t.shape[first:]:
        n *= s
    return n * t.element_size()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"combine data must be bfloat16 or float32, not {t.dtype}")


# ---------------------------------------------------------------------------
# Host-side queries
# ---------------------------------------------------------------------------

def moe_ep_capacities(K: int, E: int, W: int, max_num_tokens: int) -> Tuple[int, int, int]:
    cap, slots, ecap = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int64()
    _check("moe_ep_capacities", load().moe_ep_capacities(
        K, E, W, max_num_tokens, ctypes.byref(cap), ctypes.byref(slots),
        ctypes.byref(ecap)))
    return cap.value, slots.value, ecap.value


def moe_ep_workspace_bytes(T: int, K: int, E: int, W: int, max_num_tokens: int) -> int:
    b = ctypes.c_size_t()
    _check("moe_ep_workspace_bytes", load().moe_ep_workspace_bytes(
        T, K, E, W, max_num_tokens, ctypes.byref(b)))
    return b.value


# ---------------------------------------------------------------------------
# The four calls of the path
# ---------------------------------------------------------------------------

def _payload_array(pairs, src_row_dim: int, dst_row_dim: int,
                   src_lead: Sequence[int] = (), dst_lead: Sequence[int] = ()):
    """Descriptors for (src, dst) pairs whose dim 0 is the strided leading
    dim and whose dims from 1 on are dense; a row spans the dims from
    src_row_dim (dst_row_dim) on. src_lead / dst_lead: least sizes of the
    dims before the row (the leading dim and, for [W, cap, row] blocks, the
    rows per block)."""
    if len(pairs) > MAX_PAYLOADS:
        raise ValueError("too many payloads")
    arr = (MoeEpPayload * MAX_PAYLOADS)()
    for i, (src, dst) in enumerate(pairs):
        _dense_from(src, 1, "payload src")
        _dense_from(dst, 1, "payload dst")
        _lead_at_least(src, src_lead, f"payload {i} src")
        _lead_at_least(dst, dst_lead, f"payload {i} dst")
        rb = _row_bytes(src, src_row_dim)
        if _row_bytes(dst, dst_row_dim) != rb:
            raise ValueError("payload src and dst rows differ in size")
        arr[i].src = src.data_ptr()
        arr[i].src_stride = src.stride(0) * src.element_size()
        arr[i].dst = dst.data_ptr()
        arr[i].dst_stride = dst.stride(0) * dst.element_size()
        arr[i].row_bytes = rb
    return arr


# ---------------------------------------------------------------------------
# Shape checks. The C ABI sees pointers and strides only, so a tensor of the
# wrong size would be read or written out of bounds on the device; every
# prepare_* function checks sizes here first and raises ValueError (before
# the one-GPU check, so that host tensors can stand in for the shapes).
# ---------------------------------------------------------------------------

def _lead_at_least(t: torch.Tensor, mins: Sequence[int], name: str):
    if t.dim() < len(mins) or any(t.size(i) < m for i, m in enumerate(mins)):
        raise ValueError(f"{name}: leading dims {tuple(t.shape[:len(mins)])} "
                         f"must be at least {tuple(mins)}")


def _shape(t: Optional[torch.Tensor], shape: Sequence[int], name: str, dtypes=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")


def _blocks(t: torch.Tensor, n: int, block_elems: int, name: str, dtypes=None):
    """n blocks along dim 0 (any stride), each a dense run of block_elems
    elements."""
    if t.dim() < 1 or t.size(0) != n:
        raise ValueError(f"{name}: {n} blocks along dim 0 expected, shape {tuple(t.shape)}")
    per = 1
    for x in t.shape[1:]:
        per *= x
    if per != block_elems:
        raise ValueError(f"{name}: blocks of {per} elements, expected {block_elems}")
    _dense_from(t, 1, name)
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")


def _vector(t: torch.Tensor, n: int, name: str, dtypes=None):
    """At least n elements along one dim (any stride)."""
    if t.dim() != 1 or t.size(0) < n:
        raise ValueError(f"{name}: a vector of at least {n} elements expected, "
                         f"shape {tuple(t.shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")


def _err(err_flags: Optional[torch.Tensor]):
    if err_flags is not None:
        _vector(err_flags, 1, "err_flags", _I32T)


_I32T = (torch.int32,)
_F32T = (torch.float32,)


def _sizes(K: int, E: int, W: int, max_num_tokens: int):
    """e_local, slots, cap, expert_cap as capacities() forms them."""
    if K <= 0 or E <= 0 or W <= 0 or E % W or max_num_tokens < 0:
        raise ValueError(f"bad sizes K={K} E={E} W={W} max_num_tokens={max_num_tokens}")
    e_local = E // W
    return e_local, min(K, e_local), max_num_tokens, max_num_tokens * W


def _ranks(send_rank, send_ecnt, send_eloc, W, E):
    """Optional per-expert rank outputs of a pack: both or neither;
    send_rank shaped and strided like send_eloc, send_ecnt [W, E/W] dense."""
    if (send_rank is None) != (send_ecnt is None):
        raise ValueError("send_rank and send_ecnt go together")
    if send_rank is None:
        return
    _shape(send_rank, tuple(send_eloc.shape), "send_rank", _I32T)
    _dense_from(send_rank, 1, "send_rank")
    if send_rank.stride(0) != send_eloc.stride(0):
        raise ValueError("send_rank and send_eloc must share a rank stride")
    _shape(send_ecnt, (W, E // W), "send_ecnt", _I32T)
    _dense_from(send_ecnt, 0, "send_ecnt")


def _send_side(topk_ids, topk_weights, E, W, max_num_tokens, send_cnt, send_eloc,
               send_w, token_slot, err_flags):
    """Checks the routing inputs and metadata outputs of a pack call;
    returns (T, K, cap, slots). send_eloc / send_w: [W, cap, slots] with a
    free rank stride, shared by both."""
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T, K]")
    T, K = topk_ids.shape
    _, slots, cap, _ = _sizes(K, E, W, max_num_tokens)
    _shape(topk_ids, (T, K), "topk_ids", _I32T)
    _shape(topk_weights, (T, K), "topk_weights", _F32T)
    _dense_from(topk_ids, 0, "topk_ids")
    _dense_from(topk_weights, 0, "topk_weights")
    _vector(send_cnt, W, "send_cnt", _I32T)
    _dense_from(send_cnt, 0, "send_cnt")
    _blocks(send_eloc, W, cap * slots, "send_eloc", _I32T)
    _blocks(send_w, W, cap * slots, "send_w", _F32T)
    if send_eloc.stride(0) != send_w.stride(0):
        raise ValueError("send_eloc and send_w must share a rank stride")
    _shape(token_slot, (T, W), "token_slot", _I32T)
    _dense_from(token_slot, 0, "token_slot")
    _err(err_flags)
    return T, K, cap, slots


def _receive_side(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens):
    """Checks the received counts and local ids; returns (slots, cap,
    expert_cap)."""
    _, slots, cap, ecap = _sizes(K, e_local * W, W, max_num_tokens)
    _vector(recv_cnt, W, "recv_cnt", _I32T)
    _blocks(recv_eloc, W, cap * slots, "recv_eloc", _I32T)
    return slots, cap, ecap


class PreparedCall:
    """One call of the library with its arguments marshalled once; calling
    it passes them unchanged with the stream of the moment. It keeps the
    tensors (and the payload descriptor array) it points into alive. Every
    tensor must be on one GPU (the library takes device pointers only), and
    the stream of a call must belong to that GPU."""

    def __init__(self, name: str, args: tuple, keep: tuple):
        devices = {t.device for t in _tensors(keep)}
        if any(d.type != "cuda" for d in devices) or len(devices) > 1:
            raise ValueError(f"{name}: every tensor must be on one GPU, got "
                             f"{sorted(str(d) for d in devices)}")
        self.device = devices.pop().index if devices else None
        self.name = name
        self.fn = getattr(load(), name)
        self.args = args
        self.keep = keep

    def __call__(self, stream=None) -> None:
        if self.device is not None and not isinstance(stream, int):
            dev = (torch.cuda.current_device() if stream is None
                   else stream.device.index)
            if dev != self.device:
                raise ValueError(f"{self.name}: the stream is on cuda:{dev}, the "
                                 f"tensors on cuda:{self.device}")
        _check(self.name, self.fn(*self.args, _stream(stream)))


def _tensors(x):
    """The tensors in a nest of tuples and lists."""
    if isinstance(x, torch.Tensor):
        yield x
    elif isinstance(x, (tuple, list)):
        for y in x:
            yield from _tensors(y)


def _ws_bytes(workspace: torch.Tensor) -> int:
    return workspace.numel() * workspace.element_size()


def prepare_dispatch_pack(topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                          E: int, W: int, max_num_tokens: int,
                          payloads: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                          send_cnt: torch.Tensor, send_eloc: torch.Tensor,
                          send_w: torch.Tensor, token_slot: torch.Tensor,
                          err_flags: Optional[torch.Tensor],
                          workspace: torch.Tensor,
                          send_rank: Optional[torch.Tensor] = None,
                          send_ecnt: Optional[torch.Tensor] = None) -> PreparedCall:
    """payloads: (src [T, ...], dst [W, cap, ...]) pairs; send_eloc /
    send_w: [W, cap, slots] with one free rank stride (meta_rank_stride);
    the rank stride of each dst is free, everything below it dense.
    send_rank (like send_eloc) and send_ecnt [W, e_local]: the optional
    per-expert ranks for moe_ep_expert_batch_ranked."""
    T, K, cap, _ = _send_side(topk_ids, topk_weights, E, W, max_num_tokens, send_cnt,
                              send_eloc, send_w, token_slot, err_flags)
    _ranks(send_rank, send_ecnt, send_eloc, W, E)
    arr = _payload_array(payloads, 1, 2, (T,), (W, cap))
    args = (_ptr(topk_ids), _ptr(topk_weights), T, K, E, W, max_num_tokens,
            ctypes.addressof(arr), len(payloads), _ptr(send_cnt), _ptr(send_eloc),
            _ptr(send_w), send_eloc.stride(0), _ptr(send_rank), _ptr(send_ecnt),
            _ptr(token_slot), _ptr(err_flags), _ptr(workspace), _ws_bytes(workspace))
    return PreparedCall("moe_ep_dispatch_pack", args,
                        (arr, topk_ids, topk_weights, payloads, send_cnt, send_eloc,
                         send_w, send_rank, send_ecnt, token_slot, err_flags, workspace))


def prepare_dispatch_pack_noalloc(topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                                  E: int, W: int, max_num_tokens: int,
                                  payloads: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                                  send_cnt: torch.Tensor, send_eloc: torch.Tensor,
                                  send_w: torch.Tensor, token_slot: torch.Tensor,
                                  err_flags: Optional[torch.Tensor],
                                  send_rank: Optional[torch.Tensor] = None,
                                  send_ecnt: Optional[torch.Tensor] = None) -> PreparedCall:
    """moe_ep_dispatch_pack without a workspace: the library's own device
    scratch holds the send side's workspace (moe_ep_dispatch_pack_noalloc;
    calls that overlap on one GPU race on it)."""
    T, K, cap, _ = _send_side(topk_ids, topk_weights, E, W, max_num_tokens, send_cnt,
                              send_eloc, send_w, token_slot, err_flags)
    _ranks(send_rank, send_ecnt, send_eloc, W, E)
    arr = _payload_array(payloads, 1, 2, (T,), (W, cap))
    args = (_ptr(topk_ids), _ptr(topk_weights), T, K, E, W, max_num_tokens,
            ctypes.addressof(arr), len(payloads), _ptr(send_cnt), _ptr(send_eloc),
            _ptr(send_w), send_eloc.stride(0), _ptr(send_rank), _ptr(send_ecnt),
            _ptr(token_slot), _ptr(err_flags))
    return PreparedCall("moe_ep_dispatch_pack_noalloc", args,
                        (arr, topk_ids, topk_weights, payloads, send_cnt, send_eloc,
                         send_w, send_rank, send_ecnt, token_slot, err_flags))


def moe_ep_dispatch_pack_noalloc(topk_ids, topk_weights, E, W, max_num_tokens, payloads,
                                 send_cnt, send_eloc, send_w, token_slot, err_flags,
                                 stream=None, send_rank=None, send_ecnt=None) -> None:
    prepare_dispatch_pack_noalloc(topk_ids, topk_weights, E, W, max_num_tokens, payloads,
                                  send_cnt, send_eloc, send_w, token_slot, err_flags,
                                  send_rank, send_ecnt)(stream)


def scale_pitch(H: int, group: int) -> int:
    """fp32 scales per row of the quantised layout: H/group rounded up to 4."""
    return (H // group + 3) // 4 * 4


def prepare_dispatch_pack_fp8(topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                              E: int, W: int, max_num_tokens: int,
                              hidden: torch.Tensor, group: int,
                              send_q: torch.Tensor, send_scale: torch.Tensor,
                              payloads: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                              send_cnt: torch.Tensor, send_eloc: torch.Tensor,
                              send_w: torch.Tensor, token_slot: torch.Tensor,
                              err_flags: Optional[torch.Tensor],
                              workspace: torch.Tensor,
                              send_rank: Optional[torch.Tensor] = None,
                              send_ecnt: Optional[torch.Tensor] = None) -> PreparedCall:
    """hidden: bf16 [T, H] (token stride free, rows dense); send_q: fp8 codes
    [W, cap, H] (uint8 or float8, rank stride free); send_scale: fp32
    [W, cap, Gp], Gp = H/group rounded up to 4 (rank stride free)."""
    T, K, cap, _ = _send_side(topk_ids, topk_weights, E, W, max_num_tokens, send_cnt,
                              send_eloc, send_w, token_slot, err_flags)
    _ranks(send_rank, send_ecnt, send_eloc, W, E)
    if hidden.dtype != torch.bfloat16:
        raise ValueError("hidden must be bfloat16")
    if hidden.dim() != 2 or hidden.size(0) < T:
        raise ValueError("hidden must be [T, H]")
    _dense_from(hidden, 1, "hidden")
    H = hidden.size(1)
    if group <= 0:
        raise ValueError("group must be positive")
    if send_q.element_size() != 1:
        raise ValueError("send_q must hold one byte per code")
    _shape(send_q, (W, cap, H), "send_q")
    _shape(send_scale, (W, cap, scale_pitch(H, group)), "send_scale", _F32T)
    _dense_from(send_q, 1, "send_q")
    _dense_from(send_scale, 1, "send_scale")
    arr = _payload_array(payloads, 1, 2, (T,), (W, cap))
    args = (_ptr(topk_ids), _ptr(topk_weights), T, K, E, W, max_num_tokens,
            _ptr(hidden), hidden.stride(0) * 2, H, group,
            _ptr(send_q), send_q.stride(0) * send_q.element_size(),
            _ptr(send_scale), send_scale.stride(0),
            ctypes.addressof(arr), len(payloads), _ptr(send_cnt), _ptr(send_eloc),
            _ptr(send_w), send_eloc.stride(0), _ptr(send_rank), _ptr(send_ecnt),
            _ptr(token_slot), _ptr(err_flags), _ptr(workspace), _ws_bytes(workspace))
    return PreparedCall("moe_ep_dispatch_pack_fp8", args,
                        (arr, topk_ids, topk_weights, hidden, send_q, send_scale,
                         payloads, send_cnt, send_eloc, send_w, send_rank, send_ecnt,
                         token_slot, err_flags, workspace))


def moe_ep_dispatch_pack_fp8(topk_ids, topk_weights, E, W, max_num_tokens, hidden,
                             group, send_q, send_scale, payloads, send_cnt,
                             send_eloc, send_w, token_slot, err_flags, workspace,
                             stream=None) -> None:
    prepare_dispatch_pack_fp8(topk_ids, topk_weights, E, W, max_num_tokens, hidden,
                              group, send_q, send_scale, payloads, send_cnt,
                              send_eloc, send_w, token_slot, err_flags,
                              workspace)(stream)


def fp4_scale_pitch(H: int) -> int:
    """Bytes of a 4-bit row's scale row: H/16 rounded up to 16."""
    return (H // 16 + 15) // 16 * 16


def prepare_dispatch_pack_fp4(topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                              E: int, W: int, max_num_tokens: int,
                              hidden: torch.Tensor, send_q: torch.Tensor,
                              send_scale: torch.Tensor,
                              payloads: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                              send_cnt: torch.Tensor, send_eloc: torch.Tensor,
                              send_w: torch.Tensor, token_slot: torch.Tensor,
                              err_flags: Optional[torch.Tensor],
                              workspace: torch.Tensor,
                              send_rank: Optional[torch.Tensor] = None,
                              send_ecnt: Optional[torch.Tensor] = None) -> PreparedCall:
    """hidden: bf16 [T, H] (token stride free, rows dense); send_q: codes
    [W, cap, H/2] bytes; send_scale: e4m3 scale codes [W, cap, Sp] bytes,
    Sp = fp4_scale_pitch(H) (rank strides free)."""
    T, K, cap, _ = _send_side(topk_ids, topk_weights, E, W, max_num_tokens, send_cnt,
                              send_eloc, send_w, token_slot, err_flags)
    _ranks(send_rank, send_ecnt, send_eloc, W, E)
    if hidden.dtype != torch.bfloat16:
        raise ValueError("hidden must be bfloat16")
    if hidden.dim() != 2 or hidden.size(0) < T:
        raise ValueError("hidden must be [T, H]")
    for t, n in ((hidden, "hidden"), (send_q, "send_q"), (send_scale, "send_scale")):
        _dense_from(t, 1, n)
    H = hidden.size(1)
    if send_q.dim() != 3 or send_scale.dim() != 3:
        raise ValueError("send_q and send_scale must be [W, cap, bytes]")
    if tuple(send_q.shape[:2]) != (W, cap) or tuple(send_scale.shape[:2]) != (W, cap):
        raise ValueError("send_q and send_scale must have W x cap rows")
    if send_q.size(-1) * send_q.element_size() != H // 2:
        raise ValueError("send_q rows must hold H/2 bytes")
    if send_scale.size(-1) * send_scale.element_size() != fp4_scale_pitch(H):
        raise ValueError("send_scale rows must hold fp4_scale_pitch(H) bytes")
    arr = _payload_array(payloads, 1, 2, (T,), (W, cap))
    args = (_ptr(topk_ids), _ptr(topk_weights), T, K, E, W, max_num_tokens,
            _ptr(hidden), hidden.stride(0) * 2, H,
            _ptr(send_q), send_q.stride(0) * send_q.element_size(),
            _ptr(send_scale), send_scale.stride(0) * send_scale.element_size(),
            ctypes.addressof(arr), len(payloads), _ptr(send_cnt), _ptr(send_eloc),
            _ptr(send_w), send_eloc.stride(0), _ptr(send_rank), _ptr(send_ecnt),
            _ptr(token_slot), _ptr(err_flags), _ptr(workspace), _ws_bytes(workspace))
    return PreparedCall("moe_ep_dispatch_pack_fp4", args,
                        (arr, topk_ids, topk_weights, hidden, send_q, send_scale,
                         payloads, send_cnt, send_eloc, send_w, send_rank, send_ecnt,
                         token_slot, err_flags, workspace))


def moe_ep_dispatch_pack_fp4(topk_ids, topk_weights, E, W, max_num_tokens, hidden,
                             send_q, send_scale, payloads, send_cnt, send_eloc,
                             send_w, token_slot, err_flags, workspace,
                             stream=None) -> None:
    prepare_dispatch_pack_fp4(topk_ids, topk_weights, E, W, max_num_tokens, hidden,
                              send_q, send_scale, payloads, send_cnt, send_eloc,
                              send_w, token_slot, err_flags, workspace)(stream)


def moe_ep_dispatch_pack(topk_ids, topk_weights, E, W, max_num_tokens, payloads,
                         send_cnt, send_eloc, send_w, token_slot, err_flags,
                         workspace, stream=None, send_rank=None, send_ecnt=None) -> None:
    prepare_dispatch_pack(topk_ids, topk_weights, E, W, max_num_tokens, payloads,
                          send_cnt, send_eloc, send_w, token_slot, err_flags,
                          workspace, send_rank, send_ecnt)(stream)


def prepare_expert_batch(recv_cnt: torch.Tensor, recv_eloc: torch.Tensor,
                         W: int, e_local: int, K: int, max_num_tokens: int,
                         payloads: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                         expert_num_tokens: torch.Tensor, recv_row: torch.Tensor,
                         err_flags: Optional[torch.Tensor],
                         workspace: torch.Tensor) -> PreparedCall:
    """recv_cnt: [W] view (any stride); recv_eloc: [W, cap, slots] view (rank
    stride free); payloads: (src [W, cap, ...], dst [e_local, W*cap, ...])."""
    slots, cap, ecap = _receive_side(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens)
    _shape(recv_row, (W, cap, slots), "recv_row", _I32T)
    _dense_from(recv_row, 0, "recv_row")
    _shape(expert_num_tokens, (e_local,), "expert_num_tokens", _I32T)
    _dense_from(expert_num_tokens, 0, "expert_num_tokens")
    _err(err_flags)
    arr = _payload_array(payloads, 2, 2, (W, cap), (e_local, ecap))
    args = (_ptr(recv_cnt), recv_cnt.stride(0), _ptr(recv_eloc), recv_eloc.stride(0),
            W, e_local, K, max_num_tokens, ctypes.addressof(arr), len(payloads),
            _ptr(expert_num_tokens), _ptr(recv_row), _ptr(err_flags), _ptr(workspace),
            _ws_bytes(workspace))
    return PreparedCall("moe_ep_expert_batch", args,
                        (arr, recv_cnt, recv_eloc, payloads, expert_num_tokens,
                         recv_row, err_flags, workspace))


def moe_ep_expert_batch(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens,
                        payloads, expert_num_tokens, recv_row, err_flags,
                        workspace, stream=None) -> None:
    prepare_expert_batch(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens,
                         payloads, expert_num_tokens, recv_row, err_flags,
                         workspace)(stream)


def prepare_expert_batch_ranked(recv_cnt: torch.Tensor, recv_eloc: torch.Tensor,
                                recv_rank: torch.Tensor, recv_ecnt: torch.Tensor,
                                W: int, e_local: int, K: int, max_num_tokens: int,
                                payloads: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                                expert_num_tokens: torch.Tensor, recv_row: torch.Tensor,
                                err_flags: Optional[torch.Tensor]) -> PreparedCall:
    """moe_ep_expert_batch from the sources' per-expert ranks: recv_rank
    [W, cap, slots] with recv_eloc's rank stride; recv_ecnt [W, e_local]
    (rank stride free, rows dense). No workspace."""
    slots, cap, ecap = _receive_side(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens)
    _blocks(recv_rank, W, cap * slots, "recv_rank", _I32T)
    if recv_rank.stride(0) != recv_eloc.stride(0):
        raise ValueError("recv_rank and recv_eloc must share a rank stride")
    _shape(recv_ecnt, (W, e_local), "recv_ecnt", _I32T)
    _dense_from(recv_ecnt, 1, "recv_ecnt")
    _shape(recv_row, (W, cap, slots), "recv_row", _I32T)
    _dense_from(recv_row, 0, "recv_row")
    _shape(expert_num_tokens, (e_local,), "expert_num_tokens", _I32T)
    _dense_from(expert_num_tokens, 0, "expert_num_tokens")
    _err(err_flags)
    arr = _payload_array(payloads, 2, 2, (W, cap), (e_local, ecap))
    args = (_ptr(recv_cnt), recv_cnt.stride(0), _ptr(recv_eloc), _ptr(recv_rank),
            recv_eloc.stride(0), _ptr(recv_ecnt), recv_ecnt.stride(0), W, e_local, K,
            max_num_tokens, ctypes.addressof(arr), len(payloads), _ptr(expert_num_tokens),
            _ptr(recv_row), _ptr(err_flags))
    return PreparedCall("moe_ep_expert_batch_ranked", args,
                        (arr, recv_cnt, recv_eloc, recv_rank, recv_ecnt, payloads,
                         expert_num_tokens, recv_row, err_flags))


def moe_ep_expert_batch_ranked(recv_cnt, recv_eloc, recv_rank, recv_ecnt, W, e_local, K,
                               max_num_tokens, payloads, expert_num_tokens, recv_row,
                               err_flags, stream=None) -> None:
    prepare_expert_batch_ranked(recv_cnt, recv_eloc, recv_rank, recv_ecnt, W, e_local, K,
                                max_num_tokens, payloads, expert_num_tokens, recv_row,
                                err_flags)(stream)


def prepare_expert_batch_plan(recv_cnt: torch.Tensor, recv_eloc: torch.Tensor,
                              W: int, e_local: int, K: int, max_num_tokens: int,
                              expert_num_tokens: torch.Tensor, recv_row: torch.Tensor,
                              err_flags: Optional[torch.Tensor],
                              workspace: torch.Tensor) -> PreparedCall:
    """The receive scan half of moe_ep_expert_batch."""
    slots, cap, _ = _receive_side(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens)
    _shape(recv_row, (W, cap, slots), "recv_row", _I32T)
    _dense_from(recv_row, 0, "recv_row")
    _shape(expert_num_tokens, (e_local,), "expert_num_tokens", _I32T)
    _dense_from(expert_num_tokens, 0, "expert_num_tokens")
    _err(err_flags)
    args = (_ptr(recv_cnt), recv_cnt.stride(0), _ptr(recv_eloc), recv_eloc.stride(0),
            W, e_local, K, max_num_tokens, _ptr(expert_num_tokens), _ptr(recv_row),
            _ptr(err_flags), _ptr(workspace), _ws_bytes(workspace))
    return PreparedCall("moe_ep_expert_batch_plan", args,
                        (recv_cnt, recv_eloc, expert_num_tokens, recv_row,
                         err_flags, workspace))


def prepare_expert_batch_copy(recv_cnt: torch.Tensor, recv_eloc: torch.Tensor,
                              W: int, e_local: int, K: int, max_num_tokens: int,
                              payloads: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                              recv_row: torch.Tensor,
                              err_flags: Optional[torch.Tensor],
                              workspace: torch.Tensor) -> PreparedCall:
    """The row copy half of moe_ep_expert_batch (after the plan)."""
    slots, cap, ecap = _receive_side(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens)
    _shape(recv_row, (W, cap, slots), "recv_row", _I32T)
    _dense_from(recv_row, 0, "recv_row")
    _err(err_flags)
    arr = _payload_array(payloads, 2, 2, (W, cap), (e_local, ecap))
    args = (_ptr(recv_cnt), recv_cnt.stride(0), _ptr(recv_eloc), recv_eloc.stride(0),
            W, e_local, K, max_num_tokens, ctypes.addressof(arr), len(payloads),
            _ptr(recv_row), _ptr(err_flags), _ptr(workspace), _ws_bytes(workspace))
    return PreparedCall("moe_ep_expert_batch_copy", args,
                        (arr, recv_cnt, recv_eloc, payloads, recv_row, err_flags,
                         workspace))


def moe_ep_expert_batch_plan(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens,
                             expert_num_tokens, recv_row, err_flags, workspace,
                             stream=None) -> None:
    prepare_expert_batch_plan(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens,
                              expert_num_tokens, recv_row, err_flags, workspace)(stream)


def moe_ep_expert_batch_copy(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens,
                             payloads, recv_row, err_flags, workspace,
                             stream=None) -> None:
    prepare_expert_batch_copy(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens,
                              payloads, recv_row, err_flags, workspace)(stream)


def prepare_sanitize_expert_ids(recv_cnt: torch.Tensor, recv_eloc: torch.Tensor,
                                W: int, e_local: int, K: int, max_num_tokens: int,
                                invalid_id: int, out: torch.Tensor,
                                err_flags: Optional[torch.Tensor]) -> PreparedCall:
    """recv_eloc / out: [W, cap, slots] views (rank stride free); out may be
    recv_eloc itself."""
    slots, cap, _ = _receive_side(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens)
    _blocks(out, W, cap * slots, "out", _I32T)
    _err(err_flags)
    args = (_ptr(recv_cnt), recv_cnt.stride(0), _ptr(recv_eloc), recv_eloc.stride(0),
            W, e_local, K, max_num_tokens, invalid_id, _ptr(out), out.stride(0),
            _ptr(err_flags))
    return PreparedCall("moe_ep_sanitize_expert_ids", args,
                        (recv_cnt, recv_eloc, out, err_flags))


def moe_ep_sanitize_expert_ids(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens,
                               invalid_id, out, err_flags=None, stream=None) -> None:
    prepare_sanitize_expert_ids(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens,
                                invalid_id, out, err_flags)(stream)


def prepare_combine_reduce(expert_out: torch.Tensor, recv_cnt: torch.Tensor,
                           recv_eloc: torch.Tensor, recv_w: torch.Tensor,
                           recv_row: torch.Tensor, W: int, e_local: int, K: int,
                           max_num_tokens: int, ret: torch.Tensor,
                           self_src: Optional[int] = None) -> PreparedCall:
    """expert_out: [e_local, W*cap, H] (expert stride free, rows dense);
    recv_eloc / recv_w: [W, cap, slots] views with one rank stride;
    ret: [W, cap, H] view (rank stride free). With self_src, the call is
    moe_ep_combine_reduce_peers (that source's block is skipped)."""
    dt = _dtype_code(expert_out)
    if ret.dtype != expert_out.dtype:
        raise ValueError("ret and expert_out differ in dtype")
    slots, cap, ecap = _receive_side(recv_cnt, recv_eloc, W, e_local, K, max_num_tokens)
    _blocks(recv_w, W, cap * slots, "recv_w", _F32T)
    if recv_eloc.stride(0) != recv_w.stride(0):
        raise ValueError("recv_eloc and recv_w must share a rank stride")
    _shape(recv_row, (W, cap, slots), "recv_row", _I32T)
    _dense_from(recv_row, 0, "recv_row")
    if expert_out.dim() != 3:
        raise ValueError("expert_out must be [e_local, W*cap, H]")
    H = expert_out.size(2)
    _lead_at_least(expert_out, (e_local, ecap), "expert_out")
    _shape(ret, (W, cap, H), "ret")
    _dense_from(expert_out, 1, "expert_out")
    _dense_from(ret, 1, "ret")
    head = (_ptr(expert_out), expert_out.stride(0), dt, H, _ptr(recv_cnt),
            recv_cnt.stride(0), _ptr(recv_eloc), _ptr(recv_w), recv_eloc.stride(0),
            _ptr(recv_row), W, e_local, K, max_num_tokens)
    keep = (expert_out, recv_cnt, recv_eloc, recv_w, recv_row, ret)
    if self_src is None:
        return PreparedCall("moe_ep_combine_reduce",
                            head + (_ptr(ret), ret.stride(0)), keep)
    return PreparedCall("moe_ep_combine_reduce_peers",
                        head + (self_src, _ptr(ret), ret.stride(0)), keep)


def moe_ep_combine_reduce(expert_out, recv_cnt, recv_eloc, recv_w, recv_row, W,
                          e_local, K, max_num_tokens, ret, stream=None) -> None:
    prepare_combine_reduce(expert_out, recv_cnt, recv_eloc, recv_w, recv_row, W,
                           e_local, K, max_num_tokens, ret)(stream)


def _unpack_side(back: torch.Tensor, token_slot: torch.Tensor, max_num_tokens: int,
                 out: torch.Tensor):
    """Checks the returned partials, the context and the output of an
    unpack; returns (T, W, H)."""
    if token_slot.dim() != 2:
        raise ValueError("token_slot must be [T, W]")
    T, W = token_slot.shape
    if back.dim() != 3:
        raise ValueError("back must be [W, cap, H]")
    H = back.size(2)
    _shape(back, (W, max_num_tokens, H), "back")
    _shape(token_slot, (T, W), "token_slot", _I32T)
    _shape(out, (T, H), "out")
    _dense_from(back, 1, "back")
    _dense_from(token_slot, 0, "token_slot")
    _dense_from(out, 0, "out")
    return T, W, H


def prepare_combine_unpack(back: torch.Tensor, token_slot: torch.Tensor,
                           max_num_tokens: int, out: torch.Tensor) -> PreparedCall:
    """back: [W, cap, H] view (rank stride free); token_slot: [T, W];
    out: [T, H] dense."""
    dt = _dtype_code(back)
    if out.dtype != back.dtype:
        raise ValueError("out and back differ in dtype")
    T, W, H = _unpack_side(back, token_slot, max_num_tokens, out)
    args = (_ptr(back), back.stride(0), dt, H, _ptr(token_slot), T, W,
            max_num_tokens, _ptr(out))
    return PreparedCall("moe_ep_combine_unpack", args, (back, token_slot, out))


def moe_ep_combine_unpack(back, token_slot, max_num_tokens, out, stream=None) -> None:
    prepare_combine_unpack(back, token_slot, max_num_tokens, out)(stream)


def moe_ep_combine_reduce_peers(expert_out, recv_cnt, recv_eloc, recv_w, recv_row, W,
                                e_local, K, max_num_tokens, self_src, ret,
                                stream=None) -> None:
    prepare_combine_reduce(expert_out, recv_cnt, recv_eloc, recv_w, recv_row, W,
                           e_local, K, max_num_tokens, ret, self_src)(stream)


def prepare_combine_unpack_fused(back: torch.Tensor, token_slot: torch.Tensor,
                                 max_num_tokens: int, self_rank: int,
                                 expert_out: torch.Tensor, self_eloc: torch.Tensor,
                                 self_w: torch.Tensor, self_row: torch.Tensor,
                                 e_local: int, K: int, out: torch.Tensor) -> PreparedCall:
    """back: [W, cap, H] view; token_slot: [T, W]; expert_out: the rank's own
    [e_local, W*cap, H]; self_eloc / self_w / self_row: [cap, slots] dense
    blocks of the rank's own source; out: [T, H] dense."""
    dt = _dtype_code(back)
    if out.dtype != back.dtype or expert_out.dtype != back.dtype:
        raise ValueError("out, back and expert_out must share a dtype")
    T, W, H = _unpack_side(back, token_slot, max_num_tokens, out)
    _, slots, cap, ecap = _sizes(K, e_local * W, W, max_num_tokens)
    if expert_out.dim() != 3 or expert_out.size(2) != H:
        raise ValueError("expert_out must be [e_local, W*cap, H]")
    _lead_at_least(expert_out, (e_local, ecap), "expert_out")
    _dense_from(expert_out, 1, "expert_out")
    for t, n, dts in ((self_eloc, "self_eloc", _I32T), (self_w, "self_w", _F32T),
                      (self_row, "self_row", _I32T)):
        _shape(t, (cap, slots), n, dts)
        _dense_from(t, 0, n)
    args = (_ptr(back), back.stride(0), dt, H, _ptr(token_slot), T, W,
            max_num_tokens, self_rank, _ptr(expert_out), expert_out.stride(0),
            _ptr(self_eloc), _ptr(self_w), _ptr(self_row), e_local, K, _ptr(out))
    return PreparedCall("moe_ep_combine_unpack_fused", args,
                        (back, token_slot, expert_out, self_eloc, self_w, self_row, out))


def moe_ep_combine_unpack_fused(back, token_slot, max_num_tokens, self_rank, expert_out,
                                self_eloc, self_w, self_row, e_local, K, out,
                                stream=None) -> None:
    prepare_combine_unpack_fused(back, token_slot, max_num_tokens, self_rank, expert_out,
                                 self_eloc, self_w, self_row, e_local, K, out)(stream)
