"""The C-ABI library loads without a GPU, exports every symbol that
include/moe_ep.h declares, and rejects bad arguments with the documented
status codes before anything reaches the GPU (no valid compute call is made
here)."""
import ctypes
import os
import re
import subprocess

import pytest

from combine_topk_ids_dest_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ep.h")

# An address the checks accept as a 16-byte aligned device pointer; no call
# below passes every check, so it is never dereferenced.
FAKE = 0x7F0000000000


def _header():
    return open(HEADER).read()


def _declared():
    return re.findall(r"MOE_EP_API\s+[\w\s\*]*?\b(moe_ep_\w+)\s*\(", _header())


def _defines():
    return {m.group(1): int(m.group(2).rstrip("u"))
            for m in re.finditer(r"#define\s+(MOE_EP_\w+)\s+(-?\d+u?)", _header())}


def test_library_loads_and_exports_every_declared_symbol():
    lib = B.load()
    declared = _declared()
    assert sorted(declared) == sorted(B.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared)


def test_python_constants_match_header():
    d = _defines()
    assert (d["MOE_EP_OK"], d["MOE_EP_EINVAL"], d["MOE_EP_ECAP"],
            d["MOE_EP_EDTYPE"], d["MOE_EP_EALIGN"], d["MOE_EP_EWORKSPACE"],
            d["MOE_EP_EHIP"], d["MOE_EP_ESCRATCH"]) == \
        (B.OK, B.EINVAL, B.ECAP, B.EDTYPE, B.EALIGN, B.EWORKSPACE, B.EHIP, B.ESCRATCH)
    m = re.search(r"#define\s+MOE_EP_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)",
                  _header())
    assert int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES
    assert (d["MOE_EP_BF16"], d["MOE_EP_F32"]) == (B.BF16, B.F32)
    assert (d["MOE_EP_ERR_ID_RANGE"], d["MOE_EP_ERR_PICKS"], d["MOE_EP_ERR_ELOC"],
            d["MOE_EP_ERR_ROWCAP"], d["MOE_EP_ERR_CNT"]) == \
        (B.ERR_ID_RANGE, B.ERR_PICKS, B.ERR_ELOC, B.ERR_ROWCAP, B.ERR_CNT)
    assert d["MOE_EP_MAX_PAYLOADS"] == B.MAX_PAYLOADS
    assert ctypes.sizeof(B.MoeEpPayload) == 40


def test_capacities_and_workspace():
    assert B.moe_ep_capacities(8, 256, 8, 4096) == (4096, 8, 32768)
    assert B.moe_ep_capacities(2, 8, 8, 8192) == (8192, 1, 65536)
    assert B.moe_ep_capacities(8, 256, 32, 128) == (128, 8, 4096)
    for bad in [(0, 8, 2, 4), (2, 0, 2, 4), (2, 8, 0, 4), (2, 9, 2, 4), (2, 8, 2, -1)]:
        with pytest.raises(B.MoeEpError) as e:
            B.moe_ep_capacities(*bad)
        assert e.value.status == B.EINVAL
    ws = B.moe_ep_workspace_bytes(4096, 8, 256, 8, 4096)
    assert ws > 0 and ws % 128 == 0
    # send side: 16 token tiles x 8 ranks (counts and offsets, each padded to
    # 128 B) + in-tile ranks [4096, 8], and for the per-expert ranks the
    # picks' in-tile ranks [4096 * 8] and 16 tiles x 256 experts (counts and
    # offsets); receive side: 8*4096*8/1024 tiles x 32 experts x 4 B x 2.
    # The larger wins.
    send = 2 * 512 + 4096 * 8 * 4 + 4096 * 8 * 4 + 2 * 16 * 256 * 4
    recv = 256 * 32 * 4 * 2
    assert ws == max(send, recv) == send
    with pytest.raises(B.MoeEpError) as e:
        B.moe_ep_workspace_bytes(5000, 8, 256, 8, 4096)
    assert e.value.status == B.ECAP
    with pytest.raises(B.MoeEpError) as e:
        B.moe_ep_workspace_bytes(10, 8, 256, 128, 4096)    # W > 64
    assert e.value.status == B.EINVAL
    # huge max_num_tokens: rejected before any product can overflow (the
    # sanitizer run of these tests would report a signed overflow)
    big = 1 << 62
    assert B.moe_ep_capacities(8, 256, 1, big) == (big, 8, big)
    for bad in [(8, 256, 8, big), (8, 256, 8, (1 << 63) - 1)]:
        with pytest.raises(B.MoeEpError) as e:
            B.moe_ep_capacities(*bad)
        assert e.value.status == B.EINVAL
    for mnt in (big, (1 << 31)):
        with pytest.raises(B.MoeEpError) as e:
            B.moe_ep_workspace_bytes(0, 8, 256, 8, mnt)
        assert e.value.status == B.EINVAL
    assert B.moe_ep_workspace_bytes(0, 1, 64, 64, (1 << 31) - 1 >> 6) > 0


def test_status_strings():
    for code in (B.OK, B.EINVAL, B.ECAP, B.EDTYPE, B.EALIGN, B.EWORKSPACE, B.EHIP,
                 B.ESCRATCH):
        s = B.status_string(code)
        assert s and s != "unknown status"
    assert B.status_string(12345) == "unknown status"


def _payloads(*descs):
    arr = (B.MoeEpPayload * 8)()
    for i, (src, ss, dst, ds, rb) in enumerate(descs):
        arr[i].src, arr[i].src_stride = src, ss
        arr[i].dst, arr[i].dst_stride = dst, ds
        arr[i].row_bytes = rb
    return arr


def _pack(T=16, K=2, E=8, W=4, cap=16, pl=None, npl=1, ws_bytes=1 << 20,
          ws=FAKE, ids=FAKE, meta=None, rank=None, ecnt=None):
    lib = B.load()
    if pl is None:
        pl = _payloads((FAKE, 512, FAKE, cap * 512, 512))
    if meta is None:
        meta = cap * min(K, E // W) if W > 0 and E % W == 0 else 0
    return lib.moe_ep_dispatch_pack(ids, FAKE, T, K, E, W, cap,
                                    ctypes.addressof(pl), npl, FAKE, FAKE,
                                    FAKE, meta, rank, ecnt, FAKE, None, ws, ws_bytes, None)


def test_dispatch_pack_argument_checks():
    assert _pack(W=0) == B.EINVAL
    assert _pack(W=65, E=65 * 2) == B.EINVAL
    assert _pack(E=9) == B.EINVAL                       # E % W != 0
    assert _pack(K=0) == B.EINVAL
    assert _pack(T=17) == B.ECAP                        # T > max_num_tokens
    assert _pack(T=-1) == B.EINVAL
    assert _pack(npl=9) == B.EINVAL
    assert _pack(ids=None) == B.EINVAL
    assert _pack(pl=_payloads((FAKE, 520, FAKE, 16 * 520, 520))) == B.EALIGN
    assert _pack(pl=_payloads((FAKE + 8, 512, FAKE, 16 * 512, 512))) == B.EALIGN
    assert _pack(pl=_payloads((FAKE, 256, FAKE, 16 * 512, 512))) == B.EINVAL
    assert _pack(pl=_payloads((FAKE, 512, FAKE, 15 * 512, 512))) == B.EINVAL
    assert _pack(pl=_payloads((FAKE, 512, FAKE, 16 * 512, 0))) == B.EINVAL
    assert _pack(ws_bytes=8) == B.EWORKSPACE
    assert _pack(ws=None) == B.EWORKSPACE
    assert _pack(ws=FAKE + 4) == B.EALIGN
    assert _pack(K=65, E=65 * 4) == B.EINVAL           # slots > 64
    # size limit W * cap * slots < 2^31
    assert _pack(T=0, cap=1 << 28, K=8, E=64, W=8) == B.EINVAL
    # metadata blocks: at least cap * slots elements apart, and the offset
    # of the last one must not overflow
    assert _pack(meta=16 * 2 - 1) == B.EINVAL
    assert _pack(meta=-1) == B.EINVAL
    assert _pack(meta=(1 << 63) // 3) == B.EINVAL
    # per-expert ranks: both outputs or neither, K <= 16 and E <= 4096; the
    # workspace must hold the ranks' tables too
    assert _pack(rank=FAKE) == B.EINVAL
    assert _pack(ecnt=FAKE) == B.EINVAL
    assert _pack(rank=FAKE, ecnt=FAKE, K=17, E=4 * 32) == B.EINVAL
    assert _pack(rank=FAKE, ecnt=FAKE, K=2, E=8 * 520, W=8) == B.EINVAL
    T, W = 600, 4
    r128 = lambda x: (x + 127) // 128 * 128
    plain = 2 * r128(3 * W * 4) + r128(T * W * 4)
    ranked = plain + r128(T * 2 * 4) + 2 * r128(3 * 8 * 4)
    assert _pack(T=T, cap=T, ws_bytes=plain, rank=FAKE, ecnt=FAKE) == B.EWORKSPACE
    assert _pack(T=T, cap=T, ws_bytes=ranked - 1, rank=FAKE, ecnt=FAKE) == B.EWORKSPACE
    assert B.moe_ep_workspace_bytes(T, 2, 8, W, T) == ranked


def _pack_noalloc(T=16, K=2, E=8, W=4, cap=16, npl=1, meta=None, rank=None, ecnt=None):
    lib = B.load()
    pl = _payloads((FAKE, 512, FAKE, cap * 512, 512))
    if meta is None:
        meta = cap * min(K, E // W) if W > 0 and E % W == 0 else 0
    return lib.moe_ep_dispatch_pack_noalloc(FAKE, FAKE, T, K, E, W, cap,
                                            ctypes.addressof(pl), npl, FAKE, FAKE,
                                            FAKE, meta, rank, ecnt, FAKE, None, None)


def _send_scratch(T, W):
    r128 = lambda x: (x + 127) // 128 * 128
    return 2 * r128(-(-T // 256) * W * 4) + r128(T * W * 4)


def test_dispatch_pack_noalloc_argument_checks():
    """The allocation-free pack checks its arguments like the pack, and
    refuses sizes whose send-side scratch exceeds its device array before
    any HIP call (so no GPU is needed here)."""
    assert _pack_noalloc(W=0) == B.EINVAL
    assert _pack_noalloc(T=17) == B.ECAP
    assert _pack_noalloc(npl=9) == B.EINVAL
    assert _pack_noalloc(meta=31) == B.EINVAL
    # 2.1 M (token, destination) pairs: just past the 8 MiB array
    T, W = 1 << 16, 32
    assert _send_scratch(T, W) > B.NOALLOC_SCRATCH_BYTES
    assert _pack_noalloc(T=T, K=2, E=64, W=W, cap=T) == B.ESCRATCH
    assert _send_scratch(T, 31) <= B.NOALLOC_SCRATCH_BYTES
    # the pack with a caller workspace takes the same sizes
    assert _pack(T=T, K=2, E=64, W=W, cap=T, ws_bytes=8) == B.EWORKSPACE


def test_expert_batch_ranked_argument_checks():
    lib = B.load()

    def call(W=4, el=2, K=2, cap=16, ecnt_stride=None, rank=FAKE, eloc_stride=None):
        slots = min(K, el)
        pl = _payloads((FAKE, cap * 512, FAKE, W * cap * 512, 512))
        es = cap * slots if eloc_stride is None else eloc_stride
        cs = el if ecnt_stride is None else ecnt_stride
        return lib.moe_ep_expert_batch_ranked(FAKE, 1, FAKE, rank, es, FAKE, cs, W, el, K,
                                              cap, ctypes.addressof(pl), 1, FAKE, FAKE,
                                              None, None)

    assert call(rank=None) == B.EINVAL
    assert call(ecnt_stride=1) == B.EINVAL             # rows of e_local counts
    assert call(eloc_stride=31) == B.EINVAL
    assert call(W=8, el=513) == B.EINVAL               # W * e_local > 4096
    assert call(W=0) == B.EINVAL


def test_dispatch_pack_fp4_argument_checks():
    lib = B.load()

    def call(H=256, hs=None, q=FAKE, qs=None, sc=FAKE, ss=None, cap=16):
        hs = 2 * H if hs is None else hs
        qs = cap * H // 2 if qs is None else qs
        sp = B.fp4_scale_pitch(H)
        ss = cap * sp if ss is None else ss
        pl = _payloads()
        return lib.moe_ep_dispatch_pack_fp4(FAKE, FAKE, 16, 2, 8, 4, cap, FAKE, hs, H,
                                            q, qs, sc, ss, ctypes.addressof(pl), 0,
                                            FAKE, FAKE, FAKE, cap * 2, None, None, FAKE,
                                            None, FAKE, 1 << 20, None)

    assert B.fp4_scale_pitch(7168) == 448 and B.fp4_scale_pitch(544) == 48
    assert call(H=0) == B.EINVAL
    assert call(H=272) == B.EALIGN                   # H/2 = 136 bytes
    assert call(hs=2 * 256 - 16) == B.EINVAL
    assert call(qs=16 * 128 - 16) == B.EINVAL
    assert call(ss=16 * 16 - 16) == B.EINVAL
    assert call(q=None) == B.EINVAL
    assert call(q=FAKE + 8) == B.EALIGN
    assert call(sc=FAKE + 4) == B.EALIGN
    assert call(ss=16 * 16 + 8) == B.EALIGN


def test_expert_batch_argument_checks():
    lib = B.load()

    def call(W=4, el=2, K=2, cap=16, eloc_stride=None, ws=FAKE, ws_bytes=1 << 20,
             pl=None, npl=1, cnt=FAKE):
        slots = min(K, el)
        if eloc_stride is None:
            eloc_stride = cap * slots
        if pl is None:
            pl = _payloads((FAKE, cap * 512, FAKE, W * cap * 512, 512))
        return lib.moe_ep_expert_batch(cnt, 1, FAKE, eloc_stride, W, el, K, cap,
                                       ctypes.addressof(pl), npl, FAKE, FAKE,
                                       None, ws, ws_bytes, None)

    assert call(el=0) == B.EINVAL
    assert call(el=1025) == B.EINVAL
    assert call(W=0) == B.EINVAL
    assert call(cnt=None) == B.EINVAL
    assert call(eloc_stride=16 * 2 - 1) == B.EINVAL
    assert call(pl=_payloads((FAKE, 15 * 512, FAKE, 64 * 512, 512))) == B.EINVAL
    assert call(pl=_payloads((FAKE, 16 * 512, FAKE, 63 * 512, 512))) == B.EINVAL
    assert call(pl=_payloads((FAKE, 16 * 520, FAKE, 64 * 520, 520))) == B.EALIGN
    assert call(ws=None) == B.EWORKSPACE
    assert call(ws_bytes=4) == B.EWORKSPACE

    def plan(W=4, el=2, K=2, cap=16, ent=FAKE, ws_bytes=1 << 20):
        return lib.moe_ep_expert_batch_plan(FAKE, 1, FAKE, cap * min(K, el), W, el,
                                            K, cap, ent, FAKE, None, FAKE,
                                            ws_bytes, None)

    assert plan(el=0) == B.EINVAL
    assert plan(ent=None) == B.EINVAL
    assert plan(ws_bytes=4) == B.EWORKSPACE

    def copy(W=4, el=2, K=2, cap=16, pl=None, ws_bytes=1 << 20):
        if pl is None:
            pl = _payloads((FAKE, cap * 512, FAKE, W * cap * 512, 512))
        return lib.moe_ep_expert_batch_copy(FAKE, 1, FAKE, cap * min(K, el), W, el,
                                            K, cap, ctypes.addressof(pl), 1, FAKE,
                                            None, FAKE, ws_bytes, None)

    assert copy(W=65) == B.EINVAL
    assert copy(pl=_payloads((FAKE, 16 * 520, FAKE, 64 * 520, 520))) == B.EALIGN
    assert copy(ws_bytes=4) == B.EWORKSPACE


def test_sanitize_argument_checks():
    lib = B.load()

    def call(W=4, el=2, K=2, cap=16, es=None, os_=None, cnt=FAKE, eloc=FAKE, out=FAKE):
        slots = min(K, el)
        es = cap * slots if es is None else es
        os_ = cap * slots if os_ is None else os_
        return lib.moe_ep_sanitize_expert_ids(cnt, 1, eloc, es, W, el, K, cap, -1,
                                              out, os_, None, None)

    assert call(W=0) == B.EINVAL
    assert call(el=0) == B.EINVAL
    assert call(cap=-1) == B.EINVAL
    assert call(cnt=None) == B.EINVAL
    assert call(eloc=None) == B.EINVAL
    assert call(out=None) == B.EINVAL
    assert call(es=31) == B.EINVAL
    assert call(os_=31) == B.EINVAL
    assert call(es=40, os_=32) == B.EINVAL            # in place with another stride


def test_combine_argument_checks():
    lib = B.load()

    def reduce(dtype=B.BF16, H=256, W=4, el=2, K=2, cap=16, estride=None,
               rstride=None, y=FAKE):
        if estride is None:
            estride = W * cap * H
        if rstride is None:
            rstride = cap * H
        return lib.moe_ep_combine_reduce(y, estride, dtype, H, FAKE, 1, FAKE,
                                         FAKE, cap * min(K, el), FAKE, W, el,
                                         K, cap, FAKE, rstride, None)

    assert reduce(dtype=7) == B.EDTYPE
    assert reduce(H=0) == B.EINVAL
    assert reduce(H=260) == B.EALIGN                   # 520 B rows
    assert reduce(dtype=B.F32, H=258) == B.EALIGN
    assert reduce(estride=4 * 16 * 256 - 1) == B.EINVAL
    assert reduce(rstride=16 * 256 - 8) == B.EINVAL
    assert reduce(y=None) == B.EINVAL
    assert reduce(y=FAKE + 2) == B.EALIGN
    # sizes and strides large enough to overflow a product are rejected,
    # not multiplied (the sanitizer run of these tests checks the latter)
    huge = 1 << 62
    assert reduce(H=huge) == B.EINVAL
    assert reduce(H=1 << 40, estride=huge, rstride=huge) == B.EINVAL
    assert reduce(estride=(1 << 63) - 4, rstride=(1 << 63) - 4) == B.EALIGN

    def unpack(dtype=B.BF16, H=256, T=8, W=4, cap=16, bstride=None, out=FAKE):
        if bstride is None:
            bstride = cap * H
        return lib.moe_ep_combine_unpack(FAKE, bstride, dtype, H, FAKE, T, W,
                                         cap, out, None)

    assert unpack(dtype=3) == B.EDTYPE
    assert unpack(T=17) == B.ECAP
    assert unpack(W=65) == B.EINVAL
    assert unpack(bstride=16 * 256 - 8) == B.EINVAL
    assert unpack(out=None) == B.EINVAL
    assert unpack(H=12) == B.EALIGN
    assert unpack(H=1 << 62, bstride=1 << 62) == B.EINVAL
    assert unpack(cap=1 << 62, T=8) == B.EINVAL
    assert unpack(bstride=(1 << 63) - 4) == B.EALIGN

    def peers(self_src=0, W=4, y=FAKE):
        return lib.moe_ep_combine_reduce_peers(y, W * 16 * 256, B.BF16, 256, FAKE, 1,
                                               FAKE, FAKE, 16 * 2, FAKE, W, 2, 2, 16,
                                               self_src, FAKE, 16 * 256, None)

    assert peers(self_src=-1) == B.EINVAL
    assert peers(self_src=4) == B.EINVAL
    assert peers(y=None) == B.EINVAL
    assert peers(y=FAKE + 2) == B.EALIGN

    def fused(self_rank=0, T=8, W=4, el=2, H=256, estride=None, row=FAKE, y=FAKE):
        estride = W * 16 * H if estride is None else estride
        return lib.moe_ep_combine_unpack_fused(FAKE, 16 * H, B.BF16, H, FAKE, T, W, 16,
                                               self_rank, y, estride, FAKE, FAKE, row,
                                               el, 2, FAKE, None)

    assert fused(self_rank=-1) == B.EINVAL
    assert fused(self_rank=4) == B.EINVAL
    assert fused(T=17) == B.ECAP
    assert fused(el=0) == B.EINVAL
    assert fused(row=None) == B.EINVAL
    assert fused(estride=4 * 16 * 256 - 8) == B.EINVAL
    assert fused(y=FAKE + 2) == B.EALIGN
    assert fused(H=12, estride=4 * 16 * 16) == B.EALIGN
    assert fused(H=1 << 62, estride=1 << 62) == B.EINVAL


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        B.load(str(tmp_path / "absent.so"))


def test_stream_probe_library_checks_its_arguments():
    """The HBM stream probes of `bench.py --probe stream` live in their own
    library, which exports the probe alone and rejects ranges that are not
    whole 16 KiB chunks, extra ranges past the stream, missing buffers and
    misaligned pointers before anything is launched."""
    from combine_topk_ids_dest_amd import build as hb
    assert os.path.exists(hb.PROBE_LIB), "run __graft_entry__.build() first"
    out = subprocess.run(["nm", "-D", "--defined-only", hb.PROBE_LIB],
                         capture_output=True, text=True, check=True).stdout
    assert re.findall(r" T (moe_ep\w*)", out) == ["moe_ep_probe_stream"]
    lib = ctypes.CDLL(hb.PROBE_LIB)
    f = lib.moe_ep_probe_stream
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    P, C = 1 << 20, 16384          # a fake 16-byte-aligned address; one chunk
    ok = dict(src=P, src2=None, n=4 * C, er=0, dst=P, dst2=None, ew=0, sink=P, grid=8)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["src"], a["src2"], a["n"], a["er"], a["dst"], a["dst2"], a["ew"],
                 a["sink"], a["grid"], 1, 1, None)

    assert call(n=4 * C + 16) == -1             # not whole chunks
    assert call(n=0) == -1
    assert call(er=C) == -1                     # extra read without src2
    assert call(src2=P, er=5 * C) == -1         # extra read past the stream
    assert call(ew=C) == -1                     # extra write without dst2
    assert call(src=None, dst=None) == -1       # nothing to read or write
    assert call(dst=None, sink=None) == -1      # a read needs its sink
    assert call(dst=P + 8) == -1                # misaligned
    assert call(grid=0) == -1
