"""Seeded synthetic inputs for the MoE expert-parallel dispatch/combine path.

This module only draws inputs. It holds none of the method's arithmetic: no
destination ranks, no slots, no rows, no reductions. Both the HIP path and
the CPU oracle take their inputs from here, and nothing else is shared
between them.

Workload table (five model-shaped routing workloads):

  id  name           T     H     E    K  W   cap   routing     padding
  1   tiny           64    256   8    2  4   64    uniform     5 %
  2   dsv3_prefill   4096  7168  256  8  8   4096  uniform     0
  3   mixtral_zipf   8192  4096  8    2  8   8192  Zipf 1.1    3 %
  4   decode         128   7168  256  8  32  128   uniform     10 %
  5   multi_payload  8192  7168  256  8  8   8192  Zipf 1.2    10 %

Recipe (numpy PCG64, one generator per (workload, stream, rank)):
  stream 0  hidden rows a1 [T,H]: fp32 N(0,1), converted to bf16 by torch's
            CPU conversion (round to nearest even).
  stream 1  expert ids [T,K]: K distinct ids per token, drawn by Gumbel-top-K
            over log-popularity, kept in draw order. Uniform routing uses
            equal popularity; Zipf s gives expert perm[i] popularity
            (i+1)^-s.
  stream 2  router weights [T,K]: softmax over K fp32 N(0,1) logits, in fp32.
  stream 3  padding: exactly floor(frac*T) whole rows, chosen by a seeded
            permutation, get all K ids = -1.
  stream 4  expert outputs (combine input): bf16 N(0,1).
  stream 5  the Zipf popularity permutation, shared by all W source ranks
            (rank index 0), since popularity belongs to the model.

The multi-payload workload moves five payloads per token: bf16 hidden, an
fp8 e4m3 copy quantised per 128 columns (scale = amax/448, 1 if amax = 0),
the fp32 scales [T, H/128], the int32 ids [T,K] and the fp32 weights [T,K].
The combine returns bf16 hidden only.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np

STREAM_HIDDEN = 0
STREAM_IDS = 1
STREAM_WEIGHTS = 2
STREAM_PADDING = 3
STREAM_EXPERT_OUT = 4
STREAM_ZIPF_PERM = 5


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    T: int
    H: int
    E: int
    K: int
    W: int
    cap: int
    routing: str = "uniform"      # "uniform" or "zipf"
    zipf_s: float = 0.0
    pad_frac: float = 0.0
    multi_payload: bool = False

    @property
    def e_local(self) -> int:
        return self.E // self.W

    @property
    def n_pad(self) -> int:
        return int(np.floor(self.pad_frac * self.T + 1e-9))

    def scaled(self, **kw) -> "Workload":
        """A copy with some fields replaced (smaller shapes for fast tests)."""
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny", T=64, H=256, E=8, K=2, W=4, cap=64, pad_frac=0.05),
    2: Workload(2, "dsv3_prefill", T=4096, H=7168, E=256, K=8, W=8, cap=4096),
    3: Workload(3, "mixtral_zipf", T=8192, H=4096, E=8, K=2, W=8, cap=8192,
                routing="zipf", zipf_s=1.1, pad_frac=0.03),
    4: Workload(4, "decode", T=128, H=7168, E=256, K=8, W=32, cap=128,
                pad_frac=0.10),
    5: Workload(5, "multi_payload", T=8192, H=7168, E=256, K=8, W=8, cap=8192,
                routing="zipf", zipf_s=1.2, pad_frac=0.10, multi_payload=True),
}


def rng(wid: int, stream: int, rank: int, salt: int = 0) -> np.random.Generator:
    key = [int(wid), int(stream), int(rank)]
    if salt:
        key.append(int(salt))
    return np.random.default_rng(key)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) through torch's CPU conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _popularity_log(w: Workload, salt: int) -> np.ndarray:
    if w.routing == "uniform":
        return np.zeros(w.E, dtype=np.float64)
    if w.routing != "zipf":
        raise ValueError(f"unknown routing {w.routing!r}")
    perm = rng(w.wid, STREAM_ZIPF_PERM, 0, salt).permutation(w.E)
    logp = np.empty(w.E, dtype=np.float64)
    logp[perm] = -w.zipf_s * np.log(np.arange(1, w.E + 1, dtype=np.float64))
    return logp


def routing(w: Workload, rank: int, salt: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """(topk_ids int32 [T,K], topk_weights fp32 [T,K]) for one source rank."""
    T, K, E = w.T, w.K, w.E
    if K > E:
        raise ValueError("K distinct ids need K <= E")
    logp = _popularity_log(w, salt)
    g = rng(w.wid, STREAM_IDS, rank, salt)
    # Gumbel-top-K: the K largest perturbed log-popularities, largest first,
    # is a draw of K distinct ids without replacement in draw order.
    keys = logp[None, :] + g.gumbel(size=(T, E))
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int32)
    logits = rng(w.wid, STREAM_WEIGHTS, rank, salt).standard_normal(
        (T, K), dtype=np.float32)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    wts = (z / z.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    if w.n_pad:
        pad = rng(w.wid, STREAM_PADDING, rank, salt).permutation(T)[: w.n_pad]
        ids[pad, :] = -1
    return np.ascontiguousarray(ids), np.ascontiguousarray(wts)


def hidden_bf16(w: Workload, rank: int, salt: int = 0) -> np.ndarray:
    """a1 as bf16 bit patterns, uint16 [T,H]."""
    x = rng(w.wid, STREAM_HIDDEN, rank, salt).standard_normal(
        (w.T, w.H), dtype=np.float32)
    return f32_to_bf16_bits(x)


def hidden_f32(w: Workload, rank: int, salt: int = 0) -> np.ndarray:
    """a1 for the fp32 combine path: fp32 N(0,1) [T,H]."""
    return rng(w.wid, STREAM_HIDDEN, rank, salt).standard_normal(
        (w.T, w.H), dtype=np.float32)


def quantize_fp8_e4m3(hidden_bits: np.ndarray, group: int = 128):
    """Per-`group`-column fp8 e4m3 (OCP, finite-only) copy of bf16 rows.

    Returns (codes uint8 [T,H], scales fp32 [T,H/group]). The conversion of
    x/scale to fp8 is torch's CPU conversion (round to nearest even).
    """
    import torch
    T, H = hidden_bits.shape
    if H % group:
        raise ValueError("H must be a multiple of the quantisation group")
    if T == 0:
        return (np.zeros((0, H), np.uint8),
                np.zeros((0, H // group), np.float32))
    x = torch.from_numpy(bf16_bits_to_f32(hidden_bits)).view(T, H // group, group)
    amax = x.abs().amax(dim=2)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (x / scale[:, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return (q.view(torch.uint8).reshape(T, H).numpy(),
            scale.to(torch.float32).numpy())


def payloads(w: Workload, rank: int, salt: int = 0,
             ids: np.ndarray | None = None,
             wts: np.ndarray | None = None) -> List[np.ndarray]:
    """The payload rows one source rank dispatches, as uint8 [T, row_bytes].

    Payload 0 is always the bf16 hidden a1. The multi-payload workload adds
    the fp8 copy, its scales, the int32 ids and the fp32 weights.
    """
    def rows(a):
        a = np.ascontiguousarray(a)
        return a.view(np.uint8).reshape(w.T, a.itemsize * int(np.prod(a.shape[1:])))

    a1 = hidden_bf16(w, rank, salt)
    out = [rows(a1)]
    if w.multi_payload:
        if ids is None or wts is None:
            ids, wts = routing(w, rank, salt)
        q, s = quantize_fp8_e4m3(a1)
        out += [rows(q), rows(s), rows(ids), rows(wts)]
    return out


def expert_outputs_bf16(w: Workload, dest: int, counts: Sequence[int],
                        salt: int = 0) -> List[np.ndarray]:
    """Expert outputs of destination `dest`: for local expert e a bf16 block
    uint16 [counts[e], H]. Drawn only for the rows that hold tokens."""
    n = int(np.sum(counts))
    x = rng(w.wid, STREAM_EXPERT_OUT, dest, salt).standard_normal(
        (n, w.H), dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    out, o = [], 0
    for c in counts:
        out.append(bits[o:o + int(c)])
        o += int(c)
    return out


def expert_outputs_f32(w: Workload, dest: int, counts: Sequence[int],
                       salt: int = 0) -> List[np.ndarray]:
    n = int(np.sum(counts))
    x = rng(w.wid, STREAM_EXPERT_OUT, dest, salt).standard_normal(
        (n, w.H), dtype=np.float32)
    out, o = [], 0
    for c in counts:
        out.append(x[o:o + int(c)])
        o += int(c)
    return out


def expert_outputs_device(out, seed: int):
    """Fills a large device buffer of expert outputs with N(0,1) draws of
    torch's seeded Philox generator, for full-size runs where a host draw of
    gigabytes would dominate. Every value is a plain seeded draw."""
    import torch
    g = torch.Generator(device=out.device)
    g.manual_seed(int(seed))
    torch.randn(out.shape, generator=g, device=out.device, dtype=out.dtype, out=out)
    return out
