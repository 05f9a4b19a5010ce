"""W logical expert-parallel ranks on one GPU.

Every rank's buffers live on the one device. The exchange after the pack
(recv_r[s] = send_s[r]) and after the reduce (back_s[d] = ret_d[s]) is not a
kernel: the receive side reads the rank-stride view send[:, r] and the
unpack reads ret[:, s], through the rank-stride arguments of the C ABI.

Device layout (all dense, rank-major):
  ids, wts        [W_src, T, K]           int32 / fp32
  src[p]          [W_src, T, row_p]        payload p (uint8 rows)
  send[p]         [W_src, W_dst, cap, row_p]
  send_cnt        [W_src, W_dst]           int32
  send_eloc/_w    [W_src, W_dst, cap, slots]
  send_rank       [W_src, W_dst, cap, slots] int32 (ranked form only)
  send_ecnt       [W_src, W_dst, e_local] int32 (ranked form only)
  token_slot      [W_src, T, W_dst]        int32 (unpack context)
  b[p]            [e_local, W*cap, row_p]  one buffer per lane, reused by the
                                           destinations of that lane
  expert_num_tokens [W_dst, e_local]
  recv_row        [W_dst, W_src, cap, slots] (reduce context)
  Y               [e_local, W*cap, H]      expert outputs, one buffer per lane,
                                           reused by the destinations of that lane
  ret             [W_dst, W_src, cap, H]
  out             [W_src, T, H]

Lanes: rank i uses lane i % lanes for the buffers that ranks share (the
workspace, b and Y), so no two lanes read or write the same expert rows. With several lanes, step(streams=...) runs the ranks of
each lane on its own HIP stream, so the kernels of different ranks may
overlap (on W GPUs the ranks run at the same time anyway); the three phases
(packs, batch + reduce, unpacks) are joined across the streams with events,
since each phase reads what every rank wrote in the one before.

Allocation: buffers of 2 GiB and more (at full size the send buffer of the
hidden row and the expert-batch, expert-output and return buffers) are
physically contiguous device blocks when the device grants them
(devmem.empty_contiguous); the row-scattering kernels measured faster on
them than on the caching allocator's blocks.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import binding as B
from . import devmem

# Buffers from this size up are asked for as physically contiguous blocks:
# at full size the send buffer of the hidden row, the expert-batch, expert-
# output and return buffers. Smaller ones (sources, side payloads) stay with
# torch's allocator: making them contiguous as well (a 64 MiB threshold)
# measured slower for the multi-payload pack (231 against 210 us).
CONTIGUOUS_MIN_BYTES = 2 << 30


class LogicalEP:
    def __init__(self, T: int, H: int, E: int, K: int, W: int, cap: int,
                 row_bytes: Sequence[int], combine_dtype=torch.bfloat16,
                 device="cuda", fill: Optional[int] = None,
                 quant_group: Optional[int] = None, quant_fp4: bool = False,
                 lanes: int = 1, contiguous: bool = True, ranked: bool = False):
        """row_bytes: bytes per row of each source payload (payload 0 is the
        bf16 hidden row that the combine returns). fill: byte to pre-fill
        every buffer with (e.g. 0xFF, NaN in bf16/fp32) so unwritten tails
        stay visible; None leaves buffers uninitialised. quant_group: if set,
        the pack quantises payload 0 to fp8 e4m3 with one fp32 scale per
        quant_group columns (moe_ep_dispatch_pack_fp8), and the codes and
        the scales travel as the first two payloads instead of it.
        quant_fp4: the same with 4-bit E2M1 codes and E4M3 scales per 16
        columns (moe_ep_dispatch_pack_fp4). lanes: copies of the shared
        workspace and b buffers (see the module docstring). contiguous:
        buffers of at least CONTIGUOUS_MIN_BYTES are physically contiguous
        allocations where the device grants them (devmem), else come from
        torch's allocator; self.contiguous_bytes counts the granted ones.
        ranked: the packs also write the per-expert ranks and counts
        (send_rank, send_ecnt) and the receive side is
        moe_ep_expert_batch_ranked (no receive scan); batch_plan and
        batch_copy keep the scanned form."""
        if lanes < 1 or lanes > W:
            raise ValueError("lanes must be in [1, W]")
        self.lanes = lanes
        self.T, self.H, self.E, self.K, self.W, self.cap = T, H, E, K, W, cap
        self.e_local = E // W
        self.cap_, self.slots, self.expert_cap = B.moe_ep_capacities(K, E, W, cap)
        self.dtype = combine_dtype
        self.device = torch.device(device)
        self.quant_group = quant_group
        self.quant_fp4 = quant_fp4
        self.row_bytes = list(row_bytes)
        if quant_fp4:
            if quant_group is not None:
                raise ValueError("choose one quantised format")
            if self.row_bytes[0] != 2 * H:
                raise ValueError("quantize-on-pack needs payload 0 = bf16 [T, H]")
            self.send_row_bytes = [H // 2, B.fp4_scale_pitch(H)] + self.row_bytes[1:]
        elif quant_group is not None:
            if self.row_bytes[0] != 2 * H:
                raise ValueError("quantize-on-pack needs payload 0 = bf16 [T, H]")
            G = B.scale_pitch(H, quant_group)
            # rows that travel: codes, scales, then the further payloads
            self.send_row_bytes = [H, 4 * G] + self.row_bytes[1:]
        else:
            self.send_row_bytes = list(self.row_bytes)
        W_, el, sl = W, self.e_local, self.slots

        self.contiguous_bytes = 0

        def alloc(shape, dtype):
            t = None
            nbytes = torch.Size(shape).numel() * torch.empty((), dtype=dtype).element_size()
            if contiguous and nbytes >= CONTIGUOUS_MIN_BYTES:
                t = devmem.empty_contiguous(shape, dtype, self.device)
                if t is not None:
                    self.contiguous_bytes += nbytes
            if t is None:
                t = torch.empty(shape, dtype=dtype, device=self.device)
            if fill is not None:
                t.view(torch.uint8).fill_(fill)
            return t

        self.ids = alloc((W_, T, K), torch.int32)
        self.wts = alloc((W_, T, K), torch.float32)
        self.src = [alloc((W_, T, rb), torch.uint8) for rb in self.row_bytes]
        self.send = [alloc((W_, W_, cap, rb), torch.uint8) for rb in self.send_row_bytes]
        self.send_cnt = alloc((W_, W_), torch.int32)
        self.send_eloc = alloc((W_, W_, cap, sl), torch.int32)
        self.send_w = alloc((W_, W_, cap, sl), torch.float32)
        self.ranked = ranked
        self.send_rank = alloc((W_, W_, cap, sl), torch.int32) if ranked else None
        self.send_ecnt = alloc((W_, W_, el), torch.int32) if ranked else None
        self.token_slot = alloc((W_, T, W_), torch.int32)
        self.b_lanes = [[alloc((el, self.expert_cap, rb), torch.uint8)
                         for rb in self.send_row_bytes] for _ in range(lanes)]
        self.b = self.b_lanes[0]
        self.expert_num_tokens = alloc((W_, el), torch.int32)
        self.recv_row = alloc((W_, W_, cap, sl), torch.int32)
        # self.Y is lane 0's; share_expert_outputs() copies it to the others
        self.Y_lanes = [alloc((el, self.expert_cap, H), combine_dtype) for _ in range(lanes)]
        self.Y = self.Y_lanes[0]
        self.ret = alloc((W_, W_, cap, H), combine_dtype)
        self.out = alloc((W_, T, H), combine_dtype)
        self.err = torch.zeros(1, dtype=torch.int32, device=self.device)
        ws = B.moe_ep_workspace_bytes(cap, K, E, W, cap)
        self.workspaces = [torch.empty(max(ws, 16), dtype=torch.uint8, device=self.device)
                           for _ in range(lanes)]
        self.workspace = self.workspaces[0]
        self._calls = {}
        self._events = {}

    # -- inputs ---------------------------------------------------------
    def set_source(self, s: int, ids, wts, payload_rows: Sequence):
        """Copies one source rank's routing and payload rows (torch or numpy
        arrays, payload rows as [T, row_bytes] bytes) to the device."""
        self.ids[s].copy_(torch.as_tensor(ids))
        self.wts[s].copy_(torch.as_tensor(wts))
        for p, rows in enumerate(payload_rows):
            t = torch.as_tensor(rows).view(torch.uint8)
            self.src[p][s].copy_(t.reshape(self.T, self.row_bytes[p]))

    def share_expert_outputs(self):
        """Copies lane 0's expert outputs (self.Y) to the other lanes' Y
        buffers, for callers that draw one set of expert outputs for every
        destination."""
        for y in self.Y_lanes[1:]:
            y.copy_(self.Y)

    # -- the four calls for one logical rank ----------------------------
    # Each call is marshalled once (binding.prepare_*) and replayed; the
    # buffers never move, so the prepared arguments stay valid.
    def _prepared(self, kind: str, i: int):
        key = (kind, i)
        call = self._calls.get(key)
        if call is None:
            call = self._calls[key] = getattr(self, "_prep_" + kind)(i)
        return call

    def _prep_pack(self, s: int):
        ranks = ((self.send_rank[s], self.send_ecnt[s]) if self.ranked else (None, None))
        if self.quant_fp4:
            return B.prepare_dispatch_pack_fp4(
                self.ids[s], self.wts[s], self.E, self.W, self.cap,
                self.src[0][s].view(torch.bfloat16), self.send[0][s], self.send[1][s],
                [(self.src[p][s], self.send[p + 1][s]) for p in range(1, len(self.src))],
                self.send_cnt[s], self.send_eloc[s], self.send_w[s],
                self.token_slot[s], self.err, self.workspaces[s % self.lanes], *ranks)
        if self.quant_group is not None:
            G = B.scale_pitch(self.H, self.quant_group)
            return B.prepare_dispatch_pack_fp8(
                self.ids[s], self.wts[s], self.E, self.W, self.cap,
                self.src[0][s].view(torch.bfloat16), self.quant_group,
                self.send[0][s], self.send[1][s].view(torch.float32).view(self.W, self.cap, G),
                [(self.src[p][s], self.send[p + 1][s]) for p in range(1, len(self.src))],
                self.send_cnt[s], self.send_eloc[s], self.send_w[s],
                self.token_slot[s], self.err, self.workspaces[s % self.lanes], *ranks)
        return B.prepare_dispatch_pack(
            self.ids[s], self.wts[s], self.E, self.W, self.cap,
            [(self.src[p][s], self.send[p][s]) for p in range(len(self.src))],
            self.send_cnt[s], self.send_eloc[s], self.send_w[s],
            self.token_slot[s], self.err, self.workspaces[s % self.lanes], *ranks)

    def _prep_batch(self, r: int):
        if self.ranked:
            return B.prepare_expert_batch_ranked(
                self.send_cnt[:, r], self.send_eloc[:, r], self.send_rank[:, r],
                self.send_ecnt[:, r], self.W, self.e_local, self.K, self.cap,
                [(self.send[p][:, r], self.b_lanes[r % self.lanes][p])
                 for p in range(len(self.send))],
                self.expert_num_tokens[r], self.recv_row[r], self.err)
        return B.prepare_expert_batch(
            self.send_cnt[:, r], self.send_eloc[:, r], self.W, self.e_local,
            self.K, self.cap,
            [(self.send[p][:, r], self.b_lanes[r % self.lanes][p])
             for p in range(len(self.send))],
            self.expert_num_tokens[r], self.recv_row[r], self.err,
            self.workspaces[r % self.lanes])

    def _prep_batch_plan(self, r: int):
        return B.prepare_expert_batch_plan(
            self.send_cnt[:, r], self.send_eloc[:, r], self.W, self.e_local,
            self.K, self.cap, self.expert_num_tokens[r], self.recv_row[r],
            self.err, self.workspaces[r % self.lanes])

    def _prep_batch_copy(self, r: int):
        return B.prepare_expert_batch_copy(
            self.send_cnt[:, r], self.send_eloc[:, r], self.W, self.e_local,
            self.K, self.cap,
            [(self.send[p][:, r], self.b_lanes[r % self.lanes][p])
             for p in range(len(self.send))],
            self.recv_row[r], self.err, self.workspaces[r % self.lanes])

    def _prep_reduce(self, r: int):
        return B.prepare_combine_reduce(
            self.Y_lanes[r % self.lanes], self.send_cnt[:, r], self.send_eloc[:, r], self.send_w[:, r],
            self.recv_row[r], self.W, self.e_local, self.K, self.cap,
            self.ret[r])

    def _prep_unpack(self, s: int):
        return B.prepare_combine_unpack(self.ret[:, s], self.token_slot[s],
                                        self.cap, self.out[s])

    def _prep_reduce_peers(self, r: int):
        return B.prepare_combine_reduce(
            self.Y_lanes[r % self.lanes], self.send_cnt[:, r], self.send_eloc[:, r], self.send_w[:, r],
            self.recv_row[r], self.W, self.e_local, self.K, self.cap,
            self.ret[r], self_src=r)

    def _prep_unpack_fused(self, s: int, Y=None):
        # rank s's own source block as rank s receives it: send[s][s]
        return B.prepare_combine_unpack_fused(
            self.ret[:, s], self.token_slot[s], self.cap, s,
            self.Y_lanes[s % self.lanes] if Y is None else Y, self.send_eloc[s, s],
            self.send_w[s, s],
            self.recv_row[s, s], self.e_local, self.K, self.out[s])

    def pack(self, s: int, stream=None):
        self._prepared("pack", s)(stream)

    def batch(self, r: int, stream=None):
        self._prepared("batch", r)(stream)

    def batch_plan(self, r: int, stream=None):
        self._prepared("batch_plan", r)(stream)

    def batch_copy(self, r: int, stream=None):
        self._prepared("batch_copy", r)(stream)

    def reduce(self, r: int, stream=None):
        self._prepared("reduce", r)(stream)

    def unpack(self, s: int, stream=None):
        self._prepared("unpack", s)(stream)

    def reduce_peers(self, r: int, stream=None):
        self._prepared("reduce_peers", r)(stream)

    def unpack_fused(self, s: int, stream=None, Y=None):
        """Y: rank s's expert output (default: the shared Y buffer)."""
        if Y is None:
            self._prepared("unpack_fused", s)(stream)
        else:
            self._prep_unpack_fused(s, Y)(stream)

    def step(self, stream=None, fused_local=False, streams=None):
        """One pass of the whole path over all W logical ranks: W packs,
        then batch + reduce per destination (reusing its lane's b and Y),
        then W unpacks. fused_local: each rank's local slice is combined by
        the fused unpack (its lane's Y stands in for the rank's own expert
        output). streams: one HIP stream per lane; rank i's calls go to
        streams[i % lanes], and each phase starts on every stream only
        after the previous phase has ended on all of them. The step is
        ordered after the work already on `stream` (default: the current
        stream), and that stream waits for the whole step. A step over
        several lanes runs eagerly only (not under HIP graph capture)."""
        if streams is None:
            lane_of = [stream] * self.W
        else:
            if len(streams) != self.lanes:
                raise ValueError("one stream per lane")
            if torch.cuda.is_current_stream_capturing():
                # capturing the fork and joins ended in a crash of the
                # process at the end of the capture; not supported
                raise RuntimeError("a step over several lanes is not captured in a "
                                   "HIP graph: capture a one-lane step (streams=None)")
            lane_of = [streams[i % self.lanes] for i in range(self.W)]
            main = stream if stream is not None else torch.cuda.current_stream()
            # the lanes start after the work on `main`, which itself follows
            # the lanes' earlier steps (it waited for them at their end)
            fork = self._lane_events("fork", 1)[0]
            fork.record(main)
            for st in streams:
                st.wait_event(fork)
        for s in range(self.W):
            self.pack(s, lane_of[s])
        if streams is not None:
            self._join(streams, 0)
        for r in range(self.W):
            self.batch(r, lane_of[r])
            if fused_local:
                self.reduce_peers(r, lane_of[r])
            else:
                self.reduce(r, lane_of[r])
        if streams is not None:
            self._join(streams, 1)
        for s in range(self.W):
            if fused_local:
                self.unpack_fused(s, lane_of[s])
            else:
                self.unpack(s, lane_of[s])
        if streams is not None:
            for st, ev in zip(streams, self._lane_events("end", len(streams))):
                ev.record(st)
                main.wait_event(ev)

    # -- the step as one HIP graph per (phase, lane) -------------------------
    # Every lane's calls of a phase are captured on one stream (a plain
    # single-stream capture); a step then replays the graphs on the lanes'
    # streams with the same event joins as step(streams=...), so the host
    # enqueues 3 x lanes graph launches instead of one launch per call.
    _PHASES = 3

    def _phase_calls(self, phase: int, lane: int, fused_local: bool):
        for i in range(lane, self.W, self.lanes):
            if phase == 0:
                self.pack(i)
            elif phase == 1:
                self.batch(i)
                if fused_local:
                    self.reduce_peers(i)
                else:
                    self.reduce(i)
            elif fused_local:
                self.unpack_fused(i)
            else:
                self.unpack(i)

    def capture_lane_graphs(self, fused_local=False):
        """Captures the lane graphs (after one eager step, so that every call
        is marshalled). Replay them with step_graphs."""
        self.step(fused_local=fused_local)
        torch.cuda.synchronize()
        graphs = []
        for phase in range(self._PHASES):
            row = []
            for lane in range(self.lanes):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    self._phase_calls(phase, lane, fused_local)
                row.append(g)
            graphs.append(row)
        torch.cuda.synchronize()
        self._lane_graphs = graphs

    def step_graphs(self, streams, stream=None):
        """One step from the lane graphs: graph (phase, lane) replays on
        streams[lane]; the phases are joined across the streams as in step.
        Ordered after the work on `stream` (default: the current stream),
        which waits for the whole step."""
        if len(streams) != self.lanes:
            raise ValueError("one stream per lane")
        main = stream if stream is not None else torch.cuda.current_stream()
        fork = self._lane_events("fork", 1)[0]
        fork.record(main)
        for st in streams:
            st.wait_event(fork)
        for phase, row in enumerate(self._lane_graphs):
            if phase > 0:
                self._join(streams, phase - 1)
            for st, g in zip(streams, row):
                with torch.cuda.stream(st):
                    g.replay()
        for st, ev in zip(streams, self._lane_events("end", len(streams))):
            ev.record(st)
            main.wait_event(ev)

    def _lane_events(self, key, n: int):
        evs = self._events.get(key)
        if evs is None:
            evs = self._events[key] = [torch.cuda.Event() for _ in range(n)]
        return evs

    def _join(self, streams, phase: int):
        """Every stream in `streams` waits for the work enqueued so far on
        the others (one event per phase and lane, made once and recorded
        again at every step)."""
        evs = self._lane_events(phase, len(streams))
        for st, ev in zip(streams, evs):
            ev.record(st)
        for i, st in enumerate(streams):
            for j, ev in enumerate(evs):
                if i != j:
                    st.wait_event(ev)
