"""Static buffers and the composed MoE layer call sequence.

``MoeBuffers`` allocates, once, every device buffer the C ABI needs, sized by
``moe_plan_sizes`` (the static worst-case sizing of the dispatch regions:
rank_num x local_batch x min(topK, experts per partition) x message size).
``MoeLayer.forward`` enqueues the path on the current stream:
route -> dispatch (+ second hop) -> experts (or identity) -> E2A hop -> combine.
Nothing here computes: it allocates with torch and calls the library.
"""
from __future__ import annotations

import os
from typing import Optional

import torch

from . import (DTYPE_BF16, DTYPE_F32, GATING_SIGMOID, GATING_SOFTMAX, MOE_DEVICE_STALE_EVENT,
               MOE_ERR_STALE, PROJ_DOWN, PROJ_GATEUP, MoeError, moe_check_event,
               RET_BF16, RET_Q8_BLOCKS, RET_Q8_FROM_DISPATCH, RET_Q8_ROWS, Geom, geom, moe_combine,
               moe_dispatch_q8, moe_expert_down_q8, moe_expert_down_q8_int8ret, moe_expert_ffn_q8,
               moe_expert_gateup_q8, moe_pack_expert_weights, moe_plan_sizes, moe_quant_returns_q8,
               moe_relay_returns,
               moe_route_topk, moe_router_logits, moe_router_topk)


_BF16_BITS = (torch.bfloat16, torch.int16, torch.uint16)


def _require(name: str, t, shape, dtypes):
    """The C ABI sees only pointers: a tensor of the wrong size, type or placement
    would be read out of bounds on the device, so it is refused here."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: a torch.Tensor is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: a contiguous device tensor is required")


class PackedExpertWeights:
    """The routed experts' INT8 SwiGLU weights on the device, each projection in
    the expert GEMMs' tile image (moe_pack_expert_weights), the fp32 channel
    scales as given.  Built once from w_gateup [E][2I][H], s_gateup [E][2I],
    w_down [E][H][I], s_down [E][H] (device tensors, 16-byte aligned); every
    layer or microbatch that runs these experts shares it.  Iterates as
    (w_gateup, s_gateup, w_down, s_down) with the packed projections."""

    def __init__(self, w_gateup: torch.Tensor, s_gateup: torch.Tensor, w_down: torch.Tensor,
                 s_down: torch.Tensor):
        E, two_i, H = w_gateup.shape
        I = two_i // 2
        if tuple(w_down.shape) != (E, H, I) or w_gateup.dtype != torch.int8 \
                or w_down.dtype != torch.int8:
            raise ValueError("w_gateup [E][2I][H] and w_down [E][H][I] int8 expected")
        _require("w_gateup", w_gateup.contiguous(), (E, 2 * I, H), (torch.int8,))
        _require("w_down", w_down.contiguous(), (E, H, I), (torch.int8,))
        _require("s_gateup", s_gateup, (E, 2 * I), (torch.float32,))
        _require("s_down", s_down, (E, H), (torch.float32,))
        self.E, self.H, self.I = E, H, I
        sz = moe_plan_sizes(geom(0, H, E, E, 1, 1, 1, 1, 0), I)
        dev = w_gateup.device
        self.w_gateup = torch.empty(sz.w_gateup_packed_bytes, dtype=torch.int8, device=dev)
        self.w_down = torch.empty(sz.w_down_packed_bytes, dtype=torch.int8, device=dev)
        moe_pack_expert_weights(w_gateup.contiguous(), PROJ_GATEUP, E, H, I, self.w_gateup)
        moe_pack_expert_weights(w_down.contiguous(), PROJ_DOWN, E, H, I, self.w_down)
        self.s_gateup = s_gateup
        self.s_down = s_down

    def __iter__(self):
        return iter((self.w_gateup, self.s_gateup, self.w_down, self.s_down))


def _packed(weights):
    if weights is None or isinstance(weights, PackedExpertWeights):
        return weights
    return PackedExpertWeights(*weights)


class MoeBuffers:
    def __init__(self, g: Geom, I: int = 0, out_dtype: torch.dtype = torch.bfloat16,
                 device: str = "cuda"):
        self.g = g
        self.I = I
        sz = moe_plan_sizes(g, I)
        self.sizes = sz
        T, k, H = g.T, g.k, g.H
        i32 = dict(dtype=torch.int32, device=device)
        u8 = dict(dtype=torch.uint8, device=device)
        self.disp_buf = torch.empty(sz.dispatch_bytes, **u8)
        self.relay_buf = torch.empty(sz.relay_bytes, **u8) if g.relays else None
        self.meta = torch.empty((g.D, g.S, 4), **i32)
        self.slot_count = torch.empty(g.P, **i32)
        self.slot_offset = torch.empty(g.P + 1, **i32)
        self.slot_rows = torch.empty(T * k, **i32)
        self.disp_row = torch.empty((T, k), **i32)
        self.ret_row = torch.empty((T, k), **i32)
        self.topk_ids = torch.empty((T, k), **i32)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.phys = torch.empty((T, k), **i32)
        self.expert_counts = torch.empty(g.E, **i32)
        self.dscratch = torch.empty(sz.dispatch_scratch_bytes, **u8)
        self.fscratch = torch.empty(max(sz.ffn_scratch_bytes, 256), **u8)
        nret = sz.return_bytes // (2 * H)
        self.ret = torch.empty((nret, H), dtype=torch.int16, device=device)
        self.comb_row = torch.empty((T, k), **i32) if g.relays else None
        self.out = torch.empty((T, H), dtype=out_dtype, device=device)

    def router_buffers(self):
        """fp32 gate logits [T][E] and the router's split-K scratch (allocated on first use)."""
        if getattr(self, "_logits32", None) is None:
            dev = self.out.device
            self._logits32 = torch.empty((self.g.T, self.g.E), dtype=torch.float32, device=dev)
            self._rscratch = torch.empty(max(self.sizes.router_scratch_bytes, 256),
                                         dtype=torch.uint8, device=dev)
        return self._logits32, self._rscratch

    def ret_q8_rows(self):
        """INT8 expert return rows [T*k][ret_q8_row_bytes] bytes (allocated on first use)."""
        if getattr(self, "_ret_q8", None) is None:
            self._ret_q8 = torch.empty((self.g.T * self.g.k, self.sizes.ret_q8_row_bytes),
                                       dtype=torch.uint8, device=self.out.device)
        return self._ret_q8

    def disp_rows_view(self):
        """The dispatch buffer as [D*S*cap][msg] bytes."""
        return self.disp_buf.view(-1, self.sizes.msg_bytes)

    def device_status(self) -> int:
        return int(self.dscratch[:4].view(torch.int32).item())


def _debug_checks_default() -> bool:
    return os.environ.get("MOE_DEBUG_CHECKS", "0") not in ("", "0")


class MoeLayer:
    """One MoE layer: replica map + (optional) INT8 SwiGLU expert weights.

    With debug_checks (default: the MOE_DEBUG_CHECKS environment variable), the
    experts and the combine first run the receiver's event check (moe_check_event)
    on the dispatch's metadata and messages, wait for it, and raise MoeError with
    MOE_ERR_STALE if they belong to another dispatch event."""

    def __init__(self, g: Geom, gating: str, slot_partition: torch.Tensor,
                 slot_logical: torch.Tensor, replica_offsets: Optional[torch.Tensor] = None,
                 replica_slots: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                 weights=None, I: int = 0, out_dtype: torch.dtype = torch.bfloat16,
                 debug_checks: Optional[bool] = None):
        self.debug_checks = _debug_checks_default() if debug_checks is None else debug_checks
        self.g = g
        if gating not in ("softmax", "sigmoid"):
            raise ValueError(f"gating {gating!r}: 'softmax' or 'sigmoid'")
        self.gating = GATING_SOFTMAX if gating == "softmax" else GATING_SIGMOID
        _require("slot_partition", slot_partition, (g.P,), (torch.int32,))
        _require("slot_logical", slot_logical, (g.P,), (torch.int32,))
        if (replica_offsets is None) != (replica_slots is None):
            raise ValueError("replica_offsets and replica_slots go together")
        if replica_offsets is not None:
            _require("replica_offsets", replica_offsets, (g.E + 1,), (torch.int32,))
            if replica_slots.dim() != 1 or replica_slots.numel() < g.P:
                raise ValueError("replica_slots: a 1-D tensor of at least P entries")
            _require("replica_slots", replica_slots, replica_slots.shape, (torch.int32,))
        if bias is not None:
            _require("bias", bias, (g.E,), (torch.float32,))
        self.slot_partition = slot_partition
        self.slot_logical = slot_logical
        self.replica_offsets = replica_offsets
        self.replica_slots = replica_slots
        self.bias = bias
        self.I = I
        self.weights = weights  # PackedExpertWeights, or a plain 4-tuple packed here, or None
        self.out_dtype = out_dtype
        self.buf = MoeBuffers(g, I, out_dtype)
        self.event_id = 0

    @property
    def weights(self) -> Optional[PackedExpertWeights]:
        return self._weights

    @weights.setter
    def weights(self, w):
        """A PackedExpertWeights, None, or (w_gateup, s_gateup, w_down, s_down) device
        tensors in the plain layout, which are packed here (once)."""
        w = _packed(w)
        if w is not None and (w.E, w.H, w.I) != (self.g.E, self.g.H, self.I):
            raise ValueError(f"expert weights for E={w.E}, H={w.H}, I={w.I}; the layer has "
                             f"E={self.g.E}, H={self.g.H}, I={self.I}")
        self._weights = w

    @staticmethod
    def _dt(t: torch.Tensor) -> int:
        return DTYPE_BF16 if t.dtype in _BF16_BITS else DTYPE_F32

    def router(self, x, w_router):
        """Gate logits from the hidden states: x [T][H] bf16, w_router [E][H] bf16 ->
        fp32 logits [T][E] (returned; route() takes them)."""
        _require("x", x, (self.g.T, self.g.H), _BF16_BITS)
        _require("w_router", w_router, (self.g.E, self.g.H), _BF16_BITS)
        logits, scratch = self.buf.router_buffers()
        moe_router_logits(x, w_router, self.g, logits, scratch)
        return logits

    def route_from_hidden(self, x, w_router, keep_logits: bool = False):
        """The gate and the routing in one call (moe_router_topk): fills the same
        route buffers as route(); returns the fp32 logits when keep_logits."""
        _require("x", x, (self.g.T, self.g.H), _BF16_BITS)
        _require("w_router", w_router, (self.g.E, self.g.H), _BF16_BITS)
        logits, scratch = self.buf.router_buffers()
        b = self.buf
        moe_router_topk(x, w_router, self.bias, self.gating, self.replica_offsets,
                        self.replica_slots, self.g, logits if keep_logits else None, b.topk_ids,
                        b.topk_w, b.phys, b.expert_counts, scratch)
        return logits if keep_logits else None

    def route(self, logits):
        _require("logits", logits, (self.g.T, self.g.E), _BF16_BITS + (torch.float32,))
        b = self.buf
        moe_route_topk(logits, self._dt(logits), self.bias, self.gating, self.replica_offsets,
                       self.replica_slots, self.g, b.topk_ids, b.topk_w, b.phys, b.expert_counts)

    def dispatch(self, x):
        _require("x", x, (self.g.T, self.g.H), _BF16_BITS + (torch.float32,))
        b = self.buf
        self.event_id = (self.event_id + 1) & 0xFFFFFFFF
        moe_dispatch_q8(x, self._dt(x), b.phys, self.slot_partition, self.event_id, self.g,
                        b.disp_buf, b.meta, b.slot_count, b.slot_offset, b.slot_rows, b.disp_row,
                        b.ret_row, b.relay_buf, b.dscratch)

    def check_event(self):
        """The receiver's event check (moe_check_event) against this layer's last
        dispatch; raises MoeError(MOE_ERR_STALE) on a mismatch.  Synchronizes."""
        b = self.buf
        if getattr(self, "_ev_status", None) is None:
            self._ev_status = torch.empty(1, dtype=torch.int32, device=b.meta.device)
        status = self._ev_status
        moe_check_event(b.meta, b.disp_buf, b.slot_rows, b.slot_offset, self.g, self.event_id,
                        status)
        if int(status.item()) & MOE_DEVICE_STALE_EVENT:
            raise MoeError(MOE_ERR_STALE, "moe_check_event")

    def experts(self, acc_gateup_dbg=None, acc_down_dbg=None):
        if self.debug_checks:
            self.check_event()
        b = self.buf
        wgu, sgu, wd, sd = self.weights
        moe_expert_ffn_q8(b.disp_buf, b.slot_count, b.slot_offset, b.slot_rows, self.slot_logical,
                          wgu, sgu, wd, sd, self.I, self.g, b.ret, acc_gateup_dbg, acc_down_dbg,
                          b.fscratch)

    def experts_gateup(self):
        if self.debug_checks:
            self.check_event()
        b = self.buf
        wgu, sgu, _, _ = self.weights
        moe_expert_gateup_q8(b.disp_buf, b.slot_count, b.slot_offset, b.slot_rows,
                             self.slot_logical, wgu, sgu, self.I, self.g, None, b.fscratch)

    def experts_down(self):
        b = self.buf
        _, _, wd, sd = self.weights
        moe_expert_down_q8(b.slot_count, b.slot_offset, self.slot_logical, wd, sd, self.I, self.g,
                           b.ret, None, b.fscratch)

    def experts_down_int8ret(self, acc_down_dbg=None):
        """Down projection with INT8 return rows (one scale per 256 columns)."""
        b = self.buf
        _, _, wd, sd = self.weights
        moe_expert_down_q8_int8ret(b.slot_count, b.slot_offset, self.slot_logical, wd, sd, self.I,
                                   self.g, b.ret_q8_rows(), acc_down_dbg, b.fscratch)

    def quant_returns(self):
        """Token-wise INT8 of the bf16 return rows (one scale per row), into the INT8
        return rows that combine('q8rows') reads."""
        b = self.buf
        moe_quant_returns_q8(b.ret, b.slot_offset, self.g, b.ret_q8_rows())

    def combine(self, mode: str):
        """mode 'q8' (identity experts: dispatched messages), 'bf16' (bf16 returns),
        'q8blocks' (INT8 returns of experts_down_int8ret) or 'q8rows' (token-wise INT8
        returns of quant_returns)."""
        if self.debug_checks:
            self.check_event()
        b = self.buf
        odt = DTYPE_BF16 if self.out_dtype == torch.bfloat16 else DTYPE_F32
        if mode == "q8":
            moe_combine(RET_Q8_FROM_DISPATCH, b.disp_buf, b.disp_row, b.topk_w, self.g, odt, b.out)
        elif mode == "q8blocks":
            moe_combine(RET_Q8_BLOCKS, b.ret_q8_rows(), b.ret_row, b.topk_w, self.g, odt, b.out)
        elif mode == "q8rows":
            moe_combine(RET_Q8_ROWS, b.ret_q8_rows(), b.ret_row, b.topk_w, self.g, odt, b.out)
        else:
            row = b.ret_row
            if self.g.relays:
                moe_relay_returns(b.ret, b.phys, self.slot_partition, b.ret_row, self.g, b.comb_row)
                row = b.comb_row
            moe_combine(RET_BF16, b.ret, row, b.topk_w, self.g, odt, b.out)

    def forward(self, x, logits, combine: str = "bf16"):
        """route -> dispatch -> experts -> combine; combine 'q8blocks' runs the experts
        with INT8 return rows (block scales), 'q8rows' quantizes the bf16 returns
        token-wise before the combine."""
        self.route(logits)
        self.dispatch(x)
        self.expert_stage(combine)
        self.combine(combine)
        return self.buf.out

    def expert_stage(self, combine: str = "bf16"):
        """What forward runs between the dispatch and the combine: the experts (none
        without weights), with INT8 block returns for 'q8blocks' and the token-wise
        quantization of the returns for 'q8rows'."""
        if self.weights is None:
            return
        if combine == "q8blocks":
            self.experts_gateup()
            self.experts_down_int8ret()
        else:
            self.experts()
            if combine == "q8rows":
                self.quant_returns()

    def capture(self, x, logits, combine: str = "bf16") -> "MoeGraph":
        """forward(x, logits, combine) captured once as a HIP graph.  The step runs
        once eagerly first (kernel loading), then under capture on a side stream;
        nothing in it allocates, synchronizes or sets memory from the host (every
        clearing is a kernel).  Replays read x and logits where they are now: to run
        other inputs, copy them into these tensors.  Not with debug_checks, whose
        event check waits on the host."""
        if self.debug_checks:
            raise ValueError("capture: the debug event check waits on the host between kernels")
        self.forward(x, logits, combine)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.forward(x, logits, combine)
        torch.cuda.synchronize()
        return MoeGraph(graph, self.buf.out, self.event_id, (x, logits))


class MoeGraph:
    """One MoE step captured as a HIP graph (MoeLayer.capture): replay() reruns
    route -> dispatch -> experts -> combine on the tensors the capture read and
    the layer's static buffers, with no host work per kernel.  The dispatch
    stamps the event id that was current at capture on every replay (event_id);
    a caller that checks events captures one graph per id and alternates.  The
    graph holds the captured inputs, whose memory every replay reads."""

    def __init__(self, graph, out: torch.Tensor, event_id: int, inputs):
        self.graph = graph
        self.out = out
        self.event_id = event_id
        self.inputs = inputs

    def replay(self) -> torch.Tensor:
        self.graph.replay()
        return self.out


class MoeTicket:
    """One batch submitted to MoeOverlap: `out` is its output tensor (the layer's
    buf.out), `done` the event recorded after its combine.  wait() makes the
    current stream wait for it."""

    def __init__(self, out: torch.Tensor, done):
        self.out = out
        self.done = done

    def wait(self) -> torch.Tensor:
        torch.cuda.current_stream().wait_event(self.done)
        return self.out


class MoeOverlap:
    """Batches of one MoE layer in flight together [XDS, the overlap of
    communication with computation across microbatches (P108-P111); CMI, the
    microbatch section], on three default-priority streams: route and dispatch
    on one, the experts on a second (the batches' expert stages one after
    another), the combine on a third.  Each batch runs in one of the given
    MoeLayers (its static buffers; the layers may share one
    PackedExpertWeights), taken round robin, so one batch's route, dispatch
    and combine run beside another batch's experts.

    submit() orders a batch after the work already on the caller's stream (its
    inputs) and after the previous batch that used the same layer; nothing
    else waits, so successive submissions keep the expert stream busy.  A
    batch's output stays valid until len(layers) more batches are submitted:
    read it, on the caller's stream, before that.  Each output is its layer's
    forward output bit for bit."""

    def __init__(self, layers):
        if not layers:
            raise ValueError("MoeOverlap: at least one layer")
        self.layers = list(layers)
        dev = layers[0].slot_partition.device
        self.comm = torch.cuda.Stream(device=dev)
        self.compute = torch.cuda.Stream(device=dev)
        self.ret = torch.cuda.Stream(device=dev)
        self._next = 0
        self._free = [None] * len(self.layers)

    def submit(self, x, logits, combine: str = "bf16") -> MoeTicket:
        j = self._next % len(self.layers)
        layer = self.layers[j]
        g = layer.g
        _require("x", x, (g.T, g.H), _BF16_BITS + (torch.float32,))  # before any work is queued
        _require("logits", logits, (g.T, g.E), _BF16_BITS + (torch.float32,))
        if combine not in ("q8", "bf16", "q8blocks", "q8rows"):
            raise ValueError(f"combine {combine!r}")
        self._next += 1
        ready = torch.cuda.Event()
        ready.record(torch.cuda.current_stream())
        self.comm.wait_event(ready)
        # the inputs are read on the communication stream: their memory must not
        # go back to the caller's stream before that read is done
        x.record_stream(self.comm)
        logits.record_stream(self.comm)
        if self._free[j] is not None:  # the layer's previous batch has been combined
            self.comm.wait_event(self._free[j])
        with torch.cuda.stream(self.comm):
            layer.route(logits)
            layer.dispatch(x)
        routed = torch.cuda.Event()
        routed.record(self.comm)
        self.compute.wait_event(routed)
        with torch.cuda.stream(self.compute):
            layer.expert_stage(combine)
        computed = torch.cuda.Event()
        computed.record(self.compute)
        self.ret.wait_event(computed)
        with torch.cuda.stream(self.ret):
            layer.combine(combine)
        done = torch.cuda.Event()
        done.record(self.ret)
        self._free[j] = done
        return MoeTicket(layer.buf.out, done)

    def forward(self, inputs, combine: str = "bf16"):
        """inputs: one (x, logits) per batch, at most one per layer.  Submits them
        all, then the caller's stream waits for every one.  Returns the outputs."""
        if len(inputs) > len(self.layers):
            raise ValueError(f"{len(inputs)} batches for {len(self.layers)} layers")
        tickets = [self.submit(x, logits, combine) for x, logits in inputs]
        return [t.wait() for t in tickets]


class MoePipeline:
    """A microbatch pipeline of one MoE layer on one GPU [XDS, the microbatch
    overlap of communication with computation (P108-P111); CMI, the microbatch
    section].  The batch is split by source partitions into n microbatches,
    each with its own static buffers, run as MoeOverlap schedules them: one
    microbatch's route and dispatch, and another's combine, beside a third's
    experts.  Every token's result is independent of the split (routes, replica
    rotation by batch position, quantization, expert rows and the combine are
    per token), so the output equals MoeLayer.forward's bit for bit.
    Orchestration only: every step runs in the library's kernels."""

    def __init__(self, g: Geom, n_micro: int, gating: str, slot_partition: torch.Tensor,
                 slot_logical: torch.Tensor, replica_offsets: Optional[torch.Tensor] = None,
                 replica_slots: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                 weights=None, I: int = 0, out_dtype: torch.dtype = torch.bfloat16):
        if n_micro < 1 or g.S % n_micro:
            raise ValueError("the source partitions must split evenly into microbatches")
        if g.relays:
            raise ValueError("the two-hop geometry is not pipelined")
        self.n = n_micro
        weights = _packed(weights)  # one packed copy shared by the microbatches
        sub = Geom(g.T // n_micro, g.H, g.E, g.P, g.k, g.D, g.Epp, g.S // n_micro, g.LB,
                   g.msg_bytes, 0, 0)
        self.tm = sub.T
        layers = [MoeLayer(sub, gating, slot_partition, slot_logical, replica_offsets,
                           replica_slots, bias, weights, I, out_dtype)
                  for _ in range(n_micro)]
        self.out = torch.empty((g.T, g.H), dtype=out_dtype, device=slot_partition.device)
        for i, layer in enumerate(layers):
            layer.buf.out = self.out[i * sub.T:(i + 1) * sub.T]
        self.overlap = MoeOverlap(layers)
        self.layers = self.overlap.layers

    def forward(self, x, logits, combine: str = "bf16"):
        """The microbatches through MoeOverlap; the caller's stream waits for all of
        them.  Returns the [T][H] output."""
        tm = self.tm
        self.overlap.forward([(x[i * tm:(i + 1) * tm], logits[i * tm:(i + 1) * tm])
                              for i in range(self.n)], combine)
        return self.out
