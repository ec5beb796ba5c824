"""MI355X-native MoE route / INT8 dispatch / INT8 SwiGLU experts / combine.

Thin Python binding over the C ABI in ``include/moe_route_topk.h``
(``libmoe_route_topk.so``, built in-tree by ``build.py``).  Functions have the
C names and only marshal arguments: every step runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  There is no
CPU fallback: if the library is missing, importing ``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_route_topk.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_CAPACITY = -3
MOE_ERR_STALE = -4
MOE_ERR_HIP = -5

MOE_STATIC_SCRATCH_BYTES = 16 << 20  # the allocation-free dispatch's scratch per GPU
# the header's limits (MOE_MAX_E, MOE_MAX_P, MOE_MAX_D, MOE_MAX_K, MOE_MAX_H)
MAX_E, MAX_P, MAX_D, MAX_K, MAX_H = 1024, 1024, 1024, 16, 16384

MOE_DEVICE_BAD_ROUTE = 1
MOE_DEVICE_BAD_PARTITION = 2
MOE_DEVICE_OVER_CAPACITY = 4
MOE_DEVICE_STALE_EVENT = 8

DTYPE_F32, DTYPE_BF16 = 0, 1
GATING_SOFTMAX, GATING_SIGMOID = 0, 1
RET_Q8_FROM_DISPATCH, RET_BF16, RET_Q8_BLOCKS, RET_Q8_ROWS = 0, 1, 2, 3
RET_Q8_BLOCK = 256  # columns per scale of the INT8 expert returns
PROJ_GATEUP, PROJ_DOWN = 0, 1

EXPORTED = ("moe_plan_sizes", "moe_eplb_build_map", "moe_route_topk", "moe_dispatch_q8",
            "moe_expert_ffn_q8", "moe_expert_gateup_q8", "moe_expert_down_q8",
            "moe_expert_down_q8_int8ret", "moe_relay_returns", "moe_combine", "moe_router_logits",
            "moe_pack_expert_weights", "moe_router_topk", "moe_quant_returns_q8",
            "moe_dispatch_q8_static", "moe_check_event", "moe_probe_mfma_i8",
            "moe_status_string")


class Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "E", "P", "k", "D", "Epp", "S", "LB", "msg_bytes", "relays", "reserved")]


class Meta(ctypes.Structure):
    _fields_ = [("event_id", ctypes.c_uint32), ("offset", ctypes.c_int32),
                ("count", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("msg_bytes", "cap_rows", "dispatch_bytes", "dispatch_bytes_per_partition",
                 "combine_bytes_per_partition", "relay_bytes", "return_bytes",
                 "dispatch_scratch_bytes", "ffn_scratch_bytes", "ret_q8_row_bytes",
                 "ret_q8_bytes", "router_scratch_bytes", "w_gateup_packed_bytes",
                 "w_down_packed_bytes")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"HIP library not built: {LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_plan_sizes.argtypes = [ctypes.POINTER(Geom), _I32, ctypes.POINTER(Sizes)]
        L.moe_eplb_build_map.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P]
        L.moe_route_topk.argtypes = [_P, _I32, _P, _I32, _P, _P, ctypes.POINTER(Geom), _P, _P, _P,
                                     _P, _P]
        L.moe_dispatch_q8.argtypes = [_P, _I32, _P, _P, ctypes.c_uint32, ctypes.POINTER(Geom), _P,
                                      _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_expert_ffn_q8.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32,
                                        ctypes.POINTER(Geom), _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_expert_gateup_q8.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I32, ctypes.POINTER(Geom),
                                           _P, _P, ctypes.c_size_t, _P]
        L.moe_expert_down_q8.argtypes = [_P, _P, _P, _P, _P, _I32, ctypes.POINTER(Geom), _P, _P, _P,
                                         ctypes.c_size_t, _P]
        L.moe_expert_down_q8_int8ret.argtypes = L.moe_expert_down_q8.argtypes
        L.moe_router_logits.argtypes = [_P, _P, ctypes.POINTER(Geom), _P, _P, ctypes.c_size_t, _P]
        L.moe_pack_expert_weights.argtypes = [_P, _I32, _I32, _I32, _I32, _P, ctypes.c_size_t, _P]
        L.moe_router_topk.argtypes = [_P, _P, _P, _I32, _P, _P, ctypes.POINTER(Geom), _P, _P, _P,
                                      _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_relay_returns.argtypes = [_P, _P, _P, _P, ctypes.POINTER(Geom), _P, _P]
        L.moe_combine.argtypes = [_I32, _P, _P, _P, ctypes.POINTER(Geom), _I32, _P, _P]
        L.moe_quant_returns_q8.argtypes = [_P, _P, ctypes.POINTER(Geom), _P, _P]
        L.moe_check_event.argtypes = [_P, _P, _P, _P, ctypes.POINTER(Geom), ctypes.c_uint32, _P,
                                      _P]
        L.moe_dispatch_q8_static.argtypes = [_P, _I32, _P, _P, ctypes.c_uint32,
                                             ctypes.POINTER(Geom), _P, _P, _P, _P, _P, _P, _P,
                                             _P, _P, _P]
        L.moe_probe_mfma_i8.argtypes = [_I32, _I32, _P, _P]
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        for n in EXPORTED[:-1]:
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(st: int, what: str):
    if st != MOE_OK:
        raise MoeError(st, what)


def geom(T, H, E, P, k, D, Epp, S, LB, msg_bytes=0, relays=0) -> Geom:
    return Geom(T, H, E, P, k, D, Epp, S, LB, msg_bytes, relays, 0)


def geom_of(w) -> Geom:
    """Geometry of a moe_workloads.Workload."""
    return geom(w.T, w.H, w.E, w.P, w.k, w.D, w.Epp, w.S, w.LB, 0, w.relays)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------ host only ---

def moe_plan_sizes(g: Geom, I: int = 0) -> Sizes:
    out = Sizes()
    _check(lib().moe_plan_sizes(ctypes.byref(g), I, ctypes.byref(out)), "moe_plan_sizes")
    return out


def moe_eplb_build_map(token_count, budget: int, D: int, primary_partition, free_slots):
    """Host numpy in, host numpy out (replica_offsets, replica_slots, slot_partition,
    slot_logical, selected)."""
    import numpy as np
    tc = np.ascontiguousarray(token_count, np.int64)
    slices, E = tc.shape
    P = E + budget
    pp = np.ascontiguousarray(primary_partition, np.int32)
    fs = np.ascontiguousarray(free_slots, np.int32)
    ro = np.empty(E + 1, np.int32)
    rs = np.empty(P, np.int32)
    sp = np.empty(P, np.int32)
    sl = np.empty(P, np.int32)
    sel = np.full(max(budget, 1), -1, np.int32)
    _check(lib().moe_eplb_build_map(tc.ctypes.data, slices, E, budget, D, pp.ctypes.data,
                                    fs.ctypes.data, ro.ctypes.data, rs.ctypes.data, sp.ctypes.data,
                                    sl.ctypes.data, sel.ctypes.data), "moe_eplb_build_map")
    return ro, rs, sp, sl, sel[:budget]


# ---------------------------------------------------------- GPU entries ---

def moe_route_topk(logits, logits_dtype: int, bias, gating: int, replica_offsets, replica_slots,
                   g: Geom, topk_ids, topk_w, phys_ids, expert_counts=None, stream=None):
    _check(lib().moe_route_topk(_ptr(logits), logits_dtype, _ptr(bias), gating,
                                _ptr(replica_offsets), _ptr(replica_slots), ctypes.byref(g),
                                _ptr(topk_ids), _ptr(topk_w), _ptr(phys_ids), _ptr(expert_counts),
                                _stream(stream)), "moe_route_topk")


def moe_dispatch_q8(x, x_dtype: int, phys_ids, slot_partition, event_id: int, g: Geom, disp_buf,
                    meta, slot_count, slot_offset, slot_rows, disp_row, ret_row, relay_buf,
                    scratch, stream=None):
    _check(lib().moe_dispatch_q8(_ptr(x), x_dtype, _ptr(phys_ids), _ptr(slot_partition),
                                 event_id & 0xFFFFFFFF, ctypes.byref(g), _ptr(disp_buf), _ptr(meta),
                                 _ptr(slot_count), _ptr(slot_offset), _ptr(slot_rows),
                                 _ptr(disp_row), _ptr(ret_row), _ptr(relay_buf), _ptr(scratch),
                                 scratch.numel() * scratch.element_size(), _stream(stream)),
           "moe_dispatch_q8")


def moe_check_event(meta, disp_buf, slot_rows, slot_offset, g: Geom, event_id: int, status,
                    stream=None):
    """Writes MOE_DEVICE_STALE_EVENT to the device int32 `status` if any meta entry or
    routed message trailer carries another event id, 0 otherwise (asynchronous)."""
    _check(lib().moe_check_event(_ptr(meta), _ptr(disp_buf), _ptr(slot_rows), _ptr(slot_offset),
                                 ctypes.byref(g), event_id & 0xFFFFFFFF, _ptr(status),
                                 _stream(stream)), "moe_check_event")


def moe_dispatch_q8_static(x, x_dtype: int, phys_ids, slot_partition, event_id: int, g: Geom,
                           disp_buf, meta, slot_count, slot_offset, slot_rows, disp_row, ret_row,
                           relay_buf, status=None, stream=None):
    """moe_dispatch_q8 without a scratch argument: the library's own per-GPU array
    serves as scratch (the call allocates nothing); `status` (device int32 or None)
    receives the call's device status word."""
    _check(lib().moe_dispatch_q8_static(_ptr(x), x_dtype, _ptr(phys_ids), _ptr(slot_partition),
                                        event_id & 0xFFFFFFFF, ctypes.byref(g), _ptr(disp_buf),
                                        _ptr(meta), _ptr(slot_count), _ptr(slot_offset),
                                        _ptr(slot_rows), _ptr(disp_row), _ptr(ret_row),
                                        _ptr(relay_buf), _ptr(status), _stream(stream)),
           "moe_dispatch_q8_static")


def moe_expert_ffn_q8(disp_buf, slot_count, slot_offset, slot_rows, slot_logical, w_gateup,
                      s_gateup, w_down, s_down, I: int, g: Geom, ret, acc_gateup_dbg=None,
                      acc_down_dbg=None, scratch=None, stream=None):
    _check(lib().moe_expert_ffn_q8(_ptr(disp_buf), _ptr(slot_count), _ptr(slot_offset),
                                   _ptr(slot_rows), _ptr(slot_logical), _ptr(w_gateup),
                                   _ptr(s_gateup), _ptr(w_down), _ptr(s_down), I, ctypes.byref(g),
                                   _ptr(ret), _ptr(acc_gateup_dbg), _ptr(acc_down_dbg),
                                   _ptr(scratch), scratch.numel() * scratch.element_size(),
                                   _stream(stream)), "moe_expert_ffn_q8")


def moe_expert_gateup_q8(disp_buf, slot_count, slot_offset, slot_rows, slot_logical, w_gateup,
                         s_gateup, I: int, g: Geom, acc_gateup_dbg=None, scratch=None, stream=None):
    _check(lib().moe_expert_gateup_q8(_ptr(disp_buf), _ptr(slot_count), _ptr(slot_offset),
                                      _ptr(slot_rows), _ptr(slot_logical), _ptr(w_gateup),
                                      _ptr(s_gateup), I, ctypes.byref(g), _ptr(acc_gateup_dbg),
                                      _ptr(scratch), scratch.numel() * scratch.element_size(),
                                      _stream(stream)), "moe_expert_gateup_q8")


def moe_expert_down_q8(slot_count, slot_offset, slot_logical, w_down, s_down, I: int, g: Geom, ret,
                       acc_down_dbg=None, scratch=None, stream=None):
    _check(lib().moe_expert_down_q8(_ptr(slot_count), _ptr(slot_offset), _ptr(slot_logical),
                                    _ptr(w_down), _ptr(s_down), I, ctypes.byref(g), _ptr(ret),
                                    _ptr(acc_down_dbg), _ptr(scratch),
                                    scratch.numel() * scratch.element_size(), _stream(stream)),
           "moe_expert_down_q8")


def moe_expert_down_q8_int8ret(slot_count, slot_offset, slot_logical, w_down, s_down, I: int,
                               g: Geom, ret_q8, acc_down_dbg=None, scratch=None, stream=None):
    _check(lib().moe_expert_down_q8_int8ret(_ptr(slot_count), _ptr(slot_offset),
                                            _ptr(slot_logical), _ptr(w_down), _ptr(s_down), I,
                                            ctypes.byref(g), _ptr(ret_q8), _ptr(acc_down_dbg),
                                            _ptr(scratch), scratch.numel() * scratch.element_size(),
                                            _stream(stream)),
           "moe_expert_down_q8_int8ret")


def moe_router_logits(x, w_router, g: Geom, logits, scratch, stream=None):
    _check(lib().moe_router_logits(_ptr(x), _ptr(w_router), ctypes.byref(g), _ptr(logits),
                                   _ptr(scratch), scratch.numel() * scratch.element_size(),
                                   _stream(stream)), "moe_router_logits")


def moe_router_topk(x, w_router, bias, gating: int, replica_offsets, replica_slots, g: Geom,
                    logits, topk_ids, topk_w, phys_ids, expert_counts, scratch, stream=None):
    _check(lib().moe_router_topk(_ptr(x), _ptr(w_router), _ptr(bias), gating,
                                 _ptr(replica_offsets), _ptr(replica_slots), ctypes.byref(g),
                                 _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(phys_ids),
                                 _ptr(expert_counts), _ptr(scratch),
                                 scratch.numel() * scratch.element_size(), _stream(stream)),
           "moe_router_topk")


def moe_pack_expert_weights(w, proj: int, E: int, H: int, I: int, packed, stream=None):
    _check(lib().moe_pack_expert_weights(_ptr(w), proj, E, H, I, _ptr(packed),
                                         packed.numel() * packed.element_size(), _stream(stream)),
           "moe_pack_expert_weights")


def moe_relay_returns(ret, phys_ids, slot_partition, ret_row, g: Geom, comb_row, stream=None):
    _check(lib().moe_relay_returns(_ptr(ret), _ptr(phys_ids), _ptr(slot_partition), _ptr(ret_row),
                                   ctypes.byref(g), _ptr(comb_row), _stream(stream)),
           "moe_relay_returns")


def moe_quant_returns_q8(ret, slot_offset, g: Geom, ret_q8, stream=None):
    _check(lib().moe_quant_returns_q8(_ptr(ret), _ptr(slot_offset), ctypes.byref(g), _ptr(ret_q8),
                                      _stream(stream)), "moe_quant_returns_q8")


def moe_combine(mode: int, src, row, topk_w, g: Geom, out_dtype: int, out, stream=None):
    _check(lib().moe_combine(mode, _ptr(src), _ptr(row), _ptr(topk_w), ctypes.byref(g), out_dtype,
                             _ptr(out), _stream(stream)), "moe_combine")


def moe_probe_mfma_i8(blocks: int, iters: int, out, stream=None):
    _check(lib().moe_probe_mfma_i8(blocks, iters, _ptr(out), _stream(stream)), "moe_probe_mfma_i8")


from .layer import (MoeBuffers, MoeGraph, MoeLayer, MoeOverlap, MoePipeline, MoeTicket,  # noqa: E402,F401,E501
                    PackedExpertWeights)
