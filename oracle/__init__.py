"""Python front of the CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package.  It shares nothing
with the HIP library and never imports it.  Every function takes and returns
host numpy arrays; the arithmetic is all in the C file (plain loops), this
module only marshals arguments and composes the steps in the pages' order.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB points the tests at another build of moe_oracle.c (the
# mutation test builds copies with planted mistakes and checks that the pins
# reject each of them)
LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_DIR, "libmoe_oracle.so")
_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"oracle library not built: {LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.orc_route_topk.argtypes = [_I32, _I32, _I32, _P, _I32, _P, _I32, _P, _P, _P]
        L.orc_eplb_phys.argtypes = [_I32, _I32, _I32, _I32, _P, _P, _P, _P]
        L.orc_quant_tokens.argtypes = [_I32, _I32, _P, _I32, _P, _P]
        L.orc_dispatch_layout.argtypes = [_P, _P, _P, ctypes.c_uint32, _P, _P, _P, _P, _P, _P, _P]
        L.orc_dispatch_rows.argtypes = [_P, _P, _P, _P, _P, ctypes.c_uint32, _I64, _I64, _P]
        L.orc_expert_ffn.argtypes = [_I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.orc_combine.argtypes = [_I32, _I32, _I32, _I32, _P, _I64, _I64, _I32, _P, _P, _I32, _P]
        L.orc_quant_blocks.argtypes = [_I32, _I32, _I32, _P, _P, _P]
        L.orc_router_logits.argtypes = [_I32, _I32, _I32, _P, _P, _P]
        L.orc_eplb_plan.argtypes = [_I32, _I32, _P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P]
        L.orc_static_buffer.argtypes = [_I64, _I64, _I64, _I64, _I64, _P]
        for f in ("orc_route_topk", "orc_eplb_phys", "orc_quant_tokens", "orc_quant_blocks",
                  "orc_router_logits",
                  "orc_dispatch_layout",
                  "orc_dispatch_rows", "orc_expert_ffn", "orc_combine", "orc_eplb_plan",
                  "orc_static_buffer"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    """Address of an array the caller keeps referenced for the duration of the call
    (never pass a temporary: ctypes does not hold it alive)."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(rc, what)


class OracleError(RuntimeError):
    def __init__(self, rc, what):
        super().__init__(f"{what} failed with status {rc}")
        self.rc = rc


def set_threads(n: int):
    """OpenMP thread count of the oracle (results are identical for any count)."""
    os.environ["OMP_NUM_THREADS"] = str(n)
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
    except OSError:
        pass


# ------------------------------------------------------------------ steps ---

def router_logits(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Exact gate logits of bf16 hidden states x [T][H] and gate weights w [E][H]
    (bit patterns): float64 [T][E]."""
    x = np.ascontiguousarray(x, np.uint16)
    w = np.ascontiguousarray(w, np.uint16)
    T, H = x.shape
    E = w.shape[0]
    out = np.empty((T, E), np.float64)
    _check(lib().orc_router_logits(T, E, H, _p(x), _p(w), _p(out)), "router_logits")
    return out


def route_topk(logits: np.ndarray, k: int, gating: str, bias: Optional[np.ndarray] = None,
               logits_bf16: bool = False):
    """(topk_ids [T][k] i32, topk_score [T][k] f32, topk_w [T][k] f64)."""
    logits = np.ascontiguousarray(logits)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    sc = np.empty((T, k), np.float32)
    w = np.empty((T, k), np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    _check(lib().orc_route_topk(T, E, k, _p(logits), int(logits_bf16), _p(b),
                                0 if gating == "softmax" else 1, _p(ids), _p(sc), _p(w)),
           "route_topk")
    return ids, sc, w


def eplb_phys(topk_ids: np.ndarray, LB: int, E: int, replica_offsets=None, replica_slots=None):
    topk_ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    T, k = topk_ids.shape
    phys = np.empty((T, k), np.int32)
    ro = None if replica_offsets is None else np.ascontiguousarray(replica_offsets, np.int32)
    rs = None if replica_slots is None else np.ascontiguousarray(replica_slots, np.int32)
    _check(lib().orc_eplb_phys(T, k, LB, E, _p(topk_ids), _p(ro), _p(rs), _p(phys)), "eplb_phys")
    return phys


def quant_tokens(x: np.ndarray, x_bf16: bool):
    x = np.ascontiguousarray(x)
    T, H = x.shape
    q = np.empty((T, H), np.int8)
    s = np.empty(T, np.float32)
    _check(lib().orc_quant_tokens(T, H, _p(x), int(x_bf16), _p(q), _p(s)), "quant_tokens")
    return q, s


def geom_array(w) -> np.ndarray:
    return np.array([w.T, w.H, w.E, w.P, w.k, w.D, w.Epp, w.S, w.LB, w.msg], np.int32)


def dispatch_layout(w, phys: np.ndarray, slot_partition: np.ndarray, event_id: int):
    g = geom_array(w)
    phys = np.ascontiguousarray(phys, np.int32)
    sp = np.ascontiguousarray(slot_partition, np.int32)
    out = dict(
        meta=np.empty((w.D, w.S, 4), np.int32),
        slot_count=np.empty(w.P, np.int32),
        slot_offset=np.empty(w.P + 1, np.int32),
        slot_rows=np.empty(w.T * w.k, np.int32),
        disp_row=np.empty((w.T, w.k), np.int32),
        ret_row=np.empty((w.T, w.k), np.int32),
        slot_local=np.empty(w.P, np.int32),
    )
    _check(lib().orc_dispatch_layout(_p(g), _p(phys), _p(sp), event_id & 0xFFFFFFFF,
                                     _p(out["meta"]), _p(out["slot_count"]), _p(out["slot_offset"]),
                                     _p(out["slot_rows"]), _p(out["disp_row"]), _p(out["ret_row"]),
                                     _p(out["slot_local"])), "dispatch_layout")
    return out


def dispatch_rows(w, q, scale, phys, slot_local, event_id: int, t0: int = 0, t1: Optional[int] = None):
    """Message bytes of the routes of tokens [t0, t1), route-indexed [(t1-t0)*k][msg]."""
    g = geom_array(w)
    t1 = w.T if t1 is None else t1
    rows = np.empty(((t1 - t0) * w.k, w.msg), np.uint8)
    q = np.ascontiguousarray(q, np.int8)
    scale = np.ascontiguousarray(scale, np.float32)
    phys = np.ascontiguousarray(phys, np.int32)
    slot_local = np.ascontiguousarray(slot_local, np.int32)
    _check(lib().orc_dispatch_rows(_p(g), _p(q), _p(scale), _p(phys), _p(slot_local),
                                   event_id & 0xFFFFFFFF, t0, t1, _p(rows)), "dispatch_rows")
    return rows


def expert_ffn(q_rows, s_rows, wgu, sgu, wd, sd, want_acc: bool = False):
    """One logical expert over n rows: (y bf16 bits [n][H], hq [n][I], hs [n], acc_gu, acc_d)."""
    q_rows = np.ascontiguousarray(q_rows, np.int8)
    s_rows = np.ascontiguousarray(s_rows, np.float32)
    n, H = q_rows.shape
    I = wgu.shape[0] // 2
    y = np.empty((n, H), np.uint16)
    hq = np.empty((n, I), np.int8)
    hs = np.empty(n, np.float32)
    acc_gu = np.empty((n, 2 * I), np.int32) if want_acc else None
    acc_d = np.empty((n, H), np.int32) if want_acc else None
    wgu = np.ascontiguousarray(wgu, np.int8)
    sgu = np.ascontiguousarray(sgu, np.float32)
    wd = np.ascontiguousarray(wd, np.int8)
    sd = np.ascontiguousarray(sd, np.float32)
    _check(lib().orc_expert_ffn(n, H, I, _p(q_rows), _p(s_rows), _p(wgu), _p(sgu), _p(wd),
                                _p(sd), _p(acc_gu), _p(hq), _p(hs), _p(acc_d),
                                _p(y)), "expert_ffn")
    return y, hq, hs, acc_gu, acc_d


def combine(rows: np.ndarray, route_row: np.ndarray, w: np.ndarray, k: int, H: int, mode: str,
            out_bf16: bool, scale_offset: int = 0, scale_block: int = 0):
    """mode 'q8': rows are message rows (int8 payload, fp32 scale at scale_offset);
    mode 'bf16': rows are bf16 value rows; mode 'q8blocks': int8 payload with one fp32
    scale per `scale_block` columns, stored from scale_offset.  route_row[t][j] indexes rows."""
    rows = np.ascontiguousarray(rows)
    route_row = np.ascontiguousarray(route_row, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    T = route_row.shape[0]
    out = np.empty((T, H), np.uint16 if out_bf16 else np.float32)
    stride = rows.shape[1] * rows.itemsize
    m = {"q8": 0, "bf16": 1, "q8blocks": 2}[mode]
    _check(lib().orc_combine(T, k, H, m, _p(rows), stride, scale_offset, scale_block,
                             _p(route_row), _p(w), int(out_bf16), _p(out)), "combine")
    return out


def quant_blocks(y: np.ndarray, block: int):
    """INT8 of bf16 rows y [n][H] (bits) with one scale per `block` columns:
    (q [n][H] int8, scale [n][ceil(H / block)] f32)."""
    y = np.ascontiguousarray(y, np.uint16)
    n, H = y.shape
    nblk = (H + block - 1) // block
    q = np.empty((n, H), np.int8)
    s = np.empty((n, nblk), np.float32)
    _check(lib().orc_quant_blocks(n, H, block, _p(y), _p(q), _p(s)), "quant_blocks")
    return q, s


def int8_return_rows(q: np.ndarray, s: np.ndarray, row_bytes: int) -> np.ndarray:
    """Pack INT8 return rows: H codes, then the fp32 block scales, zero padding to row_bytes."""
    n, H = q.shape
    rows = np.zeros((n, row_bytes), np.uint8)
    rows[:, :H] = q.view(np.uint8)
    rows[:, H:H + 4 * s.shape[1]] = np.ascontiguousarray(s, np.float32).view(np.uint8)
    return rows


def eplb_plan(token_count: np.ndarray, budget: int, D: int, primary_partition: np.ndarray,
              free_slots: np.ndarray):
    token_count = np.ascontiguousarray(token_count, np.int64)
    primary_partition = np.ascontiguousarray(primary_partition, np.int32)
    free_slots = np.ascontiguousarray(free_slots, np.int32)
    slices, E = token_count.shape
    P = E + budget
    out = dict(
        replica_offsets=np.empty(E + 1, np.int32),
        replica_slots=np.empty(P, np.int32),
        slot_partition=np.empty(P, np.int32),
        slot_logical=np.empty(P, np.int32),
        selected=np.full(max(budget, 1), -1, np.int32),
        tail=np.full(budget + 1, np.nan, np.float64),
    )
    _check(lib().orc_eplb_plan(slices, E, _p(token_count), budget, D,
                               _p(primary_partition), _p(free_slots),
                               _p(out["replica_offsets"]), _p(out["replica_slots"]),
                               _p(out["slot_partition"]), _p(out["slot_logical"]),
                               _p(out["selected"]), _p(out["tail"])), "eplb_plan")
    return out


def static_buffer(rank_num: int, local_batch: int, topk: int, experts_per_die: int, msg_size: int):
    out = np.zeros(2, np.int64)
    _check(lib().orc_static_buffer(rank_num, local_batch, topk, experts_per_die, msg_size, _p(out)),
           "static_buffer")
    return int(out[0]), int(out[1])


def expert_counts(topk_ids: np.ndarray, E: int) -> np.ndarray:
    """Tokens routed to each logical expert (the EPLB collect step): a plain histogram."""
    return np.bincount(np.asarray(topk_ids).ravel(), minlength=E).astype(np.int64)


# ------------------------------------------------------- composed layer ---

def moe_layer(w, x, logits, bias, replica_offsets, replica_slots, slot_partition, slot_logical,
              event_id: int = 1, weights=None, returns=None):
    """The whole path on the CPU, in the pages' order: route -> EPLB map -> quantize ->
    dispatch layout + messages -> experts -> combine.  Returns a dict of every
    intermediate.  `weights` = (wgu, sgu, wd, sd) stacked over logical experts (swiglu);
    `returns` = route-indexed bf16 rows (synthetic experts)."""
    r = {}
    ids, sc, tw = route_topk(logits, w.k, w.gating, bias, logits_bf16=(w.logits_dtype == "bf16"))
    r.update(topk_ids=ids, topk_score=sc, topk_w=tw)
    ro = None if replica_offsets is None else replica_offsets
    r["phys"] = eplb_phys(ids, w.LB, w.E, ro, replica_slots)
    q, s = quant_tokens(x, w.x_dtype == "bf16")
    r.update(q=q, scale=s)
    r.update(dispatch_layout(w, r["phys"], slot_partition, event_id))
    r["route_rows"] = dispatch_rows(w, q, s, r["phys"], r["slot_local"], event_id)
    w32 = tw.astype(np.float32)
    r["topk_w32"] = w32
    ident = np.arange(w.T * w.k, dtype=np.int32).reshape(w.T, w.k)
    if w.experts == "identity":
        r["out"] = combine(r["route_rows"], ident, w32, w.k, w.H, "q8", w.out_dtype == "bf16",
                           scale_offset=w.H)
    else:
        if w.experts == "swiglu":
            wgu, sgu, wd, sd = weights
            y = np.empty((w.T * w.k, w.H), np.uint16)
            logical = slot_logical[r["phys"].ravel()]
            for e in np.unique(logical):
                sel = np.nonzero(logical == e)[0]
                toks = sel // w.k
                ye, *_ = expert_ffn(q[toks], s[toks], wgu[e], sgu[e], wd[e], sd[e])
                y[sel] = ye
            r["route_returns"] = y
        else:
            r["route_returns"] = returns
        r["out"] = combine(r["route_returns"], ident, w32, w.k, w.H, "bf16", w.out_dtype == "bf16")
    return r
