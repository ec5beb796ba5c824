"""Seeded synthetic inputs for the MoE route / dispatch / expert-FFN / combine path.

This module is shared by the oracle side (``oracle/``, tests) and the HIP side
(binding, tests, bench).  It only draws random numbers and lays them out as
bytes; it holds none of the method's arithmetic (no top-k, no quantization, no
layout, no expert math).  Both sides consume exactly the bytes produced here.

Streams.  Every tensor is drawn from its own numpy ``SeedSequence`` child,
``SeedSequence(seed, spawn_key=(stream, ...))``, so any tensor (or one expert's
weights, or one block of return rows) can be regenerated alone, in any order,
on any number of threads, with identical bytes.

Workload shapes follow the DeepSeek-V3/R1 deployments that the pages measure
(H=7168, 256 routed experts, top-8, local batch 96, global batches 12288 and
46080; page "xDeepServe on CloudMatrix384", sections on the co-located and the
disaggregated MoE-Attention All-to-All, P041 and P047; page "CloudMatrix384
LLM Serving", section "EP320").  The expert-load skew of the pages' Fig. 11
(measured on ShareGPT, which is not available here) is replaced by a seeded
log-Zipf logit bias; see ``zipf_bias``.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# stream ids (first element of the spawn key)
S_LOGITS, S_BIAS, S_X, S_RETURNS, S_WEIGHTS, S_SCALES, S_CALIB, S_ROUTER = range(8)

_THREADS = 8


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens (T = S * LB)
    H: int          # hidden size
    E: int          # logical routed experts
    P: int          # physical expert slots
    k: int          # routes per token
    D: int          # destination (expert) partitions
    Epp: int        # slots per destination partition
    S: int          # source partitions
    LB: int         # local batch per source partition
    gating: str     # 'softmax' | 'sigmoid'
    logits_dtype: str   # 'f32' | 'bf16'
    x_dtype: str        # 'f32' | 'bf16'
    zipf: bool          # add the seeded log-Zipf bias to the logits
    experts: str        # 'identity' | 'synthetic' (random bf16 returns) | 'swiglu'
    combine: str        # 'q8' (returns = dispatched rows) | 'bf16'
    out_dtype: str      # 'f32' | 'bf16'
    I: int = 0          # SwiGLU intermediate size
    eplb: str = "none"  # 'none' | 'plan' (replicas chosen from a calibration batch) | 'first32'
    budget: int = 0     # number of redundant slots
    relays: int = 0     # two-hop relay partitions (0 = direct)
    seed: int = 0
    calib_slices: int = 4
    calib_tokens: int = 1024

    @property
    def msg(self) -> int:
        return ((self.H + 16 + 127) // 128) * 128

    @property
    def cap(self) -> int:
        return self.LB * min(self.k, self.Epp)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five shapes, plus the layer shape the headline throughput is quoted on.
WORKLOADS = {
    "tiny": Workload("tiny", T=16, H=64, E=8, P=8, k=2, D=4, Epp=2, S=4, LB=4,
                     gating="softmax", logits_dtype="f32", x_dtype="f32", zipf=False,
                     experts="identity", combine="q8", out_dtype="f32"),
    "decode96": Workload("decode96", T=96, H=7168, E=256, P=256, k=8, D=256, Epp=1, S=1, LB=96,
                         gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=False,
                         experts="identity", combine="q8", out_dtype="f32"),
    "global12288": Workload("global12288", T=12288, H=7168, E=256, P=256, k=8, D=128, Epp=2, S=128,
                            LB=96, gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=True,
                            experts="synthetic", combine="bf16", out_dtype="bf16"),
    "eplb4096": Workload("eplb4096", T=4096, H=7168, E=256, P=288, k=8, D=288, Epp=1, S=1, LB=4096,
                         gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=True,
                         experts="swiglu", combine="bf16", out_dtype="bf16", I=2048,
                         eplb="plan", budget=32),
    "twohop46080": Workload("twohop46080", T=46080, H=7168, E=256, P=288, k=8, D=288, Epp=1, S=160,
                            LB=288, gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=False,
                            experts="synthetic", combine="bf16", out_dtype="bf16",
                            eplb="first32", budget=32, relays=160),
    "layer12288": Workload("layer12288", T=12288, H=7168, E=256, P=256, k=8, D=128, Epp=2, S=128,
                           LB=96, gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=True,
                           experts="swiglu", combine="bf16", out_dtype="bf16", I=2048),
}


def _rng(w: Workload, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(w.seed, spawn_key=tuple(key)))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def _normal_rows(w: Workload, stream: int, rows: int, cols: int, dtype: str,
                 block: int = 256) -> np.ndarray:
    """rows x cols N(0,1), generated in independent blocks of `block` rows."""
    out = np.empty((rows, cols), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def fill(b):
        r0, r1 = b * block, min(rows, (b + 1) * block)
        v = _rng(w, stream, b).standard_normal((r1 - r0, cols), dtype=np.float32)
        out[r0:r1] = to_bf16_bits(v) if dtype == "bf16" else v

    nb = (rows + block - 1) // block
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill, range(nb)))
    return out


def logits(w: Workload, calib_slice: Optional[int] = None) -> np.ndarray:
    """Gate logits [T][E] ~ N(0,1) (f32, or bf16 bit patterns).

    With ``calib_slice`` = i, returns slice i of the calibration batch used to
    plan EPLB replicas ([calib_tokens][E], drawn from its own stream)."""
    if calib_slice is None:
        return _normal_rows(w, S_LOGITS, w.T, w.E, w.logits_dtype)
    v = _rng(w, S_CALIB, calib_slice).standard_normal((w.calib_tokens, w.E), dtype=np.float32)
    return to_bf16_bits(v) if w.logits_dtype == "bf16" else v


def router_weights(w: Workload) -> np.ndarray:
    """Gate weights [E][H] as bf16 bit patterns, N(0, 1/H), so that N(0,1) hidden
    states give logits of unit variance."""
    v = _rng(w, S_ROUTER).standard_normal((w.E, w.H), dtype=np.float32) / np.float32(np.sqrt(w.H))
    return to_bf16_bits(v)


def zipf_bias(w: Workload) -> Optional[np.ndarray]:
    """Per-expert logit bias fp32(-1.1 * ln rank_e), rank = seeded permutation of 1..E.

    A log-Zipf(s=1.1) popularity profile added to N(0,1) logits; it stands in for
    the measured ShareGPT expert skew (a few experts ~30x the mean)."""
    if not w.zipf:
        return None
    rank = _rng(w, S_BIAS).permutation(w.E) + 1
    return (-1.1 * np.log(rank.astype(np.float64))).astype(np.float32)


def hidden(w: Workload) -> np.ndarray:
    """Token hidden states [T][H] ~ N(0,1) (f32, or bf16 bit patterns)."""
    return _normal_rows(w, S_X, w.T, w.H, w.x_dtype)


def route_returns(w: Workload, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Synthetic expert returns, bf16 bit patterns ~N(0,1), one row per route (t, j),
    route-indexed: row t*k + j.  Generated in blocks of 256 routes; ``rows`` (sorted
    or not) selects a subset without generating the rest."""
    n = w.T * w.k
    if rows is None:
        return _normal_rows(w, S_RETURNS, n, w.H, "bf16")
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), w.H), dtype=np.uint16)
    for b in np.unique(rows // 256):
        r0, r1 = b * 256, min(n, (b + 1) * 256)
        v = to_bf16_bits(_rng(w, S_RETURNS, int(b)).standard_normal((r1 - r0, w.H), dtype=np.float32))
        sel = np.nonzero(rows // 256 == b)[0]
        out[sel] = v[rows[sel] - r0]
    return out


def _int8_uniform127(rng: np.random.Generator, shape) -> np.ndarray:
    """int8 uniform on [-127, 127] (the value -128 is redrawn)."""
    n = int(np.prod(shape))
    bg = rng.bit_generator
    a = bg.random_raw((n + 7) // 8).view(np.int8)[:n].copy()
    bad = np.flatnonzero(a == -128)
    while bad.size:
        a[bad] = bg.random_raw((bad.size + 7) // 8).view(np.int8)[:bad.size]
        bad = bad[a[bad] == -128]
    return a.reshape(shape)


def expert_weights(w: Workload, e: int):
    """Logical expert e's INT8 SwiGLU weights and per-output-channel fp32 scales.

    Returns (w_gateup [2I][H] i8, s_gateup [2I] f32, w_down [H][I] i8, s_down [H] f32).
    Rows 0..I-1 of w_gateup are the gate projection, rows I..2I-1 the up projection.
    Scales are u / sqrt(K * 5418.67), u ~ U[0.5, 1.5], K the input width, so that a
    projection of unit-variance input has roughly unit variance (5418.67 is the
    mean square of the uniform int8 values)."""
    H, I = w.H, w.I
    wgu = _int8_uniform127(_rng(w, S_WEIGHTS, e, 0), (2 * I, H))
    wd = _int8_uniform127(_rng(w, S_WEIGHTS, e, 1), (H, I))
    rs = _rng(w, S_SCALES, e)
    sgu = (rs.uniform(0.5, 1.5, 2 * I) / np.sqrt(H * 5418.67)).astype(np.float32)
    sd = (rs.uniform(0.5, 1.5, H) / np.sqrt(I * 5418.67)).astype(np.float32)
    return wgu, sgu, wd, sd


def all_expert_weights(w: Workload, experts=None):
    """Stacked weights of the given logical experts (default all E), built on threads."""
    ids = list(range(w.E)) if experts is None else list(experts)
    n = len(ids)
    wgu = np.empty((n, 2 * w.I, w.H), np.int8)
    wd = np.empty((n, w.H, w.I), np.int8)
    sgu = np.empty((n, 2 * w.I), np.float32)
    sd = np.empty((n, w.H), np.float32)

    def fill(i):
        wgu[i], sgu[i], wd[i], sd[i] = expert_weights(w, ids[i])

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill, range(n)))
    return wgu, sgu, wd, sd


def first32_map(w: Workload):
    """Fixed replica map of the two-hop workload: logical experts 0..budget-1 get one
    redundant copy each, on partitions E..E+budget-1 (one slot per partition).

    Returns (replica_offsets [E+1], replica_slots [P], slot_partition [P], slot_logical [P]),
    with physical slot p = e for primaries (partition e) and p = E + i for replica i.
    Replica lists are in ascending slot order."""
    E, B = w.E, w.budget
    slot_logical = np.concatenate([np.arange(E), np.arange(B)]).astype(np.int32)
    slot_partition = np.arange(E + B, dtype=np.int32)
    offs = [0]
    slots = []
    for e in range(E):
        mine = [p for p in range(E + B) if slot_logical[p] == e]
        slots += mine
        offs.append(len(slots))
    return (np.array(offs, np.int32), np.array(slots, np.int32), slot_partition, slot_logical)


def identity_map(w: Workload):
    """No redundancy: slot p = logical expert p on partition p // Epp."""
    P = w.P
    return (np.arange(P + 1, dtype=np.int32), np.arange(P, dtype=np.int32),
            (np.arange(P) // w.Epp).astype(np.int32), np.arange(P, dtype=np.int32))
