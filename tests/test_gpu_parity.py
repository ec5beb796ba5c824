"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the same
seeded inputs.  Integer, byte and index results are compared bit for bit; fp32
results within 1e-5 relative + 1e-6 absolute; bf16 within 1e-2 relative +
1e-3 absolute (and, where both sides run the same fp32 operations, bit for bit).
"""
import numpy as np
import pytest
import torch

import combine_moe_route_topk_amd as moe
import moe_workloads as mw
import oracle
from _parity import (BF16_ATOL, BF16_RTOL, FP32_ATOL, FP32_RTOL, assert_close, bf16_to_f32,
                     calib_ids, dev_bits, gather_rows, host, replica_map, to_dev)

pytestmark = pytest.mark.gpu

# a multi-source case with ragged chunks (LB = 100 -> chunks of 32, 32, 32, 4),
# several slots per partition and a non-power-of-two partition count
RAGGED = mw.Workload("ragged", T=3 * 100, H=384, E=40, P=40, k=8, D=10, Epp=4, S=3, LB=100,
                     gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=True,
                     experts="identity", combine="q8", out_dtype="f32")
# small expert-FFN case: skewed slots from 1 row (less than one 32-row MFMA
# block) to several 128-row m-tiles with ragged tails; H and I span several
# 64-byte K steps, the gate/up projection's last 128-pair n-tile is half full
# (I = 192) and so is the down projection's last 256-wide n-tile (H = 384)
FFN_SMALL = mw.Workload("ffn_small", T=2 * 400, H=384, E=32, P=32, k=4, D=8, Epp=4, S=2, LB=400,
                        gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=True,
                        experts="swiglu", combine="bf16", out_dtype="bf16", I=192)
# decode-size dispatch (at most 1024 routes: one fused launch): three sources,
# H = 1408 (the second 1024-element slice is partial), skewed routes
SMALLB = mw.Workload("smallb", T=3 * 40, H=1408, E=24, P=24, k=6, D=12, Epp=2, S=3, LB=40,
                     gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=True,
                     experts="identity", combine="q8", out_dtype="f32")
# two-hop case: 4 sources, 12 destination partitions, the first 4 are relays
TWOHOP_SMALL = mw.Workload("twohop_small", T=4 * 40, H=256, E=10, P=12, k=4, D=12, Epp=1, S=4,
                           LB=40, gating="sigmoid", logits_dtype="bf16", x_dtype="bf16",
                           zipf=False, experts="synthetic", combine="bf16", out_dtype="bf16",
                           eplb="first32", budget=2, relays=4)


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _release_device_memory():
    """Full-size cases hold tens of GB of static buffers: give them back after each test."""
    yield
    import gc
    gc.collect()
    torch.cuda.empty_cache()


class Case:
    """Everything one workload needs, on the host (oracle) and on the device."""

    def __init__(self, w: mw.Workload, event_id: int = 0x1234):
        _log(f"[case] {w.name} T={w.T} H={w.H} E={w.E} P={w.P} k={w.k} D={w.D} S={w.S}")
        self.w = w
        self.event_id = event_id
        self.lg = mw.logits(w)
        self.bias = mw.zipf_bias(w)
        self.x = mw.hidden(w)
        cal = calib_ids(w) if w.eplb == "plan" else None
        self.ro, self.rs, self.sp, self.sl = replica_map(w, cal)
        self.use_map = w.eplb != "none"
        self.g = moe.geom_of(w)
        self.layer = moe.MoeLayer(
            self.g, w.gating, to_dev(self.sp), to_dev(self.sl),
            to_dev(self.ro) if self.use_map else None, to_dev(self.rs) if self.use_map else None,
            None if self.bias is None else to_dev(self.bias), None, w.I,
            torch.bfloat16 if w.out_dtype == "bf16" else torch.float32)
        self.lg_d = dev_bits(self.lg, w.logits_dtype == "bf16")
        self.x_d = dev_bits(self.x, w.x_dtype == "bf16")

    # oracle side
    def oracle_route(self):
        w = self.w
        ids, sc, tw = oracle.route_topk(self.lg, w.k, w.gating, self.bias,
                                        logits_bf16=w.logits_dtype == "bf16")
        phys = oracle.eplb_phys(ids, w.LB, w.E, self.ro if self.use_map else None,
                                self.rs if self.use_map else None)
        return ids, tw, phys

    def oracle_dispatch(self, phys):
        w = self.w
        q, s = oracle.quant_tokens(self.x, w.x_dtype == "bf16")
        lay = oracle.dispatch_layout(w, phys, self.sp, self.event_id)
        return q, s, lay


def _check_route(c: Case):
    w = c.w
    c.layer.route(c.lg_d)
    ids, tw, phys = c.oracle_route()
    b = c.layer.buf
    assert np.array_equal(host(b.topk_ids), ids), "topk ids"
    assert np.array_equal(host(b.phys), phys), "physical ids"
    assert_close(host(b.topk_w), tw, FP32_RTOL, FP32_ATOL, "topk weights")
    assert np.array_equal(host(b.expert_counts), oracle.expert_counts(ids, w.E)), "expert counts"
    return ids, tw, phys


def _check_dispatch(c: Case, phys, row_sample=None):
    w = c.w
    b = c.layer.buf
    c.layer.event_id = c.event_id - 1
    c.layer.dispatch(c.x_d)
    q, s, lay = c.oracle_dispatch(phys)
    torch.cuda.synchronize()
    assert b.device_status() == 0
    meta = host(b.meta)
    assert np.array_equal(meta[..., :3].view(np.uint32)[..., 0], lay["meta"][..., 0].view(np.uint32))
    assert np.array_equal(meta[..., 1:3], lay["meta"][..., 1:3]), "meta offset/count"
    assert np.array_equal(host(b.slot_count), lay["slot_count"])
    assert np.array_equal(host(b.slot_offset), lay["slot_offset"])
    assert np.array_equal(host(b.disp_row), lay["disp_row"]), "disp_row"
    assert np.array_equal(host(b.ret_row), lay["ret_row"]), "ret_row"
    assert np.array_equal(host(b.slot_rows), lay["slot_rows"]), "slot_rows"
    n = w.H + 16
    # the trailer's 128-byte line is stored whole: zeros behind the trailer
    pad_end = min(c.g.msg_bytes or w.msg, (n + 127) // 128 * 128)
    if row_sample is None:
        exp = oracle.dispatch_rows(w, q, s, phys, lay["slot_local"], c.event_id)
        got = gather_rows(b, lay["disp_row"].ravel())
        assert np.array_equal(got[:, :n], exp[:, :n]), "message rows"
        assert not got[:, n:pad_end].any(), "the rest of the trailer's line is zero"
    else:
        for t0, t1 in row_sample:
            exp = oracle.dispatch_rows(w, q, s, phys, lay["slot_local"], c.event_id, t0, t1)
            got = gather_rows(b, lay["disp_row"][t0:t1].ravel())
            assert np.array_equal(got[:, :n], exp[:, :n]), f"message rows of tokens [{t0}, {t1})"
            assert not got[:, n:pad_end].any(), "the rest of the trailer's line is zero"
    return q, s, lay


# ----------------------------------------------------------- gate logits ---

def _router_case(w, token_sample=None):
    """GPU gate logits of the workload's hidden states against the exact oracle,
    within the fp32 summation bound H * 2^-24 * sum |x w| (any order of fp32
    sums of the exact bf16 products stays inside it)."""
    c = Case(w)
    wr = mw.router_weights(w)
    logits = c.layer.router(c.x_d, dev_bits(wr, True))
    torch.cuda.synchronize()
    got = host(logits)
    rows = np.arange(w.T) if token_sample is None else token_sample
    ref = oracle.router_logits(np.ascontiguousarray(c.x[rows]), wr)
    mag = oracle.router_logits(np.ascontiguousarray(c.x[rows]) & np.uint16(0x7FFF),
                               wr & np.uint16(0x7FFF))
    err = np.abs(got[rows].astype(np.float64) - ref)
    bound = w.H * 2.0 ** -24 * mag + 1e-30
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"
    return c, got


@pytest.mark.parametrize("name", ["ragged", "decode96"])
def test_router_logits_and_topk(name):
    """Gate logits (bf16 MFMA, split-K, fixed-order reduction) within the fp32
    bound of the exact values; the top-k of the GPU's own fp32 logits is the
    oracle's top-k of the same logits bit for bit, and two runs give the same
    bits.  ragged: T = 300 (a partial 192-row tile), E = 40 (a partial expert
    tile), 6 K splits of one step each; decode96: T = 96, 28 K splits of 4 steps."""
    w = RAGGED if name == "ragged" else mw.WORKLOADS["decode96"]
    c, got = _router_case(w)
    again = host(c.layer.router(c.x_d, dev_bits(mw.router_weights(w), True)))
    assert np.array_equal(got, again), "deterministic"
    c.layer.route(to_dev(got))
    ids, sc, tw = oracle.route_topk(got, w.k, w.gating, c.bias, logits_bf16=False)
    b = c.layer.buf
    assert np.array_equal(host(b.topk_ids), ids), "top-k of the GPU logits"
    assert_close(host(b.topk_w), tw, FP32_RTOL, FP32_ATOL, "top-k weights")


@pytest.mark.parametrize("name", ["ragged", "decode96", "eplb4096"])
def test_router_topk_fused_equals_two_calls(name):
    """moe_router_topk (the top-k reading the gate's K-split partial sums) gives
    the same bits as moe_router_logits followed by moe_route_topk on fp32 logits:
    logits, ids, weights, physical ids (eplb4096: through the replica map) and
    expert counts; and the same routes when the logits are not kept."""
    w = RAGGED if name == "ragged" else mw.WORKLOADS[name]
    c = Case(w)
    wr = dev_bits(mw.router_weights(w), True)
    logits = c.layer.router(c.x_d, wr).clone()
    c.layer.route(logits)
    b = c.layer.buf
    outs = (b.topk_ids, b.topk_w, b.phys, b.expert_counts)
    ref = [host(t).copy() for t in outs]
    for keep in (True, False):
        for t in outs:
            t.fill_(-7)
        got = c.layer.route_from_hidden(c.x_d, wr, keep_logits=keep)
        torch.cuda.synchronize()
        if keep:
            assert np.array_equal(host(got).view(np.uint32), host(logits).view(np.uint32)), "logits"
        for label, t, r in zip(("ids", "weights", "physical ids", "counts"), outs, ref):
            a = host(t)
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  r.view(np.uint32) if r.dtype == np.float32 else r), label


@pytest.mark.parametrize("T,H,E,splits", [(4100, 192, 1020, 1), (200, 6144, 128, 32)])
def test_router_logits_tails(T, H, E, splits):
    """The gate kernel's edges through the C ABI: partial token tiles (4100 = 21 x
    192 + 68, 200 = 192 + 8), a partial expert tile (1020 = 3 x 256 + 252, and
    128 of 256), three K steps per block (one split of 3 steps; 32 splits of 96
    steps); logits within the fp32 bound of the exact values, and the same bits
    on a second run."""
    rng = np.random.default_rng(T + H + E)
    x = mw.to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    wr = mw.to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32) / np.float32(np.sqrt(H)))
    g = moe.geom(T=T, H=H, E=E, P=E, k=1, D=E, Epp=1, S=1, LB=T)
    sz = moe.moe_plan_sizes(g)
    assert sz.router_scratch_bytes == splits * T * E * 4
    scratch = torch.empty(sz.router_scratch_bytes // 4, dtype=torch.float32, device="cuda")
    runs = []
    for _ in range(2):
        logits = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
        _log(f"moe_router_logits T={T} H={H} E={E}")
        moe.moe_router_logits(dev_bits(x, True), dev_bits(wr, True), g, logits, scratch)
        torch.cuda.synchronize()
        runs.append(host(logits))
    ref = oracle.router_logits(x, wr)
    mag = oracle.router_logits(x & np.uint16(0x7FFF), wr & np.uint16(0x7FFF))
    err = np.abs(runs[0].astype(np.float64) - ref)
    assert np.all(err <= H * 2.0 ** -24 * mag + 1e-30), f"max err/bound {np.max(err / (H * 2.0 ** -24 * mag + 1e-30)):.3g}"
    assert np.array_equal(runs[0].view(np.uint32), runs[1].view(np.uint32)), "deterministic"


def test_router_logits_layer12288_sampled_tokens():
    """The gate at the headline shape (T = 12288, H = 7168, E = 256): 96 sampled
    tokens' logits within the fp32 bound of the exact values."""
    rng = np.random.default_rng(5)
    _router_case(mw.WORKLOADS["layer12288"], np.sort(rng.choice(12288, 96, replace=False)))


# ------------------------------------------------------------------ route ---

@pytest.mark.parametrize("name", ["tiny", "decode96", "global12288", "eplb4096", "twohop46080"])
def test_route_parity(name):
    c = Case(mw.WORKLOADS[name])
    _check_route(c)


def _selection_scores(rng, T, E, mode):
    if mode == "ties":      # few distinct values: most boundaries split a run of equal scores
        return rng.integers(-4, 5, (T, E)).astype(np.float32) * np.float32(0.25)
    if mode == "equal":     # every score equal: the k lowest ids, in id order
        return np.full((T, E), 0.5, np.float32)
    if mode == "zeros":     # +0 and -0 are one score
        return rng.choice(np.array([0.0, -0.0, 1.0, -1.0], np.float32), (T, E))
    return rng.standard_normal((T, E), dtype=np.float32)


@pytest.mark.parametrize("E,k,dtype,mode,biased", [
    (8, 2, "bf16", "ties", False), (96, 8, "f32", "ties", True), (200, 16, "bf16", "ties", False),
    (256, 8, "bf16", "equal", False), (256, 8, "f32", "normal", True),
    (513, 16, "f32", "normal", False), (1024, 16, "bf16", "ties", True),
    (64, 1, "f32", "zeros", False), (128, 3, "bf16", "normal", True)])
def test_route_selection_edge_cases(E, k, dtype, mode, biased):
    """The top-k select on scores built to stress it: a few distinct values
    (the k-th score is shared by many experts and the lower ids must win), all
    scores equal, +0 mixed with -0, expert counts that leave the last lanes'
    runs partial (E = 96, 200, 513) or use every lane (64 .. 1024), both logit
    dtypes, k from 1 to the maximum 16, with and without a bias.  T = 5000
    exceeds the capped grid's 4096 wavefronts, so some wavefronts take two
    tokens.  ids, weights and the expert histogram against the oracle."""
    T = 5000
    rng = np.random.default_rng(E * 131 + k)
    sc = _selection_scores(rng, T, E, mode)
    lg = mw.to_bf16_bits(sc) if dtype == "bf16" else sc
    bias = (rng.integers(-8, 9, E).astype(np.float32) * np.float32(0.125)) if biased else None
    _log(f"[case] route select E={E} k={k} {dtype} {mode} bias={biased}")
    gating = "softmax" if k % 2 else "sigmoid"
    g = moe.geom(T, 64, E, E, k, 1, E, 1, T)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    phys = torch.empty_like(ids)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    moe.moe_route_topk(dev_bits(lg, dtype == "bf16"), moe.DTYPE_BF16 if dtype == "bf16" else moe.DTYPE_F32,
                       None if bias is None else to_dev(bias),
                       moe.GATING_SOFTMAX if gating == "softmax" else moe.GATING_SIGMOID,
                       None, None, g, ids, tw, phys, counts)
    torch.cuda.synchronize()
    rids, _, rw = oracle.route_topk(lg, k, gating, bias, logits_bf16=dtype == "bf16")
    assert np.array_equal(host(ids), rids), "topk ids"
    assert np.array_equal(host(phys), rids), "physical ids without a replica map"
    assert_close(host(tw), rw, FP32_RTOL, FP32_ATOL, "topk weights")
    assert np.array_equal(host(counts), oracle.expert_counts(rids, E)), "expert counts"


# ---------------------------------------------------------- weight image ---

def _packed_image(w: np.ndarray, gateup: bool, H: int, I: int) -> np.ndarray:
    """The operand image that moe_pack_expert_weights documents, by numpy
    indexing: block (e, n, s), slot 1024 wv + 256 ks + 64 nb + l = K bytes
    64 s + 32 ks + 16 (l >> 5) .. +16 of tile row row(wv, nb, l); K padded to a
    multiple of four 64-byte steps with zeros; clamped rows in partial n-tiles."""
    E = w.shape[0]
    K = H if gateup else I
    KT = K // 64
    KTp = (KT + 3) // 4 * 4
    NT = (I + 127) // 128 if gateup else (H + 255) // 256
    out = np.zeros((E, NT, KTp, 4, 2, 2, 64, 16), np.int8)       # e n s wv ks nb l byte
    l = np.arange(64)
    for n in range(NT):
        for wv in range(4):
            for nb in range(2):
                if gateup:
                    r = nb * 128 + wv * 32 + (l & 31)
                    pair = np.minimum(n * 128 + (r % 128), I - 1)
                    rows = np.where(r < 128, pair, I + pair)
                else:
                    rows = np.minimum(n * 256 + wv * 64 + nb * 32 + (l & 31), H - 1)
                for s in range(KT):
                    for ks in range(2):
                        cols = 64 * s + 32 * ks + 16 * (l >> 5)
                        out[:, n, s, wv, ks, nb] = w[:, rows[:, None], cols[:, None] + np.arange(16)]
    return out.reshape(-1)


def test_pack_expert_weights_image():
    """The packed weights are the documented operand image byte for byte, for
    both projections, with partial n-tiles on both (I = 192 pairs of 128-pair
    tiles, H = 384 rows of 256-row tiles) and K padded to whole groups of four
    steps (K = 384: 6 -> 8 steps; K = 192: 3 -> 4)."""
    E, H, I = 3, 384, 192
    rng = np.random.default_rng(11)
    wgu = rng.integers(-128, 128, (E, 2 * I, H), dtype=np.int8)
    wd = rng.integers(-128, 128, (E, H, I), dtype=np.int8)
    sz = moe.moe_plan_sizes(moe.geom(0, H, E, E, 1, 1, 1, 1, 0), I)
    for w, proj, nbytes in ((wgu, moe.PROJ_GATEUP, sz.w_gateup_packed_bytes),
                            (wd, moe.PROJ_DOWN, sz.w_down_packed_bytes)):
        out = torch.empty(nbytes, dtype=torch.int8, device="cuda")
        moe.moe_pack_expert_weights(to_dev(w), proj, E, H, I, out)
        torch.cuda.synchronize()
        ref = _packed_image(w, proj == moe.PROJ_GATEUP, H, I)
        assert ref.size == nbytes
        assert np.array_equal(host(out), ref), f"image of projection {proj}"


# --------------------------------------------------------------- dispatch ---

@pytest.mark.parametrize("name", ["tiny", "decode96", "ragged", "smallb"])
def test_dispatch_parity_small(name):
    """tiny, decode96 and smallb take the one-launch path for at most 1024 routes,
    ragged (2400 routes) the count / scan / scatter path."""
    w = {"ragged": RAGGED, "smallb": SMALLB}.get(name) or mw.WORKLOADS[name]
    c = Case(w)
    _, _, phys = _check_route(c)
    _check_dispatch(c, phys)


def test_dispatch_parity_global12288_full():
    """T=12288, 128 sources x 96 tokens, 128 partitions x 2 slots, Zipf skew: the
    full layout and every one of the 98304 message rows."""
    c = Case(mw.WORKLOADS["global12288"])
    _, _, phys = _check_route(c)
    _check_dispatch(c, phys)


def test_dispatch_parity_eplb4096_full():
    c = Case(mw.WORKLOADS["eplb4096"])
    _, _, phys = _check_route(c)
    _check_dispatch(c, phys)


def test_expert_ffn_eplb4096_replicas_sampled_rows():
    """The EPLB layer at full size (T = 4096, 288 physical slots: 256 primaries and
    32 replicas from the planner, INT8 SwiGLU experts, I = 2048), launched as a
    caller would: the bf16 return rows of sampled rows are bit-exact against the
    oracle -- for the hottest primary, its replicas (which share the logical
    expert's weights) and two random slots -- and the layer output is within
    bf16 tolerance of the oracle's on sampled tokens."""
    w = mw.WORKLOADS["eplb4096"]
    c = Case(w)
    ids, tw, phys = _check_route(c)
    c.layer.dispatch(c.x_d)
    q, s = oracle.quant_tokens(c.x, True)
    lay = oracle.dispatch_layout(w, phys, c.sp, 1)
    _log("[eplb4096] generating weights of the routed experts")
    routed = np.unique(c.sl[phys.ravel()])
    dev = dict(device="cuda")
    wgu_d = torch.zeros((w.E, 2 * w.I, w.H), dtype=torch.int8, **dev)
    sgu_d = torch.zeros((w.E, 2 * w.I), dtype=torch.float32, **dev)
    wd_d = torch.zeros((w.E, w.H, w.I), dtype=torch.int8, **dev)
    sd_d = torch.zeros((w.E, w.H), dtype=torch.float32, **dev)
    host_w = {}
    for e in routed:
        a, b, c2, d = mw.expert_weights(w, int(e))
        host_w[int(e)] = (a, b, c2, d)
        wgu_d[e].copy_(torch.from_numpy(a))
        sgu_d[e].copy_(torch.from_numpy(b))
        wd_d[e].copy_(torch.from_numpy(c2))
        sd_d[e].copy_(torch.from_numpy(d))
    c.layer.weights = (wgu_d, sgu_d, wd_d, sd_d)
    c.layer.I = w.I
    c.layer.experts()
    c.layer.combine("bf16")
    torch.cuda.synchronize()
    b = c.layer.buf
    assert np.array_equal(host(b.ret_row), lay["ret_row"])
    ret = host(b.ret.view(torch.int16)).view(np.uint16)
    sc = lay["slot_count"]
    hot = int(np.argmax(sc[:w.E]))
    reps = [int(p) for p in range(w.E, w.P) if c.sl[p] == c.sl[hot] and sc[p] > 0]
    assert reps, "the hottest expert has a replica under the planner"
    rng = np.random.default_rng(1)
    nz = np.nonzero(sc)[0]
    slots = sorted({hot, *reps, *rng.choice(nz, 2).tolist()})
    inv = np.argsort(lay["ret_row"].ravel())
    for p in slots:
        o = lay["slot_offset"][p]
        rows = np.arange(o, o + sc[p])
        if len(rows) > 24:
            rows = np.sort(rng.choice(rows, 24, replace=False))
        toks = inv[rows] // w.k
        e = int(c.sl[p])
        y, *_ = oracle.expert_ffn(q[toks], s[toks], *host_w[e])
        assert np.array_equal(ret[rows], y), f"slot {p} (expert {e}, {sc[p]} rows)"
    # layer output of sampled tokens: oracle combine of the oracle's returns
    tsel = np.sort(rng.choice(w.T, 16, replace=False))
    out = host(b.out.view(torch.int16)).view(np.uint16)
    rr = lay["ret_row"]
    logical = c.sl[phys]
    vals = np.empty((len(tsel) * w.k, w.H), np.uint16)
    for i, t in enumerate(tsel):
        for j in range(w.k):
            e = int(logical[t, j])
            y, *_ = oracle.expert_ffn(q[t:t + 1], s[t:t + 1], *host_w[e])
            vals[i * w.k + j] = y[0]
    ident = np.arange(len(tsel) * w.k, dtype=np.int32).reshape(len(tsel), w.k)
    ref = oracle.combine(vals, ident, tw[tsel].astype(np.float32), w.k, w.H, "bf16", True)
    assert_close(bf16_to_f32(out[tsel]), bf16_to_f32(ref), BF16_RTOL, BF16_ATOL, "layer output")


def test_dispatch_twohop_small_equals_direct():
    """Two-hop (relays = 4): layout and rows equal the oracle's one-hop layout,
    and a direct run (relays = 0) writes the same bytes."""
    c = Case(TWOHOP_SMALL)
    _, _, phys = _check_route(c)
    _check_dispatch(c, phys)
    direct = Case(TWOHOP_SMALL.scaled(relays=0))
    _check_route(direct)
    direct.layer.event_id = c.event_id - 1
    direct.layer.dispatch(direct.x_d)
    rows = host(c.layer.buf.disp_row).ravel()
    n = c.w.H + 16  # codes + trailer; the line padding after them is unspecified
    assert np.array_equal(gather_rows(c.layer.buf, rows)[:, :n],
                          gather_rows(direct.layer.buf, rows)[:, :n])


@pytest.mark.parametrize("i", range(6))
def test_random_twohop_geometries(i):
    """Seeded two-hop geometries (one slot per partition, 1..E redundant slots, 1..D-1
    relay partitions): the layout and rows after the second hop bit-exact against
    the oracle's one-hop layout, and the E2A relay plus combine of synthetic bf16
    returns bit-exact against the oracle's combine of the same rows."""
    rng = np.random.default_rng(4242 + i)
    E = int(rng.choice([6, 10, 17, 30]))
    budget = int(rng.integers(1, E + 1))
    P = E + budget
    S, LB = int(rng.integers(1, 6)), int(rng.integers(5, 51))
    w = mw.Workload(f"twohop_rand{i}", T=S * LB, H=16 * int(rng.integers(1, 33)), E=E, P=P,
                    k=int(rng.integers(1, min(8, E) + 1)), D=P, Epp=1, S=S, LB=LB,
                    gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=bool(i % 2),
                    experts="synthetic", combine="bf16", out_dtype="bf16", eplb="first32",
                    budget=budget, relays=int(rng.integers(1, P)), seed=int(rng.integers(1 << 30)))
    _log(f"[twohop random] {w}")
    c = Case(w)
    ids, tw, phys = _check_route(c)
    _check_dispatch(c, phys)
    b = c.layer.buf
    rets = mw.route_returns(w)
    rr = torch.from_numpy(host(b.ret_row).ravel().astype(np.int64)).cuda()
    b.ret[: w.T * w.k].index_copy_(0, rr, torch.from_numpy(rets.view(np.int16)).cuda())
    c.layer.combine("bf16")
    torch.cuda.synchronize()
    out = host(b.out.view(torch.int16)).view(np.uint16)
    ident = np.arange(w.T * w.k, dtype=np.int32).reshape(w.T, w.k)
    ref = oracle.combine(rets, ident, host(b.topk_w), w.k, w.H, "bf16", True)
    assert np.array_equal(out, ref), "E2A relay + combine"


def test_dispatch_twohop46080_full_layout_all_rows():
    """46080 tokens from 160 sources to 288 partitions through 160 relays: full
    layout, and every one of the 368,640 message rows (checked in token chunks)."""
    c = Case(mw.WORKLOADS["twohop46080"])
    _, _, phys = _check_route(c)
    T = c.w.T
    _check_dispatch(c, phys, row_sample=[(t0, min(T, t0 + 2048)) for t0 in range(0, T, 2048)])


def test_twohop46080_e2a_combine_full_size():
    """The E2A hop and the combine at full size (46080 tokens, 288 partitions, 160
    relays; the routes to partitions >= 160 come back through relay staging):
    synthetic bf16 returns for all 368,640 routes; 1024 sampled tokens compared
    with the oracle's combine of the same returns, bit for bit given the same
    fp32 weights and within the bf16 tolerance end to end (oracle weights)."""
    w = mw.WORKLOADS["twohop46080"]
    c = Case(w)
    ids, tw, phys = _check_route(c)
    c.layer.dispatch(c.x_d)
    b = c.layer.buf
    torch.cuda.synchronize()
    rr = host(b.ret_row).ravel()
    n = w.T * w.k
    assert np.array_equal(np.sort(rr), np.arange(n)), "every route has its own return row"
    for r0 in range(0, n, 32768):
        routes = np.arange(r0, min(n, r0 + 32768))
        vals = torch.from_numpy(mw.route_returns(w, routes).view(np.int16)).cuda()
        b.ret[:n].index_copy_(0, torch.from_numpy(rr[routes].astype(np.int64)).cuda(), vals)
        del vals
    c.layer.combine("bf16")
    torch.cuda.synchronize()
    comb = host(b.comb_row)
    assert int((comb >= n).sum()) > 0.3 * n, "routes to partitions >= 160 go through the relays"
    out = host(b.out.view(torch.int16)).view(np.uint16)
    rng = np.random.default_rng(5)
    tsel = np.sort(rng.choice(w.T, 1024, replace=False))
    routes = (tsel[:, None] * w.k + np.arange(w.k)).ravel()
    vals = mw.route_returns(w, routes)
    ident = np.arange(len(routes), dtype=np.int32).reshape(len(tsel), w.k)
    w_gpu = host(b.topk_w)[tsel]
    ref = oracle.combine(vals, ident, w_gpu, w.k, w.H, "bf16", True)
    assert np.array_equal(out[tsel], ref), "E2A + combine bits (same fp32 weights)"
    ref2 = oracle.combine(vals, ident, tw[tsel].astype(np.float32), w.k, w.H, "bf16", True)
    assert_close(bf16_to_f32(out[tsel]), bf16_to_f32(ref2), BF16_RTOL, BF16_ATOL, "end to end")


def test_stale_event_detected():
    """The receiver's event check of the dispatch protocol (XDS P039-P040): the
    current dispatch's metadata and messages pass; metadata of an older dispatch,
    an expected id the buffers do not carry, or one message trailer of another
    event set the stale bit (the kernels end normally); the layer's debug mode
    turns it into MOE_ERR_STALE, and a fresh dispatch clears the condition."""
    c = Case(RAGGED)
    w = c.w
    c.layer.route(c.lg_d)
    b = c.layer.buf
    c.layer.event_id = 10
    c.layer.dispatch(c.x_d)  # event 11
    old_meta = b.meta.clone()
    c.layer.dispatch(c.x_d)  # event 12
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def check(meta, ev):
        status.fill_(-1)  # the call writes the word
        moe.moe_check_event(meta, b.disp_buf, b.slot_rows, b.slot_offset, c.g, ev, status)
        torch.cuda.synchronize()
        return int(host(status)[0])

    assert check(b.meta, 12) == 0
    assert check(old_meta, 12) == moe.MOE_DEVICE_STALE_EVENT
    assert check(b.meta, 13) == moe.MOE_DEVICE_STALE_EVENT
    # one routed row whose trailer carries the previous event (metadata current)
    row = int(host(b.slot_rows)[7])
    v = b.disp_rows_view()
    saved = v[row, w.H + 14:w.H + 16].clone()
    v[row, w.H + 14] = 11
    v[row, w.H + 15] = 0
    assert check(b.meta, 12) == moe.MOE_DEVICE_STALE_EVENT
    # the layer in debug mode refuses to consume them
    c.layer.debug_checks = True
    with pytest.raises(moe.MoeError) as err:
        c.layer.combine("q8")
    assert err.value.status == moe.MOE_ERR_STALE
    v[row, w.H + 14:w.H + 16] = saved
    c.layer.combine("q8")  # the same dispatch, restored: passes
    c.layer.event_id = 20  # the caller thinks a later dispatch ran
    with pytest.raises(moe.MoeError):
        c.layer.combine("q8")
    c.layer.dispatch(c.x_d)  # event 21: consistent again
    c.layer.combine("q8")
    torch.cuda.synchronize()
    assert b.device_status() == 0


def test_dispatch_is_deterministic():
    c = Case(RAGGED)
    c.layer.route(c.lg_d)
    c.layer.dispatch(c.x_d)
    b = c.layer.buf
    a1 = [host(t).copy() for t in (b.disp_row, b.ret_row, b.slot_rows, b.meta)]
    rows1 = gather_rows(b, a1[0].ravel())
    c.layer.event_id -= 1
    c.layer.dispatch(c.x_d)
    a2 = [host(t) for t in (b.disp_row, b.ret_row, b.slot_rows, b.meta)]
    for u, v in zip(a1, a2):
        assert np.array_equal(u, v)
    assert np.array_equal(rows1, gather_rows(b, a1[0].ravel()))


# ---------------------------------------------------------------- combine ---

@pytest.mark.parametrize("name", ["tiny", "decode96", "ragged"])
def test_combine_q8_identity_experts(name):
    """Identity experts: combine reads the dispatched INT8 rows back.  With the
    oracle's fp32 weights the output is bit-identical to the oracle's; the
    end-to-end output (GPU weights) is within the fp32 tolerance."""
    w = RAGGED if name == "ragged" else mw.WORKLOADS[name]
    c = Case(w)
    ids, tw, phys = _check_route(c)
    q, s, lay = _check_dispatch(c, phys)
    b = c.layer.buf
    rows = oracle.dispatch_rows(w, q, s, phys, lay["slot_local"], c.event_id)
    ident = np.arange(w.T * w.k, dtype=np.int32).reshape(w.T, w.k)
    w32 = tw.astype(np.float32)
    ref = oracle.combine(rows, ident, w32, w.k, w.H, "q8", False, scale_offset=w.H)
    c.layer.combine("q8")
    assert_close(host(b.out), ref, FP32_RTOL, FP32_ATOL, "combine end to end")
    out2 = torch.empty_like(b.out)
    moe.moe_combine(moe.RET_Q8_FROM_DISPATCH, b.disp_buf, b.disp_row, to_dev(w32), c.g,
                    moe.DTYPE_F32, out2)
    assert np.array_equal(host(out2), ref), "combine with identical weights is bit-exact"
    # closed form: sum_j w_j dequant(quant(x)) ~ x
    xf = bf16_to_f32(c.x) if w.x_dtype == "bf16" else c.x
    assert np.all(np.abs(host(out2) - xf) <= s[:, None] * 0.5 + 1e-5 * np.abs(xf) + 1e-6)


def _random_geometries(n=24, seed=20261202):
    """Seeded small geometries across the ABI's ranges: E from 1 to 512 (whole and
    partial 64-lane runs of the top-k), k from 1 to min(16, E), 1-4 slots per
    partition, H any multiple of 16 up to 1520, 1-5 sources of 1-49 tokens, both
    gatings and both input types, with and without the Zipf bias."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 5, 8, 13, 31, 64, 100, 257, 512]))
        k = int(rng.integers(1, min(16, E) + 1))
        Epp = int(rng.integers(1, 5))
        S, LB = int(rng.integers(1, 6)), int(rng.integers(1, 50))
        out.append(mw.Workload(
            f"rand{i}", T=S * LB, H=16 * int(rng.integers(1, 96)), E=E, P=E, k=k,
            D=(E + Epp - 1) // Epp, Epp=Epp, S=S, LB=LB,
            gating=str(rng.choice(["softmax", "sigmoid"])),
            logits_dtype=str(rng.choice(["f32", "bf16"])), x_dtype=str(rng.choice(["f32", "bf16"])),
            zipf=bool(rng.integers(0, 2)), experts="identity", combine="q8", out_dtype="f32",
            seed=int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("w", _random_geometries(), ids=lambda w: w.name)
def test_random_geometries_route_dispatch_combine(w):
    """Twenty-four seeded geometries: routing, the dispatch layout and message rows
    bit-exact against the oracle, and the INT8 combine of the dispatched rows
    bit-exact in fp32 and bf16 given the oracle's weights."""
    _log(f"[random] {w}")
    c = Case(w)
    ids, tw, phys = _check_route(c)
    q, s, lay = _check_dispatch(c, phys)
    b = c.layer.buf
    rows = oracle.dispatch_rows(w, q, s, phys, lay["slot_local"], c.event_id)
    ident = np.arange(w.T * w.k, dtype=np.int32).reshape(w.T, w.k)
    w32 = tw.astype(np.float32)
    for bf, dt in ((False, moe.DTYPE_F32), (True, moe.DTYPE_BF16)):
        ref = oracle.combine(rows, ident, w32, w.k, w.H, "q8", bf, scale_offset=w.H)
        out = torch.empty((w.T, w.H), dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
        moe.moe_combine(moe.RET_Q8_FROM_DISPATCH, b.disp_buf, b.disp_row, to_dev(w32), c.g, dt, out)
        torch.cuda.synchronize()
        got = host(out.view(torch.int16)).view(np.uint16) if bf else host(out)
        assert np.array_equal(got, ref), f"combine ({'bf16' if bf else 'fp32'} output)"


@pytest.mark.parametrize("i", range(8))
def test_random_replica_maps_route_dispatch_combine(i):
    """EPLB gather with seeded random replica maps: every expert keeps one slot and
    1..E extra slots go to random experts, the physical slot ids are shuffled, and
    the slots are dealt to partitions at random (at most Epp each).  Physical ids
    (R_e[b mod |R_e|]), the dispatch layout and rows, and the INT8 combine are
    bit-exact against the oracle on the same maps."""
    rng = np.random.default_rng(9000 + i)
    E = int(rng.choice([4, 9, 16, 33, 64]))
    extra = int(rng.integers(1, E + 1))
    P, Epp = E + extra, int(rng.integers(1, 4))
    S, LB = int(rng.integers(1, 4)), int(rng.integers(5, 60))
    w = mw.Workload(f"rmap{i}", T=S * LB, H=16 * int(rng.integers(1, 40)), E=E, P=P,
                    k=int(rng.integers(1, min(8, E) + 1)), D=(P + Epp - 1) // Epp, Epp=Epp, S=S,
                    LB=LB, gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=True,
                    experts="identity", combine="q8", out_dtype="f32", seed=int(rng.integers(1 << 30)))
    sl = np.r_[np.arange(E), rng.integers(0, E, extra)].astype(np.int32)[rng.permutation(P)]
    sp = rng.permutation(np.arange(P) // Epp).astype(np.int32)
    ro = np.zeros(E + 1, np.int32)
    ro[1:] = np.cumsum(np.bincount(sl, minlength=E))
    rs = np.argsort(sl, kind="stable").astype(np.int32)  # each expert's slots, ascending
    _log(f"[replica map] {w} copies {np.bincount(sl, minlength=E).tolist()}")
    c = Case(w)
    c.ro, c.rs, c.sp, c.sl, c.use_map = ro, rs, sp, sl, True
    c.layer = moe.MoeLayer(c.g, w.gating, to_dev(sp), to_dev(sl), to_dev(ro), to_dev(rs),
                           to_dev(c.bias), None, 0, torch.float32)
    ids, tw, phys = _check_route(c)
    assert np.array_equal(sl[phys], ids), "every route lands on a replica of its expert"
    q, s, lay = _check_dispatch(c, phys)
    rows = oracle.dispatch_rows(w, q, s, phys, lay["slot_local"], c.event_id)
    ident = np.arange(w.T * w.k, dtype=np.int32).reshape(w.T, w.k)
    w32 = tw.astype(np.float32)
    ref = oracle.combine(rows, ident, w32, w.k, w.H, "q8", False, scale_offset=w.H)
    out = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    b = c.layer.buf
    moe.moe_combine(moe.RET_Q8_FROM_DISPATCH, b.disp_buf, b.disp_row, to_dev(w32), c.g,
                    moe.DTYPE_F32, out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), ref), "combine"


# the ABI's limits: H = MOE_MAX_H (the scatter's sixteen 1024-element slices per
# row), k = MOE_MAX_K, E = P = D = 1024 (the top-k's sixteen experts per lane);
# 3072 routes take the count / scan / scatter path, 1024 the one-launch path
MAXDIM = mw.Workload("maxdim", T=2 * 96, H=16384, E=1024, P=1024, k=16, D=1024, Epp=1, S=2, LB=96,
                     gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=True,
                     experts="identity", combine="q8", out_dtype="f32")
MAXDIM_SMALL = MAXDIM.scaled(name="maxdim_small", T=64, S=1, LB=64)


@pytest.mark.parametrize("w", [MAXDIM, MAXDIM_SMALL], ids=lambda w: w.name)
def test_dispatch_and_combine_at_the_abi_limits(w):
    """Route, dispatch and the identity-expert combine at the ABI's maximum
    H, k, E, P and D: ids, layout and every message row bit-exact, the combine
    bit-exact given the same fp32 weights and within tolerance end to end."""
    assert w.H == moe.MAX_H and w.k == moe.MAX_K and w.P == moe.MAX_P and w.D == moe.MAX_D
    c = Case(w)
    ids, tw, phys = _check_route(c)
    q, s, lay = _check_dispatch(c, phys)
    assert (w.T * w.k > 1024) == (w.name == "maxdim"), "both dispatch paths are covered"
    b = c.layer.buf
    rows = oracle.dispatch_rows(w, q, s, phys, lay["slot_local"], c.event_id)
    ident = np.arange(w.T * w.k, dtype=np.int32).reshape(w.T, w.k)
    w32 = tw.astype(np.float32)
    ref = oracle.combine(rows, ident, w32, w.k, w.H, "q8", False, scale_offset=w.H)
    c.layer.combine("q8")
    assert_close(host(b.out), ref, FP32_RTOL, FP32_ATOL, "combine end to end")
    out2 = torch.empty_like(b.out)
    moe.moe_combine(moe.RET_Q8_FROM_DISPATCH, b.disp_buf, b.disp_row, to_dev(w32), c.g,
                    moe.DTYPE_F32, out2)
    assert np.array_equal(host(out2), ref), "combine with identical weights is bit-exact"


def test_combine_bf16_returns_global12288():
    """Synthetic bf16 expert returns at T=12288: bf16 output bit-identical to the
    oracle given the same fp32 weights, and within tolerance end to end."""
    c = Case(mw.WORKLOADS["global12288"])
    w = c.w
    ids, tw, phys = _check_route(c)
    c.layer.dispatch(c.x_d)
    lay = oracle.dispatch_layout(w, phys, c.sp, 1)
    b = c.layer.buf
    torch.cuda.synchronize()
    assert np.array_equal(host(b.ret_row), lay["ret_row"])
    rets = mw.route_returns(w)
    ret_d = torch.from_numpy(rets.view(np.int16)).cuda()
    b.ret.index_copy_(0, torch.from_numpy(lay["ret_row"].ravel().astype(np.int64)).cuda(), ret_d)
    del ret_d
    ident = np.arange(w.T * w.k, dtype=np.int32).reshape(w.T, w.k)
    w32 = tw.astype(np.float32)
    ref = oracle.combine(rets, ident, w32, w.k, w.H, "bf16", True)
    out2 = torch.empty_like(b.out)
    moe.moe_combine(moe.RET_BF16, b.ret, b.ret_row, to_dev(w32), c.g, moe.DTYPE_BF16, out2)
    assert np.array_equal(host(out2.view(torch.int16)).view(np.uint16), ref), "bf16 combine bits"
    c.layer.combine("bf16")
    assert_close(bf16_to_f32(host(b.out.view(torch.int16))), bf16_to_f32(ref), BF16_RTOL, BF16_ATOL,
                 "combine end to end")


def test_combine_bf16_output_rounding_edges():
    """The bf16 output's round to nearest even, bit-exact against the oracle, where
    it is hardest: each token's sum is one fp32 product w * v (the second route
    weighs 0), over random values of every exponent, subnormal products, exact
    ties (even and odd neighbours) and the bf16 maximum times (1 + 2^-9) and
    (1 + 2^-8), which round to the maximum and to infinity."""
    T, k, H = 64, 2, 1024
    g = moe.geom(T=T, H=H, E=8, P=8, k=k, D=8, Epp=1, S=1, LB=T)
    rng = np.random.default_rng(53)
    rets = np.zeros((T * k, H), np.uint16)
    w = np.zeros((T, k), np.float32)
    # random finite bf16 values up to 2^119 and weights 2^-40 .. 2^7: products stay finite
    exp_bits = rng.integers(0, 0xF7, (T, H)).astype(np.uint16)
    rets[0::k] = (rng.integers(0, 2, (T, H)).astype(np.uint16) << 15) | (exp_bits << 7) | \
        rng.integers(0, 0x80, (T, H)).astype(np.uint16)
    rets[1::k] = rng.integers(0, 0x7F00, (T, H)).astype(np.uint16)
    w[:, 0] = (rng.uniform(1, 2, T) * np.exp2(rng.integers(-40, 8, T)) *
               rng.choice([-1, 1], T)).astype(np.float32)
    w[0, 0] = np.float32(2.0 ** -15)  # token 0: products of tiny values are fp32 subnormals
    rets[0] = (rng.integers(0x0080, 0x0A00, H)).astype(np.uint16)
    f2b = lambda v: (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w[1, 0] = np.float32(1 + 2.0 ** -8)  # token 1: ties between bf16 neighbours
    rets[2, :4] = f2b([1.0, 1.0078125, -1.0, -1.0078125])
    w[2, 0] = np.float32(1 + 2.0 ** -9)  # tokens 2, 3: the bf16 maximum, rounded down / up
    w[3, 0] = np.float32(1 + 2.0 ** -8)
    rets[4, :] = 0x7F7F
    rets[6, :] = 0x7F7F
    ret_d = torch.from_numpy(rets.view(np.int16)).cuda()
    row = np.arange(T * k, dtype=np.int32).reshape(T, k)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(moe.RET_BF16, ret_d, to_dev(row), to_dev(w), g, moe.DTYPE_BF16, out)
    ref = oracle.combine(rets, row, w, k, H, "bf16", True)
    got = host(out.view(torch.int16)).view(np.uint16)
    assert np.array_equal(got, ref), "bf16 output bits"
    assert got[1, 0] == 0x3F80 and got[1, 1] == 0x3F82  # ties go to the even neighbour
    assert np.all(got[2] == 0x7F7F) and np.all(got[3] == 0x7F80)
    assert np.any((got[0] & 0x7F80) == 0) and np.any(got[0] & 0x7FFF)  # subnormal outputs


def test_combine_twohop_returns_equal_direct():
    """E2A through relays gives the same bf16 output bits as reading the returns directly."""
    c = Case(TWOHOP_SMALL)
    w = c.w
    ids, tw, phys = _check_route(c)
    c.layer.dispatch(c.x_d)
    b = c.layer.buf
    rets = mw.route_returns(w)
    rr = torch.from_numpy(host(b.ret_row).ravel().astype(np.int64)).cuda()
    b.ret[: w.T * w.k].index_copy_(0, rr, torch.from_numpy(rets.view(np.int16)).cuda())
    c.layer.combine("bf16")
    relayed = host(b.out.view(torch.int16)).copy()
    comb = host(b.comb_row)
    n_rel = int((comb >= w.T * w.k).sum())
    assert n_rel > 0, "some routes must go through a relay"
    direct = torch.empty_like(b.out)
    moe.moe_combine(moe.RET_BF16, b.ret, b.ret_row, b.topk_w, c.g, moe.DTYPE_BF16, direct)
    assert np.array_equal(relayed, host(direct.view(torch.int16)))
    ident = np.arange(w.T * w.k, dtype=np.int32).reshape(w.T, w.k)
    ref = oracle.combine(rets, ident, host(b.topk_w), w.k, w.H, "bf16", True)
    assert np.array_equal(relayed.view(np.uint16), ref)


# ------------------------------------------------------------- expert FFN ---

def _ffn_case(w):
    c = Case(w)
    ids, tw, phys = _check_route(c)
    q, s, lay = _check_dispatch(c, phys)
    wgu, sgu, wd, sd = mw.all_expert_weights(w)
    c.layer.weights = (to_dev(wgu), to_dev(sgu), to_dev(wd), to_dev(sd))
    c.layer.I = w.I
    return c, (ids, tw, phys), (q, s, lay), (wgu, sgu, wd, sd)


def _check_expert_ffn(c, phys, q, s, lay, weights):
    """Both GEMMs' int32 accumulators and the bf16 return rows of every routed
    row bit-exact against the oracle's expert FFN of the same rows."""
    w = c.w
    wgu, sgu, wd, sd = weights
    n = w.T * w.k
    acc_gu = torch.empty((n, 2 * w.I), dtype=torch.int32, device="cuda")
    acc_d = torch.empty((n, w.H), dtype=torch.int32, device="cuda")
    c.layer.experts(acc_gu, acc_d)
    torch.cuda.synchronize()
    b = c.layer.buf
    logical = c.sl[phys.ravel()]
    ret = host(b.ret.view(torch.int16)).view(np.uint16)
    agu, ad = host(acc_gu), host(acc_d)
    rr = lay["ret_row"].ravel()
    ys = {}  # expert -> (its return rows, the oracle's bf16 rows)
    for e in np.unique(logical):
        sel = np.nonzero(logical == e)[0]
        toks = sel // w.k
        y, hq, hs, o_gu, o_d = oracle.expert_ffn(q[toks], s[toks], wgu[e], sgu[e], wd[e], sd[e],
                                                 want_acc=True)
        assert np.array_equal(agu[rr[sel]], o_gu), f"gate/up accumulators, expert {e}"
        assert np.array_equal(ad[rr[sel]], o_d), f"down accumulators, expert {e}"
        assert np.array_equal(ret[rr[sel]], y), f"return rows, expert {e}"
        ys[e] = (rr[sel], y)
    return ys


def test_expert_ffn_parity_small():
    """Grouped INT8 SwiGLU: int32 accumulators of both GEMMs bit-exact, and the
    bf16 return rows bit-exact (the same fp32 epilogue on both sides)."""
    w = FFN_SMALL
    c, (ids, tw, phys), (q, s, lay), (wgu, sgu, wd, sd) = _ffn_case(w)
    sc = lay["slot_count"]
    assert sc.max() > 256, "want a slot spanning three 128-row m-tiles"
    assert 0 < sc[sc > 0].min() < 32, "want a slot smaller than one 32-row MFMA block"
    _check_expert_ffn(c, phys, q, s, lay, (wgu, sgu, wd, sd))


# expert GEMMs at the ABI's widths: I = 4096 and I = 16384 (the requantization
# takes a second pass over rows longer than 2048 values; 32 and 128 gate/up
# n-tiles), and H = MOE_MAX_H (256 K steps of gate/up, 64 down n-tiles)
FFN_WIDE = [
    mw.Workload("ffn_wide_i", T=2 * 200, H=512, E=8, P=8, k=2, D=4, Epp=2, S=2, LB=200,
                gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=True,
                experts="swiglu", combine="bf16", out_dtype="bf16", I=4096),
    mw.Workload("ffn_max_i", T=100, H=256, E=4, P=4, k=2, D=2, Epp=2, S=1, LB=100,
                gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=True,
                experts="swiglu", combine="bf16", out_dtype="bf16", I=16384),
    mw.Workload("ffn_max_h", T=160, H=16384, E=4, P=4, k=2, D=2, Epp=2, S=1, LB=160,
                gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=True,
                experts="swiglu", combine="bf16", out_dtype="bf16", I=256),
]


@pytest.mark.parametrize("w", FFN_WIDE, ids=lambda w: w.name)
def test_expert_ffn_parity_at_the_abi_widths(w):
    """Both GEMMs' int32 accumulators and the bf16 return rows bit-exact at the
    widest H and I the ABI takes."""
    c, (ids, tw, phys), (q, s, lay), (wgu, sgu, wd, sd) = _ffn_case(w)
    _check_expert_ffn(c, phys, q, s, lay, (wgu, sgu, wd, sd))


def _random_ffn_geometries(n=10, seed=7051):
    """Seeded small expert-FFN geometries: H any multiple of 128 up to 1024, I any
    multiple of 64 up to 1024, 2-24 experts, k up to min(6, E), 1-4 slots per
    partition, 1-3 sources of 10-80 tokens, with and without the Zipf bias."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(2, 25))
        Epp = int(rng.integers(1, 5))
        S, LB = int(rng.integers(1, 4)), int(rng.integers(10, 81))
        out.append(mw.Workload(
            f"ffnrand{i}", T=S * LB, H=128 * int(rng.integers(1, 9)), E=E, P=E,
            k=int(rng.integers(1, min(6, E) + 1)), D=(E + Epp - 1) // Epp, Epp=Epp, S=S, LB=LB,
            gating="sigmoid", logits_dtype="bf16", x_dtype=str(rng.choice(["f32", "bf16"])),
            zipf=bool(rng.integers(0, 2)), experts="swiglu", combine="bf16", out_dtype="bf16",
            I=64 * int(rng.integers(1, 17)), seed=int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("w", _random_ffn_geometries(), ids=lambda w: w.name)
def test_random_geometries_expert_ffn(w):
    """Ten seeded expert-FFN geometries: int32 accumulators and bf16 return rows
    bit-exact against the oracle, and both INT8 return encodings of those rows
    (one scale per 256 columns from the down epilogue, one per row from the
    quantize pass; an odd multiple of 128 for H leaves the last block half full)
    bit-exact."""
    _log(f"[random ffn] {w}")
    c, (ids, tw, phys), (q, s, lay), weights = _ffn_case(w)
    ys = _check_expert_ffn(c, phys, q, s, lay, weights)
    b = c.layer.buf
    rb = b.sizes.ret_q8_row_bytes
    c.layer.quant_returns()
    torch.cuda.synchronize()
    tokenwise = host(b.ret_q8_rows()).copy()
    c.layer.experts_gateup()
    c.layer.experts_down_int8ret()
    torch.cuda.synchronize()
    blocks = host(b.ret_q8_rows())
    nb = w.H + 4 * ((w.H + moe.RET_Q8_BLOCK - 1) // moe.RET_Q8_BLOCK)
    for e, (rows, y) in ys.items():
        exp = _int8_return_rows_oracle(w, y, rb)
        assert np.array_equal(blocks[rows, :nb], exp[:, :nb]), f"block-scaled INT8 rows, expert {e}"
        expr = _tokenwise_return_rows_oracle(w, y, rb)
        assert np.array_equal(tokenwise[rows, :w.H + 4], expr[:, :w.H + 4]), \
            f"token-wise INT8 rows, expert {e}"


def test_layer_ffn_small_end_to_end():
    """route -> dispatch -> experts -> combine against the oracle's whole layer."""
    w = FFN_SMALL
    c, (ids, tw, phys), _, weights = _ffn_case(w)
    out = host(c.layer.forward(c.x_d, c.lg_d).view(torch.int16)).view(np.uint16)
    r = oracle.moe_layer(w, c.x, c.lg, c.bias, None, None, c.sp, c.sl, event_id=1, weights=weights)
    assert_close(bf16_to_f32(out), bf16_to_f32(r["out"]), BF16_RTOL, BF16_ATOL, "layer output")


def _int8_return_rows_oracle(w, y_rows, rb):
    q, sblk = oracle.quant_blocks(y_rows, moe.RET_Q8_BLOCK)
    return oracle.int8_return_rows(q, sblk, rb)


def test_expert_int8_returns_and_combine_small():
    """INT8 expert returns (XDS P089): the down projection's INT8 rows (codes and
    one scale per 256 columns, the last block half full at H = 384) are bit-exact
    against the oracle's block quantization of its bf16 returns, the down
    accumulators are unchanged, and the combine of those rows matches the
    oracle's combine of the same rows bit for bit (fp32 and bf16 outputs)."""
    w = FFN_SMALL
    c, (ids, tw, phys), (q, s, lay), (wgu, sgu, wd, sd) = _ffn_case(w)
    n = w.T * w.k
    b = c.layer.buf
    rb = b.sizes.ret_q8_row_bytes
    assert rb == ((w.H + 4 * 2 + 127) // 128) * 128  # codes, two block scales, whole lines
    acc_d = torch.empty((n, w.H), dtype=torch.int32, device="cuda")
    c.layer.experts_gateup()
    c.layer.experts_down_int8ret(acc_d)
    torch.cuda.synchronize()
    got = host(b.ret_q8_rows())
    ad = host(acc_d)
    logical = c.sl[phys.ravel()]
    rr = lay["ret_row"].ravel()
    nb = w.H + 4 * 2
    for e in np.unique(logical):
        sel = np.nonzero(logical == e)[0]
        toks = sel // w.k
        y, _, _, _, o_d = oracle.expert_ffn(q[toks], s[toks], wgu[e], sgu[e], wd[e], sd[e],
                                            want_acc=True)
        assert np.array_equal(ad[rr[sel]], o_d), f"down accumulators, expert {e}"
        exp = _int8_return_rows_oracle(w, y, rb)
        assert np.array_equal(got[rr[sel], :nb], exp[:, :nb]), f"INT8 return rows, expert {e}"
    w32 = host(b.topk_w)
    for odt, obf in ((torch.float32, False), (torch.bfloat16, True)):
        c.layer.out_dtype = odt
        b.out = torch.empty((w.T, w.H), dtype=odt, device="cuda")
        c.layer.combine("q8blocks")
        torch.cuda.synchronize()
        ref = oracle.combine(got, lay["ret_row"], w32, w.k, w.H, "q8blocks", obf,
                             scale_offset=w.H, scale_block=moe.RET_Q8_BLOCK)
        out = host(b.out.view(torch.int16)).view(np.uint16) if obf else host(b.out)
        assert np.array_equal(out, ref), f"combine of INT8 returns ({odt})"


def test_layer_int8_returns_small_end_to_end():
    """route -> dispatch -> experts with INT8 returns -> combine, against the
    oracle's whole path (its bf16 returns quantized per 256-column block and
    combined in the same mode)."""
    w = FFN_SMALL
    c, (ids, tw, phys), (q, s, lay), weights = _ffn_case(w)
    out = host(c.layer.forward(c.x_d, c.lg_d, combine="q8blocks").view(torch.int16)).view(np.uint16)
    r = oracle.moe_layer(w, c.x, c.lg, c.bias, None, None, c.sp, c.sl, event_id=1, weights=weights)
    rb = c.layer.buf.sizes.ret_q8_row_bytes
    rows = _int8_return_rows_oracle(w, r["route_returns"], rb)
    ident = np.arange(w.T * w.k, dtype=np.int32).reshape(w.T, w.k)
    ref = oracle.combine(rows, ident, r["topk_w32"], w.k, w.H, "q8blocks", True,
                         scale_offset=w.H, scale_block=moe.RET_Q8_BLOCK)
    assert_close(bf16_to_f32(out), bf16_to_f32(ref), BF16_RTOL, BF16_ATOL, "layer output")


def _tokenwise_return_rows_oracle(w, y_rows, rb):
    """The token rule over the whole bf16 return row (one scale per row)."""
    q, s = oracle.quant_blocks(y_rows, w.H)
    return oracle.int8_return_rows(q, s, rb)


def test_expert_int8_tokenwise_returns_and_combine_small():
    """Token-wise INT8 expert returns (XDS P085's one scale per token applied to
    P089's quantized outputs): every row bit-exact (H codes and the row scale)
    against the oracle's token rule on its bf16 returns, and the combine of those
    rows bit-exact against the oracle's combine of the same rows (fp32 and bf16)."""
    w = FFN_SMALL
    c, (ids, tw, phys), (q, s, lay), (wgu, sgu, wd, sd) = _ffn_case(w)
    b = c.layer.buf
    rb = b.sizes.ret_q8_row_bytes
    c.layer.experts()
    c.layer.quant_returns()
    torch.cuda.synchronize()
    got = host(b.ret_q8_rows())
    logical = c.sl[phys.ravel()]
    rr = lay["ret_row"].ravel()
    for e in np.unique(logical):
        sel = np.nonzero(logical == e)[0]
        toks = sel // w.k
        y, *_ = oracle.expert_ffn(q[toks], s[toks], wgu[e], sgu[e], wd[e], sd[e])
        exp = _tokenwise_return_rows_oracle(w, y, rb)
        assert np.array_equal(got[rr[sel], :w.H + 4], exp[:, :w.H + 4]), f"rows, expert {e}"
        line_end = min(rb, (w.H + 4 + 127) // 128 * 128)
        assert not got[rr[sel], w.H + 4:line_end].any(), "the rest of the scale's line is zero"
    w32 = host(b.topk_w)
    for odt, obf in ((torch.float32, False), (torch.bfloat16, True)):
        c.layer.out_dtype = odt
        b.out = torch.empty((w.T, w.H), dtype=odt, device="cuda")
        c.layer.combine("q8rows")
        torch.cuda.synchronize()
        ref = oracle.combine(got, lay["ret_row"], w32, w.k, w.H, "q8", obf, scale_offset=w.H)
        out = host(b.out.view(torch.int16)).view(np.uint16) if obf else host(b.out)
        assert np.array_equal(out, ref), f"combine of token-wise INT8 returns ({odt})"


def test_quant_returns_edge_rows():
    """The token rule on hand-made bf16 return rows, bit-exact: an all-zero row
    (s = 0, q = 0), a row of one value repeated, exact halves at s = 1 (round half
    to even), signed zeros, subnormal rows (s below 2^-100: the division path),
    values near the bf16 maximum, and a ragged tail of rows (T*k = 7 rows)."""
    H = 1024
    g = moe.geom(T=7, H=H, E=1, P=1, k=1, D=1, Epp=1, S=1, LB=7)
    rng = np.random.default_rng(41)
    yf = rng.standard_normal((7, H)).astype(np.float32)
    yf[0] = 0.0
    yf[1] = -3.25
    yf[2] = 0.5 + rng.integers(-127, 127, H).astype(np.float32)
    yf[2, :3] = [127.0, 2.5, -2.5]
    yf[3] = np.where(rng.random(H) < 0.5, np.float32(-0.0), yf[3] * np.float32(1e-30))
    yf[4] = rng.integers(-3, 4, H).astype(np.float32) * np.float32(2.0 ** -130)
    yf[5] = rng.uniform(-3e38, 3e38, H).astype(np.float32)
    y = mw.to_bf16_bits(yf)
    sz = moe.moe_plan_sizes(g, 0)
    rb = sz.ret_q8_row_bytes
    out = torch.full((7, rb), 0x5A, dtype=torch.uint8, device="cuda")
    moe.moe_quant_returns_q8(to_dev(y.view(np.int16)), to_dev(np.array([0, 7], np.int32)), g, out)
    torch.cuda.synchronize()
    got = host(out)
    q, sc = oracle.quant_blocks(y, H)
    exp = oracle.int8_return_rows(q, sc, rb)
    assert np.array_equal(got[:, :H + 4], exp[:, :H + 4])
    line_end = min(rb, (H + 4 + 127) // 128 * 128)
    assert line_end > H + 4 and not got[:, H + 4:line_end].any(), \
        "the rest of the scale's 128-byte line is zero"
    assert np.all(got[:, line_end:] == 0x5A), "bytes after that line are left as they were"
    assert sc[0, 0] == 0 and np.all(q[0] == 0) and sc[2, 0] == 1 and q[2, :3].tolist() == [127, 2, -2]


def test_layer_int8_tokenwise_returns_small_end_to_end():
    """route -> dispatch -> experts -> token-wise INT8 returns -> combine, against
    the oracle's whole path (its bf16 returns quantized per row, combined in the
    INT8 mode), within the bf16 tolerance."""
    w = FFN_SMALL
    c, (ids, tw, phys), (q, s, lay), weights = _ffn_case(w)
    out = host(c.layer.forward(c.x_d, c.lg_d, combine="q8rows").view(torch.int16)).view(np.uint16)
    r = oracle.moe_layer(w, c.x, c.lg, c.bias, None, None, c.sp, c.sl, event_id=1, weights=weights)
    rb = c.layer.buf.sizes.ret_q8_row_bytes
    rows = _tokenwise_return_rows_oracle(w, r["route_returns"], rb)
    ident = np.arange(w.T * w.k, dtype=np.int32).reshape(w.T, w.k)
    ref = oracle.combine(rows, ident, r["topk_w32"], w.k, w.H, "q8", True, scale_offset=w.H)
    assert_close(bf16_to_f32(out), bf16_to_f32(ref), BF16_RTOL, BF16_ATOL, "layer output")


@pytest.mark.parametrize("name,n_micro", [("ffn_small", 2), ("ragged", 3)])
def test_microbatch_pipeline_equals_one_batch(name, n_micro):
    """The microbatch pipeline (one microbatch per source partition group,
    scheduled by MoeOverlap on a communication and a compute stream) gives the single-batch layer's output bit for bit, twice
    in a row, and matches the oracle's whole layer within the output tolerance;
    ffn_small runs the INT8 SwiGLU experts, ragged identity experts with the
    INT8 combine."""
    w = FFN_SMALL if name == "ffn_small" else RAGGED
    if w.experts == "swiglu":
        c, _, _, weights = _ffn_case(w)
        mode = "bf16"
    else:
        c = Case(w)
        mode = "q8"
    ref = c.layer.forward(c.x_d, c.lg_d, combine=mode).clone()
    pipe = moe.MoePipeline(c.g, n_micro, w.gating, to_dev(c.sp), to_dev(c.sl), None, None,
                           None if c.bias is None else to_dev(c.bias), c.layer.weights, w.I,
                           c.layer.out_dtype)
    r = oracle.moe_layer(w, c.x, c.lg, c.bias, None, None, c.sp, c.sl, event_id=1,
                         weights=weights if w.experts == "swiglu" else None)
    for _ in range(2):
        out = pipe.forward(c.x_d, c.lg_d, combine=mode)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                           ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref)
        # against the oracle's whole layer (its own routing weights)
        if out.dtype == torch.bfloat16:
            got = bf16_to_f32(host(out.view(torch.int16)).view(np.uint16))
            assert_close(got, bf16_to_f32(r["out"]), BF16_RTOL, BF16_ATOL, "pipeline vs oracle")
        else:
            assert_close(host(out), r["out"], FP32_RTOL, FP32_ATOL, "pipeline vs oracle")


@pytest.mark.parametrize("name,mode,n", [("ffn_small", "bf16", 2), ("ffn_small", "q8blocks", 3),
                                         ("ffn_small", "q8rows", 2), ("ragged", "q8", 3)])
def test_overlap_of_whole_batches_equals_one_at_a_time(name, mode, n):
    """MoeOverlap: n batches in flight on a communication and a compute stream
    (each batch's route, dispatch and combine beside another batch's experts)
    give every batch the output of its own step run alone, bit for bit, on two
    calls in a row; the batches are the workload's tokens rolled by 0, 1, 2 rows."""
    w = FFN_SMALL if name == "ffn_small" else RAGGED
    if w.experts == "swiglu":
        c, _, _, _ = _ffn_case(w)
    else:
        c = Case(w)
    inputs = [(torch.roll(c.x_d, i, 0).contiguous(), torch.roll(c.lg_d, i, 0).contiguous())
              for i in range(n)]

    def bits(t):
        return t.view(torch.int16).clone() if t.dtype == torch.bfloat16 else t.clone()

    refs = [bits(c.layer.forward(x, lg, combine=mode)) for x, lg in inputs]
    torch.cuda.synchronize()
    layers = [moe.MoeLayer(c.g, w.gating, c.layer.slot_partition, c.layer.slot_logical,
                           c.layer.replica_offsets, c.layer.replica_slots, c.layer.bias,
                           c.layer.weights, w.I, c.layer.out_dtype) for _ in range(n)]
    ov = moe.MoeOverlap(layers)
    for call in range(2):
        _log(f"[overlap] {name} {mode} n={n} call {call}")
        outs = ov.forward(inputs, combine=mode)
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(bits(o), r), f"batch {i}, call {call}"


def test_overlap_streaming_submissions_reuse_layers_in_turn():
    """MoeOverlap.submit: seven batches over two layers' buffers, each output copied
    on the caller's stream right after its ticket (before the layer is reused two
    submissions later), equal the steps run alone bit for bit; more batches than
    layers in one forward() are refused."""
    w = FFN_SMALL
    c, _, _, _ = _ffn_case(w)
    inputs = [(torch.roll(c.x_d, 3 * i, 0).contiguous(), torch.roll(c.lg_d, 5 * i, 0).contiguous())
              for i in range(7)]
    refs = [c.layer.forward(x, lg).view(torch.int16).clone() for x, lg in inputs]
    torch.cuda.synchronize()
    layers = [moe.MoeLayer(c.g, w.gating, c.layer.slot_partition, c.layer.slot_logical,
                           bias=c.layer.bias, weights=c.layer.weights, I=w.I) for _ in range(2)]
    ov = moe.MoeOverlap(layers)
    got = []
    pending = []
    for x, lg in inputs:
        pending.append(ov.submit(x, lg))
        if len(pending) == 2:  # the oldest batch's layer is taken by the next submission
            got.append(pending.pop(0).wait().view(torch.int16).clone())
    got += [t.wait().view(torch.int16).clone() for t in pending]
    torch.cuda.synchronize()
    for i, (g_, r) in enumerate(zip(got, refs)):
        assert torch.equal(g_, r), f"batch {i}"
    with pytest.raises(ValueError):
        ov.forward(inputs[:3])
    with pytest.raises(ValueError):  # refused before anything is queued
        ov.submit(inputs[0][0][:-1], inputs[0][1])
    assert torch.equal(ov.submit(*inputs[0]).wait().view(torch.int16), refs[0])


@pytest.mark.parametrize("name,mode", [("ffn_small", "bf16"), ("ffn_small", "q8rows"),
                                       ("ffn_small", "q8blocks"), ("ragged", "q8"),
                                       ("twohop_small", "bf16")])
def test_layer_graph_replay_equals_eager(name, mode):
    """MoeLayer.capture: the whole step captured once as a HIP graph gives the
    eager step's output bit for bit on every replay, with eager steps of another
    input and host synchronizations between the replays, and follows new inputs
    copied into the captured tensors (rows and logits rolled by one token)."""
    w = {"ffn_small": FFN_SMALL, "ragged": RAGGED, "twohop_small": TWOHOP_SMALL}[name]
    if w.experts == "swiglu":
        c, _, _, _ = _ffn_case(w)
    else:
        c = Case(w)
        if w.experts == "synthetic":  # no experts: the combine reads fixed return rows
            gen = torch.Generator(device="cuda").manual_seed(7)
            ret = c.layer.buf.ret
            ret.copy_(torch.randn(ret.shape, generator=gen, device="cuda",
                                  dtype=torch.bfloat16).view(torch.int16))

    def bits(t):
        return t.view(torch.int16).clone() if t.dtype == torch.bfloat16 else t.clone()

    xin, lin = c.x_d.clone(), c.lg_d.clone()
    x2, l2 = torch.roll(xin, 1, 0).contiguous(), torch.roll(lin, 1, 0).contiguous()
    ref1 = bits(c.layer.forward(xin, lin, combine=mode))
    ref2 = bits(c.layer.forward(x2, l2, combine=mode))
    torch.cuda.synchronize()
    assert not torch.equal(ref1, ref2)
    graph = c.layer.capture(xin, lin, combine=mode)
    with pytest.raises(ValueError):
        moe.MoeLayer(c.g, w.gating, c.layer.slot_partition, c.layer.slot_logical,
                     debug_checks=True).capture(xin, lin, combine=mode)
    x1, l1 = xin.clone(), lin.clone()
    for i in range(3):
        _log(f"[graph] {name} {mode} replay {i}")
        out = graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), ref1), f"replay {i}"
        assert torch.equal(bits(c.layer.forward(x2, l2, combine=mode)), ref2), f"eager {i}"
        torch.cuda.synchronize()
        xin.copy_(x2)
        lin.copy_(l2)
        assert torch.equal(bits(graph.replay()), ref2), f"replay {i} of the rolled input"
        xin.copy_(x1)
        lin.copy_(l1)
        torch.cuda.synchronize()


def test_expert_ffn_layer12288_sampled_rows():
    """The headline layer (T=12288, 256 experts, I=2048, Zipf routing), launched as
    the bench launches it: the oracle recomputes 32 rows of each of four slots
    (the hottest, the least loaded non-empty and two random ones) bit for bit, with
    their INT8 returns in both granularities; the whole layer output equals the
    oracle's combine of the GPU's return rows; 64 sampled tokens end to end."""
    w = mw.WORKLOADS["layer12288"]
    c = Case(w)
    ids, tw, phys = _check_route(c)
    c.layer.dispatch(c.x_d)
    q, s = oracle.quant_tokens(c.x, True)
    lay = oracle.dispatch_layout(w, phys, c.sp, 1)
    _log("[layer12288] generating weights")
    wgu, sgu, wd, sd = mw.all_expert_weights(w)
    c.layer.weights = (to_dev(wgu), to_dev(sgu), to_dev(wd), to_dev(sd))
    c.layer.experts()
    torch.cuda.synchronize()
    b = c.layer.buf
    assert np.array_equal(host(b.ret_row), lay["ret_row"])
    ret = host(b.ret.view(torch.int16)).view(np.uint16)
    sc = lay["slot_count"]
    nz = np.nonzero(sc)[0]
    rng = np.random.default_rng(0)
    slots = {int(np.argmax(sc)), int(nz[np.argmin(sc[nz])])} | set(rng.choice(nz, 2).tolist())
    inv = np.argsort(lay["ret_row"].ravel())  # ret row -> route index
    # the layer output: the combine of the GPU's own return rows, every token,
    # bit for bit against the oracle's combine of the same rows and weights
    c.layer.combine("bf16")
    torch.cuda.synchronize()
    out = host(b.out.view(torch.int16)).view(np.uint16)
    w_gpu = host(b.topk_w)
    ref_all = oracle.combine(ret, lay["ret_row"], w_gpu, w.k, w.H, "bf16", True)
    assert np.array_equal(out, ref_all), "combine of the GPU returns, all 12288 tokens"
    # token-wise INT8 returns of the same rows
    c.layer.quant_returns()
    torch.cuda.synchronize()
    q8r = host(b.ret_q8_rows()).copy()
    rb = b.sizes.ret_q8_row_bytes
    c.layer.experts_down_int8ret()  # INT8 returns from the same h (scratch still holds it)
    torch.cuda.synchronize()
    q8 = host(b.ret_q8_rows())
    nb = w.H + 4 * (w.H // moe.RET_Q8_BLOCK)
    for p in sorted(slots):
        o = lay["slot_offset"][p]
        rows = np.arange(o, o + sc[p])
        if len(rows) > 32:
            rows = np.sort(rng.choice(rows, 32, replace=False))
        routes = inv[rows]
        toks = routes // w.k
        e = c.sl[p]
        y, *_ = oracle.expert_ffn(q[toks], s[toks], wgu[e], sgu[e], wd[e], sd[e])
        assert np.array_equal(ret[rows], y), f"slot {p} (expert {e}, {sc[p]} rows)"
        exp = _int8_return_rows_oracle(w, y, rb)
        assert np.array_equal(q8[rows, :nb], exp[:, :nb]), f"INT8 returns, slot {p}"
        expr = _tokenwise_return_rows_oracle(w, y, rb)
        assert np.array_equal(q8r[rows, :w.H + 4], expr[:, :w.H + 4]), f"token-wise rows, slot {p}"
    # end to end on 64 sampled tokens: the oracle recomputes all k expert rows of
    # each (its own routes, quantization and FFN) and combines with its weights
    tsel = np.sort(rng.choice(w.T, 64, replace=False))
    logical = c.sl[phys]
    vals = np.empty((len(tsel) * w.k, w.H), np.uint16)
    for e in np.unique(logical[tsel]):
        ii, jj = np.nonzero(logical[tsel] == e)
        y, *_ = oracle.expert_ffn(q[tsel[ii]], s[tsel[ii]], wgu[e], sgu[e], wd[e], sd[e])
        vals[ii * w.k + jj] = y
    ident = np.arange(len(tsel) * w.k, dtype=np.int32).reshape(len(tsel), w.k)
    ref = oracle.combine(vals, ident, tw[tsel].astype(np.float32), w.k, w.H, "bf16", True)
    assert_close(bf16_to_f32(out[tsel]), bf16_to_f32(ref), BF16_RTOL, BF16_ATOL,
                 "layer output end to end, 64 tokens")


# ------------------------------------------------------------ edge cases ---

def test_empty_batch():
    """T = 0 (every source partition sends nothing): all entry points succeed,
    meta counts and slot counts are zero, the expert histogram is zero."""
    w = mw.WORKLOADS["tiny"].scaled(name="empty", T=0, LB=0)
    c = Case(w)
    c.layer.buf.meta.fill_(-7)
    c.layer.buf.slot_count.fill_(-7)
    c.layer.buf.expert_counts.fill_(-7)
    c.layer.route(c.lg_d)
    c.layer.dispatch(c.x_d)
    c.layer.combine("q8")
    torch.cuda.synchronize()
    b = c.layer.buf
    assert np.all(host(b.meta)[..., 1:3] == 0) and np.all(host(b.slot_count) == 0)
    assert np.all(host(b.slot_offset) == 0) and np.all(host(b.expert_counts) == 0)
    assert b.device_status() == 0


def test_single_token_and_zero_token():
    """One token per source, one of them all-zero: scale 0, codes 0, output 0."""
    w = mw.WORKLOADS["tiny"].scaled(name="one", T=4, LB=1)
    c = Case(w)
    c.x[2] = 0
    c.x_d = dev_bits(c.x, False)
    _, _, phys = _check_route(c)
    q, s, lay = _check_dispatch(c, phys)
    assert s[2] == 0 and np.all(q[2] == 0)
    c.layer.combine("q8")
    assert np.all(host(c.layer.buf.out)[2] == 0)


def test_dispatch_quantization_special_tokens():
    """fp32 tokens at the edges of the token-wise INT8 rule, bit-exact against
    the oracle: subnormal tokens whose scale underflows to 2^-149 so that the
    clamp to +-127 decides the codes (both signs of the amax element), an
    all-zero token, exact halves at scale 1 (round half to even), signed zeros
    with tiny normals, and values near the top of the fp32 range."""
    w = mw.WORKLOADS["tiny"]
    c = Case(w)
    rng = np.random.default_rng(31)
    m = rng.integers(-150, 151, w.H)
    m[0], m[1] = 150, -149
    c.x[0] = m.astype(np.float32) * np.float32(2.0 ** -149)
    c.x[1] = -c.x[0]
    c.x[2] = 0.0
    c.x[3] = 0.5 + rng.integers(-127, 127, w.H).astype(np.float32)
    c.x[3, :3] = [127.0, 2.5, -2.5]
    c.x[4] = np.where(rng.random(w.H) < 0.5, np.float32(-0.0),
                      rng.standard_normal(w.H).astype(np.float32) * np.float32(1e-37))
    c.x[5] = rng.uniform(-3e38, 3e38, w.H).astype(np.float32)
    c.x_d = dev_bits(c.x, False)
    _, _, phys = _check_route(c)
    q, s, _ = _check_dispatch(c, phys)
    assert s[0] == np.float32(2.0 ** -149) and q[0, 0] == 127 and q[1, 0] == -127
    assert s[2] == 0 and np.all(q[2] == 0)
    assert s[3] == 1 and q[3, :3].tolist() == [127, 2, -2]


def _bf16_bits(v) -> np.ndarray:
    """bf16 bit patterns of fp32 values that bf16 represents exactly."""
    b = np.asarray(v, np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "not a bf16 value"
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("T,H", [(300, 384), (1200, 7168)], ids=["per_route", "per_token"])
def test_dispatch_quantization_special_bf16_tokens(T, H):
    """bf16 tokens at the edges of the token-wise INT8 rule, bit-exact against the
    oracle's IEEE quotients, through both scatter shapes (one wavefront per route
    at 300 tokens, one per token at 1200): subnormal rows (scale below 2^-100),
    a row whose scale is exactly 2^-100, the largest finite bf16 amax, exact
    halves at scale 1 (round half to even), signed zeros beside tiny normals, and
    rows of random bit patterns over the whole finite range."""
    w = RAGGED.scaled(name=f"ragged_bf16_{T}x{H}", T=T, H=H, LB=T // 3)
    c = Case(w)
    rng = np.random.default_rng(47)
    x = c.x  # uint16 bf16 bits [T][H]
    sign = lambda n: (rng.integers(0, 2, n).astype(np.uint16) << 15)
    x[0] = rng.integers(0, 0x80, H).astype(np.uint16) | sign(H)  # subnormals
    x[0, 0] = 0x007F
    # |values| <= 127 * 2^-100 (truncated to bf16), the largest one exactly that
    x[1] = ((rng.uniform(-1, 1, H) * (127.0 * 2.0 ** -100)).astype(np.float32)
            .view(np.uint32) >> 16).astype(np.uint16)
    x[1, 0] = _bf16_bits([127.0 * 2.0 ** -100])[0]
    x[2] = rng.integers(0, 0x7F80, H).astype(np.uint16) | sign(H)  # every finite magnitude
    x[2, 0] = 0x7F7F
    x[3] = _bf16_bits(rng.integers(-127, 127, H).astype(np.float32) + np.float32(0.5))
    x[3, :4] = _bf16_bits([127.0, 2.5, -2.5, 0.5])
    x[4] = np.where(rng.random(H) < 0.5, np.uint16(0x8000),
                    rng.integers(0x0080, 0x0200, H).astype(np.uint16) | sign(H))
    for r in range(5, 12):
        x[r] = rng.integers(0, 0x7F80, H).astype(np.uint16) | sign(H)
    c.x_d = dev_bits(x, True)
    _, _, phys = _check_route(c)
    q, s, _ = _check_dispatch(c, phys)
    f32 = lambda b: (np.asarray(b, np.uint32) << 16).view(np.float32)
    assert s[0] < np.float32(2.0 ** -100) and s[1] == np.float32(2.0 ** -100)
    assert s[2] == f32(0x7F7F) / np.float32(127)
    assert s[3] == 1 and q[3, :4].tolist() == [127, 2, -2, 0]


def test_invalid_routes_are_flagged_not_written():
    """Out-of-range physical ids are dropped (row indices -1) and reported in the
    device status word; nothing is written out of bounds."""
    c = Case(RAGGED)
    c.layer.route(c.lg_d)
    b = c.layer.buf
    b.phys[5, 3] = 10_000
    b.phys[7, 0] = -3
    c.layer.dispatch(c.x_d)
    torch.cuda.synchronize()
    assert b.device_status() & moe.MOE_DEVICE_BAD_ROUTE
    dr = host(b.disp_row)
    assert dr[5, 3] == -1 and dr[7, 0] == -1
    assert int(host(b.meta)[..., 2].sum()) == c.w.T * c.w.k - 2


def _layout_by_definition(w, phys, sp, event_id):
    """The dispatch layout written out from its definition (valid routes only,
    route order t k + j): a route's row in region (d, s) is the number of valid
    routes before it there (-1 from cap on), its slot row the slot's offset plus
    the number of valid routes before it to that slot; the status bits flag
    invalid slots, invalid partitions and full regions."""
    T, k, P, D, S, LB = w.T, w.k, w.P, w.D, w.S, w.LB
    cap = LB * min(k, w.Epp)
    ph = phys.reshape(-1)
    n = T * k
    valid = np.zeros(n, bool)
    d = np.full(n, -1)
    bits = 0
    for g in range(n):
        p = int(ph[g])
        if not 0 <= p < P:
            bits |= moe.MOE_DEVICE_BAD_ROUTE
        elif not 0 <= int(sp[p]) < D:
            bits |= moe.MOE_DEVICE_BAD_PARTITION
        else:
            valid[g], d[g] = True, int(sp[p])
    src = np.arange(n) // k // LB
    count_ds = np.zeros((D, S), np.int64)
    count_p = np.zeros(P, np.int64)
    rank_d = np.zeros(n, np.int64)
    rank_p = np.zeros(n, np.int64)
    for g in np.nonzero(valid)[0]:
        rank_d[g] = count_ds[d[g], src[g]]
        rank_p[g] = count_p[ph[g]]
        count_ds[d[g], src[g]] += 1
        count_p[ph[g]] += 1
    if (count_ds > cap).any():
        bits |= moe.MOE_DEVICE_OVER_CAPACITY
    slot_offset = np.concatenate([[0], np.cumsum(count_p)]).astype(np.int32)
    disp_row = np.full(n, -1, np.int32)
    ret_row = np.full(n, -1, np.int32)
    slot_rows = np.full(n, -7, np.int32)  # rows no valid route owns are not checked
    for g in np.nonzero(valid)[0]:
        r = slot_offset[ph[g]] + rank_p[g]
        dr = (d[g] * S + src[g]) * cap + rank_d[g] if rank_d[g] < cap else -1
        disp_row[g], ret_row[g], slot_rows[r] = dr, r, dr
    meta_off = np.concatenate([np.zeros((D, 1), np.int64), np.cumsum(count_ds, 1)[:, :-1]], 1)
    return dict(bits=bits, disp_row=disp_row.reshape(T, k), ret_row=ret_row.reshape(T, k),
                slot_rows=slot_rows, slot_count=count_p.astype(np.int32), slot_offset=slot_offset,
                meta_off=meta_off, meta_count=count_ds)


@pytest.mark.parametrize("name", ["smallb", "ragged"])
def test_dispatch_layout_with_bad_routes_and_a_full_region(name):
    """Both dispatch paths (smallb: the one-launch path; ragged: count / scan /
    scatter) against the layout's definition when the routes are not clean:
    out-of-range slot ids, a slot whose partition is out of range, and one
    source sending every route to partition 0 so that region (0, 0) overflows;
    status bits, row indices, slot counts and offsets, and meta are compared."""
    w = SMALLB if name == "smallb" else RAGGED
    c = Case(w)
    c.layer.route(c.lg_d)
    b = c.layer.buf
    sp = c.sp.copy()
    bad_slot = w.P - 1
    sp[bad_slot] = w.D + 5
    c.layer.slot_partition.copy_(to_dev(sp))
    phys = host(b.phys).copy()
    phys[:w.LB] = np.arange(w.k)[None, :] % w.Epp  # source 0: every route to partition 0
    phys[w.LB + 2, 3] = 10_000
    phys[w.LB + 3, 0] = -3
    phys[w.LB + 4, 1] = bad_slot
    b.phys.copy_(to_dev(phys.astype(np.int32)))
    c.layer.event_id = 76  # the layer advances it: this dispatch carries 77
    c.layer.dispatch(c.x_d)
    torch.cuda.synchronize()
    ref = _layout_by_definition(w, phys, sp, 77)
    assert b.device_status() == ref["bits"] == (moe.MOE_DEVICE_BAD_ROUTE | moe.MOE_DEVICE_BAD_PARTITION
                                                | moe.MOE_DEVICE_OVER_CAPACITY)
    assert np.array_equal(host(b.disp_row), ref["disp_row"]), "disp_row"
    assert np.array_equal(host(b.ret_row), ref["ret_row"]), "ret_row"
    sr = host(b.slot_rows)
    own = ref["slot_rows"] != -7
    assert np.array_equal(sr[own], ref["slot_rows"][own]), "slot_rows"
    assert np.array_equal(host(b.slot_count), ref["slot_count"])
    assert np.array_equal(host(b.slot_offset), ref["slot_offset"])
    meta = host(b.meta)
    assert np.all(meta[..., 0].view(np.uint32) == 77)
    assert np.array_equal(meta[..., 1], ref["meta_off"]) and np.array_equal(meta[..., 2], ref["meta_count"])


def test_all_tokens_to_one_partition():
    """Every route of every token lands on partition 0 (its Epp slots): regions
    fill to exactly cap rows."""
    w = RAGGED.scaled(name="hot", D=10, Epp=4)
    c = Case(w)
    lg = np.full((w.T, w.E), -5.0, np.float32)
    lg[:, :w.k] = np.linspace(3, 1, w.k)  # experts 0..k-1 win everywhere
    c.lg = mw.to_bf16_bits(lg)
    c.lg_d = dev_bits(c.lg, True)
    c.bias = None
    c.layer.bias = None
    # slots 0..3 on partition 0, 4..7 on partition 1 -> cap = LB * min(k, Epp) = 400 per region
    _, _, phys = _check_route(c)
    q, s, lay = _check_dispatch(c, phys)
    assert lay["meta"][0, :, 2].max() == w.LB * min(w.k, w.Epp)


def test_layer_refuses_mismatched_tensors():
    """The C ABI sees only pointers; the layer refuses tensors whose shape, dtype
    or placement would make a kernel read out of bounds, before any launch."""
    w = mw.WORKLOADS["tiny"]
    g = moe.geom_of(w)
    ro, rs, sp, sl = mw.identity_map(w)
    sp_d, sl_d = to_dev(sp), to_dev(sl)
    with pytest.raises(ValueError):
        moe.MoeLayer(g, w.gating, sp_d[:-1].contiguous(), sl_d)            # P - 1 slots
    with pytest.raises(ValueError):
        moe.MoeLayer(g, w.gating, sp_d, sl_d.to(torch.int64))               # wrong dtype
    with pytest.raises(ValueError):
        moe.MoeLayer(g, w.gating, sp_d, sl_d, bias=torch.zeros(w.E + 1, device="cuda"))
    with pytest.raises(ValueError):
        moe.MoeLayer(g, "relu", sp_d, sl_d)
    layer = moe.MoeLayer(g, w.gating, sp_d, sl_d)
    with pytest.raises(ValueError):
        layer.route(torch.zeros((w.T, w.E - 1), device="cuda"))             # [T][E-1] logits
    with pytest.raises(ValueError):
        layer.dispatch(torch.zeros((w.T, w.H), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        layer.route(torch.zeros((w.E, w.T), device="cuda").t())             # not contiguous
    # expert weights: scales of the wrong shape, and weights for another I
    E, H, I = 2, 128, 64
    wgu = torch.zeros((E, 2 * I, H), dtype=torch.int8, device="cuda")
    wd = torch.zeros((E, H, I), dtype=torch.int8, device="cuda")
    sgu, sd = torch.ones((E, 2 * I), device="cuda"), torch.ones((E, H), device="cuda")
    with pytest.raises(ValueError):
        moe.PackedExpertWeights(wgu, sgu[:, :I].contiguous(), wd, sd)
    packed = moe.PackedExpertWeights(wgu, sgu, wd, sd)
    g2 = moe.geom(T=8, H=H, E=E, P=E, k=1, D=1, Epp=E, S=1, LB=8)
    eye = torch.arange(E, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        moe.MoeLayer(g2, "sigmoid", torch.zeros(E, dtype=torch.int32, device="cuda"), eye,
                     weights=packed, I=2 * I)
    moe.MoeLayer(g2, "sigmoid", torch.zeros(E, dtype=torch.int32, device="cuda"), eye,
                 weights=packed, I=I)


def test_expert_gemm_slot_size_boundaries():
    """The grouped GEMMs called directly, one launch over slots of 0, 1, 31, 32, 33,
    127, 128, 129, 255, 256, 257 and 1025 rows (the edges of the 32-row MFMA blocks
    and the 128-row m-tiles; 1025 rows make a full group of eight m-tiles and a
    lone ninth, whose weights load non-temporal), rows gathered from a shuffled
    dispatch buffer, slots
    mapped to logical experts out of order, a half-full gate/up n-tile (I = 192)
    and a half-full down n-tile (H = 384): both projections' int32 accumulators
    and the bf16 return rows bit-exact against the oracle, slot by slot."""
    counts = np.array([0, 1, 31, 32, 33, 127, 128, 129, 255, 256, 257, 1025], np.int32)
    P = E = len(counts)
    H, I = 384, 192
    R = int(counts.sum())
    g = moe.geom(T=R, H=H, E=E, P=P, k=1, D=1, Epp=P, S=1, LB=R)
    sz = moe.moe_plan_sizes(g, I)
    rng = np.random.default_rng(23)
    msg = np.zeros((R, sz.msg_bytes), np.uint8)
    q = rng.integers(-127, 128, (R, H), dtype=np.int8)
    s = (rng.random(R, dtype=np.float32) * np.float32(0.05) + np.float32(1e-3)).astype(np.float32)
    msg[:, :H] = q.view(np.uint8)
    msg[:, H:H + 4] = s.view(np.uint8).reshape(R, 4)
    slot_rows = rng.permutation(R).astype(np.int32)        # dense row i -> dispatch row
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    logical = np.array([(7 * p + 3) % E for p in range(P)], np.int32)
    wgu = rng.integers(-127, 128, (E, 2 * I, H), dtype=np.int8)
    wd = rng.integers(-127, 128, (E, H, I), dtype=np.int8)
    sgu = (rng.random((E, 2 * I), dtype=np.float32) * np.float32(2e-3)).astype(np.float32)
    sd = (rng.random((E, H), dtype=np.float32) * np.float32(2e-3)).astype(np.float32)
    packed = moe.PackedExpertWeights(to_dev(wgu), to_dev(sgu), to_dev(wd), to_dev(sd))
    ret = torch.empty((R, H), dtype=torch.int16, device="cuda")
    acc_gu = torch.empty((R, 2 * I), dtype=torch.int32, device="cuda")
    acc_d = torch.empty((R, H), dtype=torch.int32, device="cuda")
    scratch = torch.empty(sz.ffn_scratch_bytes, dtype=torch.uint8, device="cuda")
    _log(f"[case] slot boundaries R={R} P={P} H={H} I={I}")
    moe.moe_expert_ffn_q8(to_dev(msg), to_dev(counts), to_dev(offsets), to_dev(slot_rows),
                          to_dev(logical), packed.w_gateup, packed.s_gateup, packed.w_down,
                          packed.s_down, I, g, ret, acc_gu, acc_d, scratch)
    torch.cuda.synchronize()
    y_all, agu, ad = host(ret).view(np.uint16), host(acc_gu), host(acc_d)
    for p in range(P):
        if counts[p] == 0:
            continue
        rows = np.arange(offsets[p], offsets[p + 1])
        src = slot_rows[rows]
        e = logical[p]
        y, hq, hs, o_gu, o_d = oracle.expert_ffn(q[src], s[src], wgu[e], sgu[e], wd[e], sd[e],
                                                 want_acc=True)
        assert np.array_equal(agu[rows], o_gu), f"gate/up accumulators, slot of {counts[p]} rows"
        assert np.array_equal(ad[rows], o_d), f"down accumulators, slot of {counts[p]} rows"
        assert np.array_equal(y_all[rows], y), f"return rows, slot of {counts[p]} rows"
