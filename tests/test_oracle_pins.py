"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what it pins: a worked example or printed value of the pages
(tests/golden/), a closed form, a library routine (torch / numpy), brute force
on tiny inputs, or an invariant the pages state.  Pages:
XDS = "xDeepServe on CloudMatrix384", CMI = "CloudMatrix384 LLM Serving".
"""
import json
import os
import struct

import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------- c0' gate logits ---

def test_router_logits_exact_on_integers_and_library_on_floats():
    """Gate logits: with small-integer bf16 inputs every dot product is an exact
    integer (int64 matmul); with N(0,1) inputs they equal a float64 library
    matmul of the decoded values to double rounding."""
    rng = np.random.default_rng(31)
    T, E, H = 24, 12, 352
    xi = rng.integers(-8, 9, (T, H))
    wi = rng.integers(-8, 9, (E, H))
    xb = mw.to_bf16_bits(xi.astype(np.float32))
    wb = mw.to_bf16_bits(wi.astype(np.float32))
    got = oracle.router_logits(xb, wb)
    assert np.array_equal(got, (xi @ wi.T).astype(np.float64))
    xb = mw.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = mw.to_bf16_bits((rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32))
    got = oracle.router_logits(xb, wb)
    ref = _bf16_to_f32(xb).astype(np.float64) @ _bf16_to_f32(wb).astype(np.float64).T
    mag = np.abs(_bf16_to_f32(xb)).astype(np.float64) @ np.abs(_bf16_to_f32(wb)).astype(np.float64).T
    assert np.all(np.abs(got - ref) <= 1e-13 * mag)


# ------------------------------------------------------------- c1 top-k ---

@pytest.mark.parametrize("E,k,gating,bf16", [(8, 2, "softmax", False), (16, 5, "sigmoid", True),
                                             (64, 8, "sigmoid", True), (7, 7, "softmax", False)])
def test_topk_bruteforce_sort(E, k, gating, bf16):
    """Brute force: a full stable sort by (score desc, id asc) of every token's
    scores (numpy lexsort) picks the same ids in the same order."""
    rng = np.random.default_rng(E * 100 + k)
    T = 200
    v = rng.standard_normal((T, E)).astype(np.float32)
    if bf16:
        # coarse values make exact ties frequent
        v = np.round(v * 4) / 4
        lg = mw.to_bf16_bits(v)
        vf = _bf16_to_f32(lg)
    else:
        lg = v
        vf = v
    bias = rng.standard_normal(E).astype(np.float32) if gating == "sigmoid" else None
    ids, sc, w = oracle.route_topk(lg, k, gating, bias, logits_bf16=bf16)
    score = vf + (bias if bias is not None else np.float32(0))
    assert score.dtype == np.float32
    for t in range(T):
        order = np.lexsort((np.arange(E), -score[t].astype(np.float64)))
        assert list(ids[t]) == list(order[:k])
        assert np.array_equal(sc[t], score[t][order[:k]])
    assert np.all(np.diff(w, axis=1) <= 1e-15), "weights must not increase with the route slot"
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)


def test_topk_softmax_full_equals_library_softmax():
    """k = E with softmax: the weights are torch.softmax of the scores (reordered)."""
    rng = np.random.default_rng(1)
    T, E = 64, 8
    v = rng.standard_normal((T, E)).astype(np.float32)
    ids, _, w = oracle.route_topk(v, E, "softmax")
    ref = torch.softmax(torch.from_numpy(v).double(), dim=1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids.astype(np.int64), 1), rtol=1e-13, atol=1e-15)


def test_topk_weight_ratios_match_library_activations():
    """Pairwise ratios w_i / w_j equal the activation ratios, using torch.sigmoid /
    torch.exp; a dropped bias or a wrong sign inside exp fails this."""
    rng = np.random.default_rng(2)
    T, E, k = 50, 32, 6
    v = rng.standard_normal((T, E)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    ids, sc, w = oracle.route_topk(v, k, "sigmoid", b)
    s = torch.from_numpy(sc).double()
    sig = torch.sigmoid(s).numpy()
    np.testing.assert_allclose(w / w[:, :1], sig / sig[:, :1], rtol=1e-13)
    ids2, sc2, w2 = oracle.route_topk(v, k, "softmax", b)
    ex = torch.exp(torch.from_numpy(sc2).double() - torch.from_numpy(sc2[:, :1]).double()).numpy()
    np.testing.assert_allclose(w2 / w2[:, :1], ex, rtol=1e-13)


def test_topk_tie_break_lowest_id():
    """Equal scores: the lower expert id is chosen first (the reading the oracle takes)."""
    lg = np.array([[0.5, 2.0, 2.0, -1.0, 2.0]], np.float32)
    ids, _, w = oracle.route_topk(lg, 3, "softmax")
    assert list(ids[0]) == [1, 2, 4]
    np.testing.assert_allclose(w[0], [1 / 3] * 3, rtol=1e-15)
    # negative zero and positive zero tie as equal values
    lg = np.array([[-0.0, 0.0, -1.0]], np.float32)
    ids, _, _ = oracle.route_topk(lg, 1, "softmax")
    assert ids[0, 0] == 0


# --------------------------------------------------------- c2 EPLB gather ---

def test_eplb_fig12_rotation():
    """XDS P079 / Fig. 12 worked example (golden): expert 1 with copies in slots
    {1, 2} rotates 1, 2, 1, 2 over the 4 token positions of a step."""
    g = _golden("eplb_fig12_rotation.json")
    E, T = g["logical_experts"], g["tokens_per_step"]
    # replica lists: expert 1 -> [1, 2]; every other expert e -> one slot of its own
    slots, offs = [], [0]
    nxt = 3
    for e in range(E):
        if e == g["expert"]:
            slots += g["replica_slots_ascending"]
        else:
            slots.append(nxt if e not in (1, 2) else 0)
            nxt += 1
        offs.append(len(slots))
    ids = np.full((T, 1), g["expert"], np.int32)
    phys = oracle.eplb_phys(ids, LB=T, E=E, replica_offsets=np.array(offs, np.int32),
                            replica_slots=np.array(slots, np.int32))
    assert list(phys[:, 0]) == g["expected_column"]


def test_eplb_rotation_counts_bruteforce():
    """Per-replica counts equal #{b : e in topk(b), b mod |R_e| = r} (brute force),
    positions are local to each source partition, and when every position picks e
    the replica loads differ by at most one (XDS P079)."""
    rng = np.random.default_rng(3)
    E, k, S, LB = 12, 3, 3, 37
    T = S * LB
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[:, 0] = 5  # every position selects expert 5
    nrep = rng.integers(1, 4, E)
    offs = np.concatenate([[0], np.cumsum(nrep)]).astype(np.int32)
    slots = rng.permutation(int(offs[-1])).astype(np.int32)
    for e in range(E):
        slots[offs[e]:offs[e + 1]].sort()
    phys = oracle.eplb_phys(ids, LB, E, offs, slots)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            r = (t % LB) % nrep[e]
            assert phys[t, j] == slots[offs[e] + r]
    cnt = np.bincount(phys[:, 0], minlength=int(offs[-1]))
    loads = cnt[slots[offs[5]:offs[6]]]
    assert loads.max() - loads.min() <= S  # at most one per source partition
    assert oracle.eplb_phys(ids, LB, E).tolist() == ids.tolist()


# ------------------------------------------------------- c3 quantization ---

def test_quant_half_even_closed_form():
    """amax = 127 makes s = 1 exactly, so q = round-half-even(x): values on .5
    go to the even neighbour; the amax element maps to 127."""
    x = np.zeros((1, 16), np.float32)
    x[0, :8] = [127, 0.5, 1.5, 2.5, -0.5, -2.5, 3.49, -126.5]
    q, s = oracle.quant_tokens(x, False)
    assert s[0] == np.float32(1.0)
    assert list(q[0, :8]) == [127, 0, 2, 2, 0, -2, 3, -126]


def test_quant_matches_library_rounding_and_bounds():
    """torch.round (half to even) of x / s with s = amax / 127 in fp32 gives the
    same codes; |x - q s| <= s (0.5 + 2^-16); the amax element maps to +-127;
    an all-zero token gives s = 0, q = 0; bf16 input decodes exactly.
    Rows 8 and 9 are subnormal tokens (integers m times 2^-149, |m| <= 150):
    s = fl(amax / 127) rounds to 2^-149, x / s = m, and the clamp is what keeps
    the codes in [-127, 127] (the amax element still maps to +-127; the
    half-step error bound does not hold there and is checked on the other rows)."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 256)).astype(np.float32) * rng.uniform(1e-3, 1e3, (64, 1)).astype(np.float32)
    x[7] = 0.0
    m = rng.integers(-150, 151, 256)
    m[0], m[1] = 150, -150
    x[8] = m.astype(np.float32) * np.float32(2.0 ** -149)
    x[9] = -x[8]
    xb = mw.to_bf16_bits(x)
    for arr, is_bf16, xf in ((x, False, x), (xb, True, _bf16_to_f32(xb))):
        q, s = oracle.quant_tokens(arr, is_bf16)
        xt = torch.from_numpy(xf)
        amax = xt.abs().amax(1)
        st = amax / torch.tensor(127.0, dtype=torch.float32)
        assert np.array_equal(st.numpy(), s)
        nz = st > 0
        ref = torch.zeros_like(xt)
        ref[nz] = torch.round(xt[nz] / st[nz, None]).clamp(-127, 127)
        assert np.array_equal(ref.numpy().astype(np.int8), q)
        assert np.all(q[7] == 0) and s[7] == 0
        i = np.abs(xf).argmax(1)
        rows = np.arange(64)[nz.numpy()]
        assert np.all(np.abs(q[rows, i[rows]]) == 127)
        assert q.min() >= -127
        if not is_bf16:  # bf16 cannot hold the subnormal rows (they round to zero tokens)
            assert s[8] == np.float32(2.0 ** -149) and q[8].tolist() == np.clip(m, -127, 127).tolist()
            assert q[9].tolist() == np.clip(-m, -127, 127).tolist()
        normal = np.setdiff1d(np.arange(64), [8, 9])
        err = np.abs(xf[normal].astype(np.float64) - q[normal].astype(np.float64) * s[normal, None])
        assert np.all(err <= s[normal, None].astype(np.float64) * (0.5 + 2.0 ** -16))


# ---------------------------------------------------- c4 dispatch layout ---

def _small_workload(**kw):
    base = dict(name="t", T=6 * 40, H=32, E=24, P=24, k=4, D=6, Epp=4, S=6, LB=40,
                gating="sigmoid", logits_dtype="f32", x_dtype="f32", zipf=False,
                experts="identity", combine="q8", out_dtype="f32")
    base.update(kw)
    return mw.Workload(**base)


def _layout_case(w, rng):
    phys = np.stack([rng.choice(w.P, w.k, replace=False) for _ in range(w.T)]).astype(np.int32)
    sp = rng.permutation(np.arange(w.P) // w.Epp).astype(np.int32)
    return phys, sp


@pytest.mark.parametrize("S,LB,D,Epp,k", [(6, 40, 6, 4, 4), (1, 100, 24, 1, 3), (4, 4, 4, 2, 2)])
def test_dispatch_layout_library_pins(S, LB, D, Epp, k):
    """Layout against numpy's stable argsort and bincount/cumsum: the rank of a
    route in its (d, s) region and in its slot is its position in a stable sort
    by that key over routes in (t, j) order; counts are bincounts; offsets are
    exclusive cumulative sums; slot_rows[ret_row] = disp_row; capacity holds."""
    w = _small_workload(T=S * LB, S=S, LB=LB, D=D, Epp=Epp, P=D * Epp, E=D * Epp, k=k)
    rng = np.random.default_rng(S * 1000 + LB)
    phys, sp = _layout_case(w, rng)
    out = oracle.dispatch_layout(w, phys, sp, event_id=0xABCD1234)
    f = phys.ravel()
    d = sp[f]
    s = np.repeat(np.arange(w.T) // w.LB, w.k)
    region = d * w.S + s
    nreg = w.D * w.S
    cnt = np.bincount(region, minlength=nreg)
    start = np.concatenate([[0], np.cumsum(cnt)[:-1]])
    pos = np.empty_like(region)
    pos[np.argsort(region, kind="stable")] = np.arange(len(region))
    r = pos - start[region]
    assert np.all(r < w.cap)
    assert np.array_equal(out["disp_row"].ravel(), region * w.cap + r)
    m = out["meta"]
    assert np.all(m[..., 0] == np.int32(np.uint32(0xABCD1234).view(np.int32)))
    assert np.array_equal(m[..., 2].ravel(), cnt)
    c2 = cnt.reshape(w.D, w.S)
    assert np.array_equal(m[..., 1], np.cumsum(c2, axis=1) - c2)
    sc = np.bincount(f, minlength=w.P)
    assert np.array_equal(out["slot_count"], sc)
    assert np.array_equal(out["slot_offset"], np.concatenate([[0], np.cumsum(sc)]))
    rpos = np.empty_like(f)
    rpos[np.argsort(f, kind="stable")] = np.arange(len(f))
    assert np.array_equal(out["ret_row"].ravel(), rpos)
    assert np.array_equal(out["slot_rows"][out["ret_row"].ravel()], out["disp_row"].ravel())
    # every (t, j) exactly once, sum of counts = T k
    assert len(np.unique(out["disp_row"])) == w.T * w.k and m[..., 2].sum() == w.T * w.k
    # slot_local: index of p among its partition's slots, ascending p
    for p in range(w.P):
        assert out["slot_local"][p] == np.sum(sp[:p] == sp[p])


def test_dispatch_capacity_error():
    """A partition with more slots than declared can receive more than
    cap = LB min(k, Epp) routes from one source: the oracle reports capacity
    from the first route past cap (cap + 1 routes fail, cap routes fit)."""
    w = _small_workload(T=8, S=1, LB=8, D=2, Epp=1, P=4, E=4, k=2)
    sp = np.array([0, 0, 1, 1], np.int32)  # two slots on partition 0 but Epp = 1
    # cap = 8: every token's first route goes to partition 0; token 5's second too
    phys = np.tile(np.array([0, 2], np.int32), (8, 1))
    assert oracle.dispatch_layout(w, phys, sp, 1)["meta"][0, 0, 2] == 8
    phys[5, 1] = 1
    with pytest.raises(oracle.OracleError) as ei:
        oracle.dispatch_layout(w, phys, sp, 1)
    assert ei.value.rc == -3


def test_dispatch_rows_trailer_roundtrip():
    """Every message carries its token's codes and a trailer that decodes back
    to (scale, source partition, batch slot, route slot, local slot, event)."""
    w = _small_workload()
    rng = np.random.default_rng(5)
    phys, sp = _layout_case(w, rng)
    x = rng.standard_normal((w.T, w.H)).astype(np.float32)
    q, s = oracle.quant_tokens(x, False)
    lay = oracle.dispatch_layout(w, phys, sp, 0x12345)
    rows = oracle.dispatch_rows(w, q, s, phys, lay["slot_local"], 0x12345)
    part = oracle.dispatch_rows(w, q, s, phys, lay["slot_local"], 0x12345, t0=37, t1=101)
    assert np.array_equal(part, rows[37 * w.k:101 * w.k])
    for t in range(0, w.T, 7):
        for j in range(w.k):
            row = rows[t * w.k + j]
            assert np.array_equal(row[:w.H].view(np.int8), q[t])
            sc, src, b, rj, loc, ev = struct.unpack("<fiiBBH", row[w.H:w.H + 16].tobytes())
            assert (sc, src, b, rj) == (s[t], t // w.LB, t % w.LB, j)
            assert loc == lay["slot_local"][phys[t, j]] and ev == 0x2345


# -------------------------------------------------------- c5/c6 experts ---

def _expert_case(n, H, I, seed):
    w = mw.Workload("e", T=n, H=H, E=1, P=1, k=1, D=1, Epp=1, S=1, LB=n, gating="sigmoid",
                    logits_dtype="f32", x_dtype="f32", zipf=False, experts="swiglu",
                    combine="bf16", out_dtype="bf16", I=I, seed=seed)
    wgu, sgu, wd, sd = mw.expert_weights(w, 0)
    x = np.random.default_rng(seed).standard_normal((n, H)).astype(np.float32)
    q, s = oracle.quant_tokens(x, False)
    return q, s, wgu, sgu, wd, sd


def test_expert_accumulators_equal_float64_matmul():
    """int32 accumulators equal an fp64 matmul of the int8 operands (exact: every
    partial sum is an integer far below 2^53); gate rows are 0..I-1, up rows I..2I-1."""
    q, s, wgu, sgu, wd, sd = _expert_case(9, 256, 96, 6)
    y, hq, hs, acc_gu, acc_d = oracle.expert_ffn(q, s, wgu, sgu, wd, sd, want_acc=True)
    ref = q.astype(np.float64) @ wgu.astype(np.float64).T
    assert np.array_equal(acc_gu.astype(np.float64), ref)
    refd = hq.astype(np.float64) @ wd.astype(np.float64).T
    assert np.array_equal(acc_d.astype(np.float64), refd)


def test_expert_swiglu_against_float64_library_model():
    """The whole expert against torch in float64 (library SiLU): gate/up not
    swapped, scales applied once each, requant codes within one step of the
    float64 codes and y within bf16 precision of the float64 output."""
    n, H, I = 12, 384, 128
    q, s, wgu, sgu, wd, sd = _expert_case(n, H, I, 7)
    y, hq, hs, _, _ = oracle.expert_ffn(q, s, wgu, sgu, wd, sd)
    qt = torch.from_numpy(q).double()
    gu = (qt @ torch.from_numpy(wgu).double().T) * torch.from_numpy(s).double()[:, None] \
        * torch.from_numpy(sgu).double()[None]
    h = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
    hs_ref = h.abs().amax(1) / 127
    np.testing.assert_allclose(hs, hs_ref.numpy(), rtol=1e-6)
    hq_ref = torch.round(h / hs_ref[:, None]).numpy()
    assert np.max(np.abs(hq.astype(np.float64) - hq_ref)) <= 1
    yd = (torch.from_numpy(hq).double() @ torch.from_numpy(wd).double().T) \
        * torch.from_numpy(hs).double()[:, None] * torch.from_numpy(sd).double()[None]
    np.testing.assert_allclose(_bf16_to_f32(y), yd.numpy(), rtol=2 ** -8, atol=1e-30)
    # and the full float64 chain (no intermediate requant) agrees to INT8 precision
    yfull = (h @ torch.from_numpy(wd).double().T) * torch.from_numpy(sd).double()[None]
    rel = np.linalg.norm(_bf16_to_f32(y) - yfull.numpy()) / np.linalg.norm(yfull.numpy())
    assert rel < 0.02


def test_expert_zero_rows():
    """A zero token gives acc = 0, h = 0, hs = 0, hq = 0 and y = 0."""
    q, s, wgu, sgu, wd, sd = _expert_case(3, 64, 32, 8)
    q[1] = 0
    s[1] = 0
    y, hq, hs, _, _ = oracle.expert_ffn(q, s, wgu, sgu, wd, sd)
    assert hs[1] == 0 and np.all(hq[1] == 0) and np.all(y[1] == 0)


# ------------------------------------------------------------- c7 combine ---

def test_combine_identity_experts_closed_form():
    """Identity experts: out = (sum_j w_j) q s, and with weights summing to 1 the
    output reproduces x to within half a quantization step (plus fp32 rounding)."""
    w = _small_workload(T=4 * 30, S=4, LB=30, D=4, Epp=3, P=12, E=12, k=3)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((w.T, w.H)).astype(np.float32)
    logits = rng.standard_normal((w.T, w.E)).astype(np.float32)
    ro, rs, sp, sl = mw.identity_map(w)
    r = oracle.moe_layer(w, x, logits, None, None, None, sp, sl, event_id=3)
    out = r["out"]
    s = r["scale"][:, None].astype(np.float64)
    assert np.all(np.abs(out - x) <= s * 0.5 + 1e-5 * np.abs(x) + 1e-7)
    deq = r["q"].astype(np.float64) * s
    np.testing.assert_allclose(out, deq * r["topk_w32"].astype(np.float64).sum(1, keepdims=True),
                               rtol=2e-6, atol=1e-9)


def test_combine_against_float64_einsum_and_unit_weight():
    """bf16 returns: fp32 accumulation agrees with a float64 einsum to fp32
    rounding; k = 1 with weight 1 returns the row exactly; bf16 output rounds
    the fp32 result to nearest even."""
    rng = np.random.default_rng(10)
    T, k, H = 40, 8, 96
    vals = mw.to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    wts = rng.uniform(0, 1, (T, k)).astype(np.float32)
    rr = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    out = oracle.combine(vals, rr, wts, k, H, "bf16", False)
    v = _bf16_to_f32(vals).astype(np.float64)[rr]
    ref = np.einsum("tj,tjc->tc", wts.astype(np.float64), v)
    bound = 8 * 2.0 ** -24 * np.einsum("tj,tjc->tc", wts.astype(np.float64), np.abs(v))
    assert np.all(np.abs(out - ref) <= bound + 1e-30)
    outb = oracle.combine(vals, rr, wts, k, H, "bf16", True)
    assert np.array_equal(outb, mw.to_bf16_bits(out))
    one = oracle.combine(vals, rr[:, :1], np.ones((T, 1), np.float32), 1, H, "bf16", False)
    assert np.array_equal(one, _bf16_to_f32(vals)[rr[:, 0]])


# ----------------------------------------- c6' INT8 returns (block scales) ---

def test_combine_bf16_output_equals_library_rounding():
    """k = 1, weight 1: the bf16 output is the fp32 value q * s rounded to bf16,
    which must equal torch's float32 -> bfloat16 conversion (round to nearest,
    ties to even) -- including exact ties such as 1 + 2^-8 and 3 + 2^-7, and
    values of every magnitude."""
    rng = np.random.default_rng(21)
    H = 64
    sc = np.concatenate([np.float32([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1.5 + 2.0 ** -8]),
                         rng.uniform(0.5, 2.0, 125).astype(np.float32)
                         * np.float32(2.0) ** rng.integers(-60, 60, 125).astype(np.float32)])
    q = rng.integers(-127, 128, (sc.size, H)).astype(np.int8)
    q[:3, :4] = [1, 2, 3, -1]
    rows = np.zeros((sc.size, H + 16), np.uint8)
    rows[:, :H] = q.view(np.uint8)
    rows[:, H:H + 4] = sc.view(np.uint8).reshape(-1, 4)
    rr = np.arange(sc.size, dtype=np.int32).reshape(-1, 1)
    out = oracle.combine(rows, rr, np.ones((sc.size, 1), np.float32), 1, H, "q8", True, scale_offset=H)
    v = torch.from_numpy(q.astype(np.float32) * sc[:, None])
    ref = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)


def test_quant_blocks_equal_token_rule_per_block():
    """XDS P089 (outputs quantized to INT8 before they travel): each 256-column
    block of a row, partial last block included, gets exactly the codes and
    scale that the pinned token rule (c3) gives that block on its own; an
    all-zero block has s = 0, q = 0; the block amax element maps to +-127 and
    |y - q s| <= s (0.5 + 2^-16)."""
    rng = np.random.default_rng(21)
    n, H, B = 24, 640, 256  # blocks of 256, 256 and 128 columns
    yf = rng.standard_normal((n, H)).astype(np.float32) * rng.uniform(1e-3, 1e2, (n, 1)).astype(np.float32)
    yf[3, 256:512] = 0.0
    y = mw.to_bf16_bits(yf)
    q, s = oracle.quant_blocks(y, B)
    assert s.shape == (n, 3)
    for b in range(3):
        c0, c1 = b * B, min(H, (b + 1) * B)
        qt, st = oracle.quant_tokens(np.ascontiguousarray(y[:, c0:c1]), True)
        assert np.array_equal(q[:, c0:c1], qt) and np.array_equal(s[:, b], st)
    assert s[3, 1] == 0 and np.all(q[3, 256:512] == 0)
    yd = _bf16_to_f32(y).astype(np.float64)
    sb = np.repeat(s, B, axis=1)[:, :H].astype(np.float64)
    assert np.all(np.abs(yd - q * sb) <= sb * (0.5 + 2.0 ** -16))
    for b in range(3):
        c0, c1 = b * B, min(H, (b + 1) * B)
        i = np.abs(yd[:, c0:c1]).argmax(1)
        live = s[:, b] > 0
        assert np.all(np.abs(q[np.arange(n)[live], c0 + i[live]]) == 127)


def test_quant_tokenwise_returns_equal_token_rule():
    """Token-wise INT8 expert returns (XDS P085's one scale per token applied to the
    outputs P089 quantizes): the row mode (one block spanning the row) gives exactly
    the codes and scale of the pinned token rule (c3) on the bf16 row, for normal,
    all-zero, subnormal, huge and exactly-half rows; the row amax maps to +-127."""
    rng = np.random.default_rng(24)
    n, H = 12, 384
    yf = rng.standard_normal((n, H)).astype(np.float32) * rng.uniform(1e-3, 1e3, (n, 1)).astype(np.float32)
    yf[1] = 0.0
    yf[2] = rng.integers(-3, 4, H).astype(np.float32) * np.float32(2.0 ** -130)
    yf[3] = rng.uniform(-3e38, 3e38, H).astype(np.float32)
    yf[4] = 0.5 + rng.integers(-127, 127, H).astype(np.float32)
    yf[4, :3] = [127.0, 2.5, -2.5]
    y = mw.to_bf16_bits(yf)
    q, s = oracle.quant_blocks(y, H)
    qt, st = oracle.quant_tokens(y, True)
    assert s.shape == (n, 1)
    assert np.array_equal(q, qt) and np.array_equal(s[:, 0].view(np.uint32), st.view(np.uint32))
    assert s[1, 0] == 0 and np.all(q[1] == 0)
    assert s[4, 0] == 1 and q[4, :3].tolist() == [127, 2, -2]
    live = s[:, 0] > 0
    i = np.abs(_bf16_to_f32(y)).argmax(1)
    assert np.all(np.abs(q[np.arange(n)[live], i[live]]) == 127)


def test_combine_block_scales_reduce_to_row_scale_and_closed_form():
    """Combine of INT8 rows with block scales: with one block spanning the row it
    is the pinned single-scale INT8 mode exactly; k = 1, w = 1 gives q * s of
    each column's block exactly; fp32 accumulation agrees with a float64 einsum
    of the dequantized rows to fp32 rounding."""
    rng = np.random.default_rng(22)
    T, k, H, B = 30, 4, 320, 128
    y = mw.to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    q, sblk = oracle.quant_blocks(y, B)
    rb = ((H + 4 * sblk.shape[1] + 15) // 16) * 16
    rows = oracle.int8_return_rows(q, sblk, rb)
    wts = rng.uniform(0, 1, (T, k)).astype(np.float32)
    rr = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    out = oracle.combine(rows, rr, wts, k, H, "q8blocks", False, scale_offset=H, scale_block=B)
    v = q.astype(np.float64) * np.repeat(sblk, B, axis=1)[:, :H]
    ref = np.einsum("tj,tjc->tc", wts.astype(np.float64), v[rr])
    bound = 8 * 2.0 ** -24 * np.einsum("tj,tjc->tc", wts.astype(np.float64), np.abs(v[rr]))
    assert np.all(np.abs(out - ref) <= bound + 1e-30)
    one = oracle.combine(rows, rr[:, :1], np.ones((T, 1), np.float32), 1, H, "q8blocks", False,
                         scale_offset=H, scale_block=B)
    assert np.array_equal(one, (q.astype(np.float32) * np.repeat(sblk, B, axis=1)[:, :H])[rr[:, 0]])
    q1, s1 = oracle.quant_blocks(y, H)
    rows1 = oracle.int8_return_rows(q1, s1, rb)
    a = oracle.combine(rows1, rr, wts, k, H, "q8blocks", False, scale_offset=H, scale_block=H)
    b = oracle.combine(rows1, rr, wts, k, H, "q8", False, scale_offset=H)
    assert np.array_equal(a, b)


# ------------------------------------------------------------ c2' planner ---

def test_eplb_plan_worked_example():
    """Hand-worked example of the selection/placement procedure (golden)."""
    g = _golden("eplb_tiny_worked.json")
    out = oracle.eplb_plan(np.array(g["token_count"]), g["budget"], g["D"],
                           np.array(g["primary_partition"]), np.array(g["free_slots"]))
    assert out["selected"].tolist() == g["expected_selected"]
    np.testing.assert_allclose(out["tail"], g["expected_tail"])
    assert out["slot_partition"].tolist() == g["expected_slot_partition"]
    assert out["slot_logical"].tolist() == g["expected_slot_logical"]
    assert out["replica_offsets"].tolist() == g["expected_replica_offsets"]
    assert out["replica_slots"].tolist() == g["expected_replica_slots"]


def test_eplb_plan_invariants_on_skewed_counts():
    """Skewed counts: the tail never increases round to round; the budget is
    spent; every expert keeps >= 1 copy (XDS 故障恢复, note on P119: every logical
    expert needs at least one physical copy);
    replica lists are ascending; every round's pick is the best candidate by a
    brute-force search over all experts that are some slice's hottest."""
    rng = np.random.default_rng(11)
    E, slices, budget = 32, 4, 8
    pop = np.exp(-1.1 * np.log(rng.permutation(E) + 1.0))
    cnt = np.stack([rng.multinomial(2000, pop / pop.sum()) for _ in range(slices)]).astype(np.int64)
    D = E + budget
    out = oracle.eplb_plan(cnt, budget, D, np.arange(E), np.r_[np.zeros(E), np.ones(budget)].astype(np.int32))
    tail = out["tail"]
    assert np.all(np.diff(tail) <= 1e-9)
    assert np.all(out["selected"] >= 0)
    ro, rs = out["replica_offsets"], out["replica_slots"]
    assert ro[-1] == E + budget and np.all(np.diff(ro) >= 1)
    for e in range(E):
        assert np.all(np.diff(rs[ro[e]:ro[e + 1]]) > 0)
        assert np.all(out["slot_logical"][rs[ro[e]:ro[e + 1]]] == e)
    copies = np.ones(E)
    for r, c in enumerate(out["selected"]):
        best = None
        cands = sorted({int(np.argmax(cnt[t] / copies)) for t in range(slices)})
        for cand in cands:
            cp = copies.copy()
            cp[cand] += 1
            tl = sum((cnt[t] / cp).max() for t in range(slices))
            if best is None or tl < best[0]:
                best = (tl, cand)
        assert best[1] == c
        copies[c] += 1
    # replicas go to the free slots (partitions E..E+budget-1), which all start
    # empty: the heaviest replica takes the lowest partition id, and so on up
    # (SELECT_AND_PLACE_REPLICAS sorts by load; ties of partition load go to
    # the lower id), which reproduces the single-slot placement 256, 257, ...
    order = sorted(range(budget), key=lambda i: (-cnt.sum(0)[out["selected"][i]], i))
    placed = [int(out["slot_logical"][E + i]) for i in range(budget)]
    assert placed == [int(out["selected"][i]) for i in order]
    assert out["slot_partition"][E:].tolist() == list(range(E, E + budget))


def test_eplb_plan_candidate_tie_rules_worked():
    """Hand-worked: one slice, counts (3, 10, 10), one redundant slot.  The
    candidates are the slices' hottest experts, the lower id on a tie, so the
    only candidate is expert 1; its extra copy leaves the tail at 10 (expert 2
    still carries 10).  Expert 1 is selected -- neither the higher-id tied
    expert 2 nor expert 0, which gives the same tail but is no slice's hottest
    (XDS 专家负载均衡, SELECT_AND_PLACE_REPLICAS)."""
    out = oracle.eplb_plan(np.array([[3, 10, 10]]), 1, 2, np.array([0, 0, 1]), np.array([0, 1]))
    assert out["selected"].tolist() == [1]
    np.testing.assert_allclose(out["tail"], [10.0, 10.0])
    assert out["slot_logical"].tolist() == [0, 1, 2, 1]
    assert out["slot_partition"].tolist() == [0, 0, 1, 1]


def test_eplb_plan_primary_shares_worked():
    """Hand-worked placement where replicas may share a partition with primaries:
    one slice, counts (100, 10, 60, 45), primaries {0, 1} on partition 0 and
    {2, 3} on partition 1, one free slot on each, one redundant slot.  Expert 0
    is the hottest and gets the copy (tail 100 -> 60).  A primary's partition
    carries total / copies: partition 0 holds 100/2 + 10 = 60 and partition 1
    holds 60 + 45 = 105, so the replica (load 50) goes to partition 0."""
    out = oracle.eplb_plan(np.array([[100, 10, 60, 45]]), 1, 2, np.array([0, 0, 1, 1]),
                           np.array([1, 1]))
    assert out["selected"].tolist() == [0]
    np.testing.assert_allclose(out["tail"], [100.0, 60.0])
    assert out["slot_partition"].tolist() == [0, 0, 1, 1, 0]
    assert out["slot_logical"].tolist() == [0, 1, 2, 3, 0]
    assert out["replica_offsets"].tolist() == [0, 2, 3, 4, 5]
    assert out["replica_slots"].tolist() == [0, 4, 1, 2, 3]


# ---------------------------------------------------------- c4' sizes ---

def test_static_buffer_printed_values():
    """CMI 缓冲区公式 printed values (golden): 225 MB dispatch + 420 MB combine
    = 645 MB per die at 320 ranks, local batch 96, one expert per die."""
    g = _golden("static_buffers_ep320.json")
    mt, disp = oracle.static_buffer(g["rank_num"], g["local_batch"], g["topk"], g["experts_per_die"],
                                    g["dispatch_msg_bytes"])
    _, comb = oracle.static_buffer(g["rank_num"], g["local_batch"], g["topk"], g["experts_per_die"],
                                   g["combine_msg_bytes"])
    assert mt == g["expected_max_tokens"]
    assert disp == g["expected_dispatch_MiB"] * 2 ** 20
    assert comb == g["expected_combine_MiB"] * 2 ** 20
    assert disp + comb == g["expected_total_MiB"] * 2 ** 20
    a, b, c = g["global_batches"]["ep128"]
    assert a * b == c


# ------------------------------------------------------- composed path ---

def test_layer_tiny_workload_end_to_end():
    """The tiny workload (T=16, H=64, 8 experts on 4 partitions, top-2 softmax,
    identity experts): every token appears exactly k times in the dispatch
    buffers, per-expert counts sum to T k, and the combine returns
    sum_j w_j dequant(quant(x)) ~ x."""
    w = mw.WORKLOADS["tiny"]
    x = mw.hidden(w)
    lg = mw.logits(w)
    ro, rs, sp, sl = mw.identity_map(w)
    r = oracle.moe_layer(w, x, lg, None, None, None, sp, sl, event_id=7)
    toks = []
    for rr in range(w.T * w.k):
        row = r["route_rows"][rr]
        sc, src, b, j, loc, ev = struct.unpack("<fiiBBH", row[w.H:w.H + 16].tobytes())
        toks.append(src * w.LB + b)
    assert np.array_equal(np.bincount(toks, minlength=w.T), np.full(w.T, w.k))
    assert oracle.expert_counts(r["topk_ids"], w.E).sum() == w.T * w.k
    assert np.all(np.abs(r["out"] - x) <= r["scale"][:, None] * 0.5 + 1e-6)


def test_eplb_plan_honours_primary_partition_of_any_int_dtype():
    """Regression: integer arrays of any dtype (converted by the wrapper) reach the
    planner intact; primaries stay on their partitions."""
    cnt = np.array([[50, 3, 2, 1, 1, 1]], np.int64)
    prim = np.array([5, 4, 3, 2, 1, 0], np.int64)
    for _ in range(20):
        out = oracle.eplb_plan(cnt, 2, 8, prim, np.array([0, 0, 0, 0, 0, 0, 1, 1], np.int64))
        assert out["slot_partition"][:6].tolist() == prim.tolist()
        assert sorted(out["slot_partition"][6:].tolist()) == [6, 7]
