"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, sizes buffers per the static-buffer formula, rejects bad arguments
before any launch, and its EPLB planner matches the oracle's."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import combine_moe_route_topk_amd as moe
import moe_workloads as mw
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        txt = open(h).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        names |= set(re.findall(r"^\s*(?:int|const char\s*\*)\s*(moe_\w+)\s*\(", txt, flags=re.M))
    return names


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    decl = _declared_symbols()
    assert decl == set(moe.EXPORTED), decl ^ set(moe.EXPORTED)
    for n in decl:
        assert hasattr(L, n)
    assert moe.status_string(moe.MOE_ERR_CAPACITY) == "capacity exceeded"


def test_limits_match_the_header_and_bound_the_geometry():
    """The binding's limits are the header's #defines, and the host validation
    takes each limit and refuses one past it."""
    txt = open(os.path.join(ROOT, "include", "moe_route_topk.h")).read()
    for name in ("E", "P", "D", "K", "H"):
        m = re.search(r"#define MOE_MAX_%s (\d+)" % name, txt)
        assert m and int(m.group(1)) == getattr(moe, "MAX_" + name), name
    ok = dict(T=64, H=moe.MAX_H, E=moe.MAX_E, P=moe.MAX_P, k=moe.MAX_K, D=moe.MAX_D, Epp=1, S=1,
              LB=64)
    assert moe.moe_plan_sizes(moe.geom(**ok), 2048).cap_rows == 64
    for key, bad in (("H", moe.MAX_H + 16), ("k", moe.MAX_K + 1)):
        with pytest.raises(moe.MoeError) as e:
            moe.moe_plan_sizes(moe.geom(**dict(ok, **{key: bad})), 2048)
        assert e.value.status == moe.MOE_ERR_UNSUPPORTED, key
    for key in ("E", "P", "D"):
        big = dict(ok, E=moe.MAX_E + 1, P=moe.MAX_P + 1, D=moe.MAX_D + 1)
        big = dict(ok, **{k: v for k, v in big.items() if k in ("P", key)})
        with pytest.raises(moe.MoeError) as e:
            moe.moe_plan_sizes(moe.geom(**big), 2048)
        assert e.value.status == moe.MOE_ERR_UNSUPPORTED, key


def test_plan_sizes_reproduce_printed_static_buffers():
    """CMI 缓冲区公式: 320 ranks, local batch 96, 1 expert per die, top-8 ->
    225 MiB dispatch (7680-byte messages) and 420 MiB bf16 combine per die."""
    g = moe.geom(T=320 * 96, H=7168, E=320, P=320, k=8, D=320, Epp=1, S=320, LB=96, msg_bytes=7680)
    s = moe.moe_plan_sizes(g, 2048)
    assert s.cap_rows == 96
    assert s.dispatch_bytes_per_partition == 225 * 2 ** 20
    assert s.combine_bytes_per_partition == 420 * 2 ** 20
    assert s.dispatch_bytes == 320 * 225 * 2 ** 20
    # default message: H codes + 16-byte trailer, padded to a 128-byte line
    g.msg_bytes = 0
    s = moe.moe_plan_sizes(g, 0)
    assert s.msg_bytes == 7296 and s.ffn_scratch_bytes == 0


@pytest.mark.parametrize("name", list(mw.WORKLOADS))
def test_plan_sizes_of_every_workload(name):
    w = mw.WORKLOADS[name]
    s = moe.moe_plan_sizes(moe.geom_of(w), w.I)
    assert s.cap_rows == w.cap and s.msg_bytes == w.msg
    assert s.dispatch_bytes == w.D * w.S * w.cap * w.msg
    if w.relays:
        assert s.relay_bytes == (w.D - w.relays) * w.S * w.cap * w.msg


def test_invalid_arguments_rejected_before_launch():
    """Host validation returns an error code and launches nothing (runs without a GPU)."""
    L = moe.lib()
    g = moe.geom(T=16, H=64, E=8, P=8, k=2, D=4, Epp=2, S=4, LB=4)
    bad = moe.geom(T=15, H=64, E=8, P=8, k=2, D=4, Epp=2, S=4, LB=4)  # T != S * LB
    assert L.moe_route_topk(None, 0, None, 0, None, None, ctypes.byref(g), None, None, None, None,
                            None) == moe.MOE_ERR_INVALID_ARG
    fake = ctypes.c_void_p(0x1000)
    assert L.moe_route_topk(fake, 0, None, 0, None, None, ctypes.byref(bad), fake, fake, fake,
                            None, None) == moe.MOE_ERR_INVALID_ARG
    odd = moe.geom(T=16, H=60, E=8, P=8, k=2, D=4, Epp=2, S=4, LB=4)
    assert L.moe_combine(0, fake, fake, fake, ctypes.byref(odd), 0, fake, None) == moe.MOE_ERR_UNSUPPORTED
    bigk = moe.geom(T=16, H=64, E=32, P=32, k=17, D=4, Epp=8, S=4, LB=4)
    assert L.moe_combine(0, fake, fake, fake, ctypes.byref(bigk), 0, fake, None) == moe.MOE_ERR_UNSUPPORTED
    # misaligned buffer
    assert L.moe_combine(0, ctypes.c_void_p(0x1004), fake, fake, ctypes.byref(g), 0, fake,
                         None) == moe.MOE_ERR_INVALID_ARG
    # scratch too small
    s = moe.moe_plan_sizes(g)
    assert L.moe_dispatch_q8(fake, 0, fake, fake, 1, ctypes.byref(g), fake, fake, fake, fake, fake,
                             fake, fake, None, fake, s.dispatch_scratch_bytes - 1,
                             None) == moe.MOE_ERR_CAPACITY
    # FFN needs H % 128 == 0 and I % 64 == 0 (whole 64-byte K steps)
    for bad_i in (96, 160):
        assert L.moe_expert_ffn_q8(fake, fake, fake, fake, fake, fake, fake, fake, fake, bad_i,
                                   ctypes.byref(g), fake, None, None, fake, 1 << 30,
                                   None) == moe.MOE_ERR_UNSUPPORTED
    # the expert epilogues read the channel scales four at a time: 16-byte aligned
    g128 = moe.geom(T=16, H=128, E=8, P=8, k=2, D=4, Epp=2, S=4, LB=4)
    odd4 = ctypes.c_void_p(0x1004)
    assert L.moe_expert_gateup_q8(fake, fake, fake, fake, fake, fake, odd4, 64, ctypes.byref(g128),
                                  None, fake, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_expert_down_q8(fake, fake, fake, fake, odd4, 64, ctypes.byref(g128), fake, None,
                                fake, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    # relay hop without relays configured
    assert L.moe_relay_returns(fake, fake, fake, fake, ctypes.byref(g), fake,
                               None) == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError):
        moe.moe_plan_sizes(bad)


def test_int8_returns_and_router_validation():
    """The INT8-return and gate-logit entry points check their arguments on the
    host and return an error code without launching (runs without a GPU)."""
    L = moe.lib()
    fake = ctypes.c_void_p(0x1000)
    g = moe.geom(T=16, H=256, E=8, P=8, k=2, D=4, Epp=2, S=4, LB=4)
    s = moe.moe_plan_sizes(g, 256)
    # INT8 return rows: H codes + one fp32 scale per 256 columns, whole 128-byte lines
    assert s.ret_q8_row_bytes == 384 and s.ret_q8_bytes == 16 * 2 * 384
    g2 = moe.geom(T=16, H=7168, E=8, P=8, k=2, D=4, Epp=2, S=4, LB=4)
    assert moe.moe_plan_sizes(g2, 256).ret_q8_row_bytes == 7296  # 7168 + 112 -> 57 lines
    relay = moe.geom(T=16, H=256, E=8, P=8, k=2, D=4, Epp=1, S=4, LB=4, relays=2)
    assert L.moe_expert_down_q8_int8ret(fake, fake, fake, fake, fake, 256, ctypes.byref(relay),
                                        fake, None, fake, 1 << 30, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_down_q8_int8ret(None, fake, fake, fake, fake, 256, ctypes.byref(g), fake,
                                        None, fake, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    # combine: an unknown return mode
    assert L.moe_combine(4, fake, fake, fake, ctypes.byref(g), 0, fake, None) == moe.MOE_ERR_INVALID_ARG
    # token-wise INT8 returns: not with relays, NULL and misaligned pointers refused
    assert L.moe_quant_returns_q8(fake, fake, ctypes.byref(relay), fake,
                                  None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_quant_returns_q8(None, fake, ctypes.byref(g), fake, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_quant_returns_q8(fake, fake, ctypes.byref(g), ctypes.c_void_p(0x1004),
                                  None) == moe.MOE_ERR_INVALID_ARG
    # router: H a multiple of 64, E a multiple of 4, scratch large enough, 16-byte alignment
    for h in (80, 96):
        odd_h = moe.geom(T=16, H=h, E=8, P=8, k=2, D=4, Epp=2, S=4, LB=4)
        assert L.moe_router_logits(fake, fake, ctypes.byref(odd_h), fake, fake, 1 << 30,
                                   None) == moe.MOE_ERR_UNSUPPORTED
    odd_e = moe.geom(T=16, H=256, E=6, P=6, k=2, D=3, Epp=2, S=4, LB=4)
    assert L.moe_router_logits(fake, fake, ctypes.byref(odd_e), fake, fake, 1 << 30,
                               None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_router_logits(fake, fake, ctypes.byref(g), fake, fake,
                               s.router_scratch_bytes - 1, None) == moe.MOE_ERR_CAPACITY
    assert L.moe_router_logits(ctypes.c_void_p(0x1008), fake, ctypes.byref(g), fake, fake,
                               1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    # split count: 192-token x 256-expert tiles; the largest divisor of the
    # 64-element step count keeping tiles x splits <= 256 (at most 32);
    # scratch = splits x T x E fp32
    def splits(T, H, E):
        gg = moe.geom(T=T, H=H, E=E, P=E, k=1, D=E, Epp=1, S=1, LB=T)
        return moe.moe_plan_sizes(gg, 256).router_scratch_bytes // (T * E * 4)
    assert splits(16, 256, 8) == 4                # 1 tile, 4 steps
    assert splits(12288, 7168, 256) == 4          # 64 tiles x 4 = 256 blocks
    assert splits(46080, 7168, 256) == 1          # 240 tiles
    assert splits(4096, 7168, 256) == 8           # 22 tiles, 112 steps
    assert splits(96, 7168, 256) == 28            # 1 tile: 28 of the 112 steps' divisors
    assert splits(300, 384, 40) == 6              # 2 tiles, 6 steps: one step per split
    assert splits(16, 64, 8) == 1                 # a single step
    assert splits(4100, 192, 1020) == 1           # 88 tiles x 3 steps > 256


def test_pack_expert_weights_validation_and_sizes():
    """The weight packer's sizes (one 16 KB block per expert, n-tile and 64-byte
    K step; partial n-tiles padded, K padded to whole groups of four steps) and
    its host-side argument checks (no launch)."""
    L = moe.lib()
    s = moe.moe_plan_sizes(moe.geom(T=0, H=7168, E=256, P=256, k=1, D=1, Epp=1, S=1, LB=0), 2048)
    assert s.w_gateup_packed_bytes == 256 * 2 * 2048 * 7168
    assert s.w_down_packed_bytes == 256 * 7168 * 2048
    s = moe.moe_plan_sizes(moe.geom(T=0, H=384, E=3, P=3, k=1, D=1, Epp=1, S=1, LB=0), 192)
    assert s.w_gateup_packed_bytes == 3 * 2 * 8 * 16384   # two n-tiles of 128 pairs, 6 -> 8 K steps
    assert s.w_down_packed_bytes == 3 * 2 * 4 * 16384     # two n-tiles of 256 rows, 3 -> 4 K steps
    w, pk = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x40000000)
    ok = s.w_gateup_packed_bytes
    G, D = moe.PROJ_GATEUP, moe.PROJ_DOWN
    assert L.moe_pack_expert_weights(None, G, 3, 384, 192, pk, ok, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_expert_weights(w, G, 3, 384, 192, None, ok, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_expert_weights(ctypes.c_void_p(0x10008), G, 3, 384, 192, pk, ok,
                                     None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_expert_weights(w, 2, 3, 384, 192, pk, ok, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_expert_weights(w, G, 0, 384, 192, pk, ok, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_expert_weights(w, G, 3, 320, 192, pk, ok, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_expert_weights(w, D, 3, 384, 96, pk, ok, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_expert_weights(w, G, 3, 384, 192, pk, ok - 1, None) == moe.MOE_ERR_CAPACITY
    # the image may not overlap the plain weights
    assert L.moe_pack_expert_weights(w, G, 3, 384, 192, ctypes.c_void_p(0x10000 + 4096), ok,
                                     None) == moe.MOE_ERR_INVALID_ARG


def test_router_topk_validation():
    """The one-call gate + top-k checks both halves' arguments on the host and
    returns before any launch (runs without a GPU)."""
    L = moe.lib()
    fake = ctypes.c_void_p(0x1000)
    g = moe.geom(T=16, H=256, E=8, P=8, k=2, D=4, Epp=2, S=4, LB=4)
    s = moe.moe_plan_sizes(g, 0)
    args = lambda **kw: [kw.get("x", fake), fake, None, kw.get("gating", moe.GATING_SIGMOID),
                         kw.get("ro", None), None, ctypes.byref(kw.get("g", g)), None, fake, fake,
                         fake, None, fake, kw.get("sb", s.router_scratch_bytes), None]
    assert L.moe_router_topk(*args(gating=5)) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_router_topk(*args(ro=fake)) == moe.MOE_ERR_INVALID_ARG     # offsets without slots
    assert L.moe_router_topk(*args(sb=s.router_scratch_bytes - 1)) == moe.MOE_ERR_CAPACITY
    assert L.moe_router_topk(*args(x=ctypes.c_void_p(0x1008))) == moe.MOE_ERR_INVALID_ARG
    odd_e = moe.geom(T=16, H=256, E=6, P=6, k=2, D=3, Epp=2, S=4, LB=4)
    assert L.moe_router_topk(*args(g=odd_e)) == moe.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("seed,E,slices,budget", [(0, 32, 4, 8), (1, 64, 3, 16), (2, 8, 1, 5)])
def test_eplb_planner_matches_oracle(seed, E, slices, budget):
    rng = np.random.default_rng(seed)
    pop = np.exp(-1.1 * np.log(rng.permutation(E) + 1.0))
    cnt = np.stack([rng.multinomial(3000, pop / pop.sum()) for _ in range(slices)]).astype(np.int64)
    D = E // 2 + budget
    prim = (np.arange(E) // 2).astype(np.int32)
    free = np.r_[np.zeros(E // 2), np.ones(budget)].astype(np.int32)
    ro, rs, sp, sl, sel = moe.moe_eplb_build_map(cnt, budget, D, prim, free)
    o = oracle.eplb_plan(cnt, budget, D, prim, free)
    assert np.array_equal(ro, o["replica_offsets"]) and np.array_equal(rs, o["replica_slots"])
    assert np.array_equal(sp, o["slot_partition"]) and np.array_equal(sl, o["slot_logical"])
    assert np.array_equal(sel, o["selected"][:budget])


def test_eplb_planner_capacity_error():
    cnt = np.array([[10, 1, 1, 1]], np.int64)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_eplb_build_map(cnt, 3, 2, np.array([0, 0, 1, 1]), np.array([1, 1]))
    assert ei.value.status == moe.MOE_ERR_CAPACITY


def test_eplb_planner_on_the_eplb_workload():
    """The 4096-token EPLB workload: 32 redundant slots planned from the
    calibration batch land on partitions 256..287 and match the oracle."""
    w = mw.WORKLOADS["eplb4096"]
    bias = mw.zipf_bias(w)
    counts = np.stack([oracle.expert_counts(
        oracle.route_topk(mw.logits(w, i), w.k, w.gating, bias, logits_bf16=True)[0], w.E)
        for i in range(w.calib_slices)])
    prim = np.arange(w.E, dtype=np.int32)
    free = np.r_[np.zeros(w.E), np.ones(w.budget)].astype(np.int32)
    ro, rs, sp, sl, sel = moe.moe_eplb_build_map(counts, w.budget, w.D, prim, free)
    o = oracle.eplb_plan(counts, w.budget, w.D, prim, free)
    assert np.array_equal(sl, o["slot_logical"]) and np.array_equal(sp, o["slot_partition"])
    assert sorted(sp[w.E:].tolist()) == list(range(w.E, w.E + w.budget))
    assert np.all(np.diff(o["tail"]) <= 1e-9)


def test_static_dispatch_validation():
    """The allocation-free dispatch refuses a geometry whose scratch exceeds its
    static array, and invalid arguments, before any launch (no GPU needed)."""
    L = moe.lib()
    fake = ctypes.c_void_p(0x1000)
    g = moe.geom(T=1 << 20, H=128, E=1024, P=1024, k=16, D=1024, Epp=1, S=1, LB=1 << 20)
    assert moe.moe_plan_sizes(g, 0).dispatch_scratch_bytes > moe.MOE_STATIC_SCRATCH_BYTES
    assert L.moe_dispatch_q8_static(fake, moe.DTYPE_BF16, fake, fake, 1, ctypes.byref(g), fake,
                                    fake, fake, fake, fake, fake, fake, None, None,
                                    None) == moe.MOE_ERR_CAPACITY
    bad = moe.geom(T=16, H=100, E=8, P=8, k=2, D=4, Epp=2, S=4, LB=4)  # H % 16 != 0
    assert L.moe_dispatch_q8_static(fake, moe.DTYPE_BF16, fake, fake, 1, ctypes.byref(bad), fake,
                                    fake, fake, fake, fake, fake, fake, None, None,
                                    None) == moe.MOE_ERR_UNSUPPORTED


def test_check_event_validation_and_status_string():
    """moe_check_event refuses NULL pointers before any launch; MOE_ERR_STALE has a name."""
    L = moe.lib()
    fake = ctypes.c_void_p(0x1000)
    g = moe.geom(T=16, H=256, E=8, P=8, k=2, D=4, Epp=2, S=4, LB=4)
    assert L.moe_check_event(None, fake, fake, fake, ctypes.byref(g), 1, fake,
                             None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_check_event(fake, fake, fake, fake, ctypes.byref(g), 1, None,
                             None) == moe.MOE_ERR_INVALID_ARG
    assert "stale" in moe.status_string(moe.MOE_ERR_STALE)


def test_mfma_probe_validation():
    """The MFMA rate probe refuses empty launches and a NULL output before any launch."""
    L = moe.lib()
    fake = ctypes.c_void_p(0x1000)
    assert L.moe_probe_mfma_i8(0, 8, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_probe_mfma_i8(4, 0, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_probe_mfma_i8(4, 8, None, None) == moe.MOE_ERR_INVALID_ARG
