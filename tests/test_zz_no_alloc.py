"""The allocation-free dispatch (moe_dispatch_q8_static) against moe_dispatch_q8:
every output bit-identical, on two calls in a row that share the library's
static scratch, the second smaller than the first (and with one invalid route,
so the device status words are compared too)."""
import numpy as np
import pytest
import torch

import combine_moe_route_topk_amd as moe
import moe_workloads as mw
from _parity import dev_bits, host

pytestmark = pytest.mark.gpu

FIRST = mw.Workload("noalloc_first", T=3 * 100, H=384, E=40, P=40, k=8, D=10, Epp=4, S=3, LB=100,
                    gating="sigmoid", logits_dtype="bf16", x_dtype="bf16", zipf=True,
                    experts="identity", combine="q8", out_dtype="f32")
SECOND = mw.WORKLOADS["tiny"]


def _layer(w):
    ro, rs, sp, sl = mw.identity_map(w)
    bias = mw.zipf_bias(w)
    return moe.MoeLayer(moe.geom_of(w), w.gating, torch.from_numpy(sp).cuda(),
                        torch.from_numpy(sl).cuda(),
                        bias=None if bias is None else torch.from_numpy(bias).cuda(),
                        out_dtype=torch.float32)


def _compare(w, bad_route=None, event_id=0x5151):
    print(f"[no-alloc] {w.name} T={w.T} H={w.H} P={w.P} D={w.D} S={w.S}", flush=True)
    ref, new = _layer(w), _layer(w)
    x = dev_bits(mw.hidden(w), w.x_dtype == "bf16")
    ref.route(dev_bits(mw.logits(w), w.logits_dtype == "bf16"))
    if bad_route is not None:
        ref.buf.phys[bad_route] = w.P + 5
    new.buf.phys.copy_(ref.buf.phys)
    a, b = ref.buf, new.buf
    ref.event_id = event_id - 1
    ref.dispatch(x)  # moe_dispatch_q8 with the layer's own scratch
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    moe.moe_dispatch_q8_static(x, moe.DTYPE_BF16 if w.x_dtype == "bf16" else moe.DTYPE_F32,
                               b.phys, new.slot_partition, event_id, new.g, b.disp_buf, b.meta,
                               b.slot_count, b.slot_offset, b.slot_rows, b.disp_row, b.ret_row,
                               b.relay_buf, status)
    torch.cuda.synchronize()
    for name in ("meta", "slot_count", "slot_offset", "slot_rows", "disp_row", "ret_row"):
        assert np.array_equal(host(getattr(a, name)), host(getattr(b, name))), name
    assert int(host(status)[0]) == a.device_status(), "device status word"
    rows = host(a.disp_row).ravel()
    rows = rows[rows >= 0]
    idx = torch.from_numpy(rows.astype(np.int64)).cuda()
    n = w.H + 16  # codes + trailer; the line padding after them is unspecified
    ra = a.disp_rows_view().index_select(0, idx)[:, :n]
    rb = b.disp_rows_view().index_select(0, idx)[:, :n]
    assert torch.equal(ra, rb), "message rows"
    return a.device_status()


def test_static_dispatch_equals_dispatch_twice():
    assert _compare(FIRST) == 0
    st = _compare(SECOND, bad_route=(3, 1), event_id=0x6262)
    assert st & moe.MOE_DEVICE_BAD_ROUTE
