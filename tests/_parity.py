"""Helpers shared by the GPU parity tests: inputs on the device from the seeded
generators, the same bytes on the host for the oracle, and comparisons."""
from __future__ import annotations

import numpy as np
import torch

import combine_moe_route_topk_amd as moe
import moe_workloads as mw
import oracle

FP32_RTOL, FP32_ATOL = 1e-5, 1e-6      # fp32 outputs (weights, fp32 combine)
BF16_RTOL, BF16_ATOL = 1e-2, 1e-3      # bf16 outputs


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b).view(np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def dev_bits(a: np.ndarray, is_bf16: bool) -> torch.Tensor:
    """uint16 bf16 bit patterns -> a torch.bfloat16 device tensor with the same bits."""
    if is_bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def replica_map(w: mw.Workload, calib_ids=None):
    """(replica_offsets, replica_slots, slot_partition, slot_logical) on the host."""
    if w.eplb == "first32":
        return mw.first32_map(w)
    if w.eplb == "plan":
        # counts of the calibration slices -> the planner (oracle side)
        counts = np.stack([oracle.expert_counts(ids, w.E) for ids in calib_ids])
        out = oracle.eplb_plan(counts, w.budget, w.D, np.arange(w.E),
                               np.r_[np.zeros(w.E), np.ones(w.budget)].astype(np.int32))
        return out["replica_offsets"], out["replica_slots"], out["slot_partition"], out["slot_logical"]
    return mw.identity_map(w)


def calib_ids(w: mw.Workload):
    bias = mw.zipf_bias(w)
    return [oracle.route_topk(mw.logits(w, i), w.k, w.gating, bias,
                              logits_bf16=w.logits_dtype == "bf16")[0]
            for i in range(w.calib_slices)]


def assert_close(got, ref, rtol, atol, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at "
                             f"{tuple(i)}: got {got[tuple(i)]!r} ref {ref[tuple(i)]!r}")


def gather_rows(buf: moe.MoeBuffers, rows: np.ndarray) -> np.ndarray:
    """Message rows of the dispatch buffer at the given row indices (host bytes)."""
    v = buf.disp_rows_view()
    idx = torch.from_numpy(np.ascontiguousarray(rows, np.int64)).cuda()
    return v.index_select(0, idx).cpu().numpy()
