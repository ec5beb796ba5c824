#!/usr/bin/env python3
"""Throughput of the MoE hot path on one MI355X.

One step = one pass of the whole path over one batch, every stage in the
library's HIP kernels: gate top-k routing -> INT8 quantization fused into the
dispatch scatter -> grouped INT8 SwiGLU experts (gate/up stage, then
requant + down stage) -> combine of the bf16 returns.  The workload is the
12288-token layer (128 source partitions x 96 tokens, H=7168, 256 experts on
128 partitions x 2, top-8, I=2048, sigmoid gate with a seeded log-Zipf skew),
inputs resident in HBM before timing starts.

Prints ONE JSON line: tokens/s of the layer (value), dispatch+combine GB/s and
its fraction of the 8 TB/s HBM peak, per-stage times, the roofline of the
dominant kernel (the gate/up INT8 GEMM) and the CPU oracle's throughput on a
bounded sample of the same workload (cpu_baseline).

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 MFMA
COPY_BYTES = 1 << 30       # the calibration copy: 1 GiB read + 1 GiB written per launch
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "layer12288_ffn_gateup_traffic.txt")
GEMM_SRC = os.path.join(ROOT, "combine_moe_route_topk_amd", "csrc", "ffn_q8.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic(w):
    """Bytes / ops each stage must move or compute (never capacity or padding)."""
    T, H, E, k, I = w.T, w.H, w.E, w.k, w.I
    R = T * k
    return {
        # read logits (bf16) + write ids, weights, physical ids
        "route_bytes": T * E * 2 + R * 12,
        # read x (bf16) and phys ids, write the k messages (H + 16 B each),
        # the three row-index arrays and the (d, s) metadata
        "dispatch_bytes": T * H * 2 + R * 4 + R * (H + 16) + 3 * R * 4 + w.D * w.S * 16,
        # read bf16 returns, row ids and weights, write the bf16 output
        "combine_bytes": R * H * 2 + R * 8 + T * H * 2,
        # INT8 returns: read R rows of H codes + H/256 fp32 scales instead of bf16 rows
        "combine_q8_bytes": R * (H + 4 * (H // 256)) + R * 8 + T * H * 2,
        # 2 ops per multiply-add: gate and up (2I outputs over K = H), down (H outputs over K = I)
        "gateup_ops": 2 * R * H * 2 * I,
        "down_ops": 2 * R * I * H,
    }


def build_layer(w, log_every=64):
    import numpy as np
    import torch
    from concurrent.futures import ThreadPoolExecutor

    import combine_moe_route_topk_amd as moe
    import moe_workloads as mw

    t0 = time.time()
    x = torch.from_numpy(mw.hidden(w).view(np.int16)).view(torch.bfloat16).cuda()
    lg = torch.from_numpy(mw.logits(w).view(np.int16)).view(torch.bfloat16).cuda()
    bias = torch.from_numpy(mw.zipf_bias(w)).cuda()
    ro, rs, sp, sl = mw.identity_map(w)
    dev = dict(device="cuda")
    wgu = torch.empty((w.E, 2 * w.I, w.H), dtype=torch.int8, **dev)
    sgu = torch.empty((w.E, 2 * w.I), dtype=torch.float32, **dev)
    wd = torch.empty((w.E, w.H, w.I), dtype=torch.int8, **dev)
    sd = torch.empty((w.E, w.H), dtype=torch.float32, **dev)

    def fill(e):
        a, b, c, d = mw.expert_weights(w, e)
        wgu[e].copy_(torch.from_numpy(a))
        sgu[e].copy_(torch.from_numpy(b))
        wd[e].copy_(torch.from_numpy(c))
        sd[e].copy_(torch.from_numpy(d))
        if e % log_every == 0:
            log(f"[bench] weights of expert {e} generated ({time.time() - t0:.1f}s)")

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(fill, range(w.E)))
    torch.cuda.synchronize()
    log(f"[bench] inputs and weights resident in HBM ({time.time() - t0:.1f}s)")
    # the layer keeps the weights in the expert GEMMs' tile image (packed once,
    # outside any timed region); the plain copies are released afterwards
    layer = moe.MoeLayer(moe.geom_of(w), w.gating, torch.from_numpy(sp).cuda(),
                         torch.from_numpy(sl).cuda(), bias=bias, weights=(wgu, sgu, wd, sd),
                         I=w.I, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    del wgu, wd
    torch.cuda.empty_cache()
    log(f"[bench] expert weights packed ({time.time() - t0:.1f}s)")
    return layer, x, lg


def time_gpu(layer, x, lg, steps, warmup, returns="bf16", flush=None):
    """Per-step and per-stage times of `steps` whole steps.  returns: 'bf16' (the
    workload's expert returns), 'q8blocks' (INT8 returns, one scale per 256
    columns, quantized in the down projection's epilogue) or 'q8rows' (token-wise
    INT8 returns: one scale per row, quantized by moe_quant_returns_q8).  With
    `flush` (a device buffer), the buffer is overwritten before every step, outside
    the timed steps, so that each step starts with cold caches.

    The steps are timed twice.  First with one event at each step boundary (a pair
    around each step with `flush`), which gives the step time and its spread; then
    again with a pair of events around every stage, which gives the stage times.
    Events between the stages add time of their own, so the step time comes from
    the first pass."""
    import torch
    down = {"bf16": layer.experts_down, "q8rows": layer.experts_down,
            "q8blocks": layer.experts_down_int8ret}[returns]
    stages = [("route", lambda: layer.route(lg)),
              ("dispatch", lambda: layer.dispatch(x)),
              ("gateup", layer.experts_gateup),
              ("down", down)]
    if returns == "q8rows":
        stages.append(("quant_returns", layer.quant_returns))
    stages.append(("combine", lambda: layer.combine(returns)))

    def ev():
        return torch.cuda.Event(enable_timing=True)

    for _ in range(warmup):
        for _, f in stages:
            f()
    torch.cuda.synchronize()
    # pass 1: whole steps
    marks = [(ev(), ev()) if flush is not None else (ev(), None) for _ in range(steps)]
    last = ev()
    torch.cuda.synchronize()
    for s, (a, b) in enumerate(marks):
        if flush is not None:
            flush.fill_(s & 0xFF)
        a.record()
        for _, f in stages:
            f()
        if b is not None:
            b.record()
    last.record()
    torch.cuda.synchronize()
    if flush is None:
        ends = [m[0] for m in marks[1:]] + [last]
        step_ms = [a.elapsed_time(e) for (a, _), e in zip(marks, ends)]
        ms = marks[0][0].elapsed_time(last) / steps
    else:
        step_ms = [a.elapsed_time(b) for a, b in marks]
        ms = sum(step_ms) / steps
    step_ms.sort()
    q = lambda f: step_ms[min(len(step_ms) - 1, int(f * len(step_ms)))]
    dist = {"median": q(0.5), "p10": q(0.1), "p90": q(0.9)}
    # pass 2: every stage between its own pair of events
    evs = [[(ev(), ev()) for _ in stages] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        if flush is not None:
            flush.fill_(s & 0xFF)
        for (name, f), (a, b) in zip(stages, evs[s]):
            a.record()
            f()
            b.record()
    torch.cuda.synchronize()
    per = {name: sum(evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(steps)) / steps
           for i, (name, _) in enumerate(stages)}
    return ms, per, dist


def time_pipeline(layer, x, lg, w, steps, warmup, n_micro=2):
    """Whole steps of the same layer as a pipeline of n_micro microbatches (source
    partition groups), each on its own stream."""
    import torch
    import combine_moe_route_topk_amd as moe
    pipe = moe.MoePipeline(layer.g, n_micro, w.gating, layer.slot_partition, layer.slot_logical,
                           None, None, layer.bias, layer.weights, w.I, torch.bfloat16)
    for _ in range(warmup):
        pipe.forward(x, lg)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        pipe.forward(x, lg)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    del pipe
    torch.cuda.empty_cache()
    return {"n_micro": n_micro, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(w.T / (ms * 1e-3), 1),
            "note": "microbatches of T/2 tokens scheduled by MoeOverlap (route, dispatch and "
                    "combine on one stream beside the other microbatch's experts on another); "
                    "each microbatch's experts read every routed expert's weights; the output "
                    "equals the one-batch step's bit for bit"}


def time_batch_overlap(layer, x, lg, w, steps, warmup, n=2):
    """A stream of whole batches of the workload (its tokens rolled by 0..n-1 rows,
    in turn), each batch in one of n layers with their own static buffers: run one
    after another on one stream, and submitted to MoeOverlap back to back (route,
    dispatch and combine of one batch beside another's experts); mean time per
    batch of each over `steps` batches."""
    import torch
    import combine_moe_route_topk_amd as moe
    layers = [layer] + [moe.MoeLayer(layer.g, w.gating, layer.slot_partition,
                                     layer.slot_logical, bias=layer.bias, weights=layer.weights,
                                     I=w.I, out_dtype=torch.bfloat16) for _ in range(n - 1)]
    inputs = [(x, lg)] + [(torch.roll(x, i, 0).contiguous(), torch.roll(lg, i, 0).contiguous())
                          for i in range(1, n)]
    ov = moe.MoeOverlap(layers)

    def one_at_a_time(count):
        for i in range(count):
            layers[i % n].forward(*inputs[i % n])

    def overlapped(count):
        tickets = [ov.submit(*inputs[i % n]) for i in range(count)]
        for t in tickets[-n:]:
            t.wait()

    def per_batch_us(fn):
        fn(max(warmup, n))
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(steps)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / steps

    seq_us = per_batch_us(one_at_a_time)
    ovl_us = per_batch_us(overlapped)
    del ov, layers[1:], inputs
    torch.cuda.empty_cache()
    return {"n_layers": n, "batches": steps, "ms_per_batch": round(ovl_us * 1e-3, 4),
            "one_at_a_time_ms_per_batch": round(seq_us * 1e-3, 4),
            "tokens_per_s": round(w.T / (ovl_us * 1e-6), 1),
            "note": f"{steps} batches of {w.T} tokens submitted back to back to MoeOverlap over "
                    f"{n} layers' buffers: each batch's route, dispatch and combine run beside "
                    "another batch's experts; kernels that share the CUs slow each other"}


def time_router(layer, x, w, steps, warmup):
    """The gate from the hidden states, timed alone (the headline step starts from the
    logits): moe_router_logits (x [T][H] . W_router^T -> fp32 [T][E]), and
    moe_router_topk (the same logits consumed by the top-k in one call, routes and
    counts out, logits not kept) next to moe_router_logits + moe_route_topk."""
    import numpy as np
    import torch
    import moe_workloads as mw
    wr = torch.from_numpy(mw.router_weights(w).view(np.int16)).view(torch.bfloat16).cuda()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps * 1e3

    us = timed(lambda: layer.router(x, wr))
    two = timed(lambda: layer.route(layer.router(x, wr)))
    fused = timed(lambda: layer.route_from_hidden(x, wr))
    flops = 2.0 * w.T * w.E * w.H
    nbytes = w.T * w.H * 2 + w.E * w.H * 2 + w.T * w.E * 4
    return {"us": round(us, 2), "TFLOPS": round(flops / (us * 1e-6) / 1e12, 1),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "splits": int(layer.buf.sizes.router_scratch_bytes // (w.T * w.E * 4)),
            "gate_and_topk_us": {"two_calls": round(two, 2), "fused": round(fused, 2)},
            "note": "bf16 MFMA, fp32 accumulation; timed alone (the workload's step starts "
                    "from the logits); fused = moe_router_topk"}


def _median_us(fn, reps, warmup=3):
    """Median device time of fn() in microseconds, one pair of events per call."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    return t[len(t) // 2]


def _rate_us(fn, reps, warmup=3):
    """Mean device time per call of fn() in microseconds over `reps` calls issued
    back to back (one pair of events around all of them): the rate at which the
    stream drains a steady stream of calls, host launch cost included."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def time_graph(layer, x, lg, mode, reps):
    """Whole steps issued back to back, eagerly (one host call per kernel) and as
    replays of the step captured once as a HIP graph (MoeLayer.capture)."""
    eager_us = _rate_us(lambda: layer.forward(x, lg, combine=mode), reps)
    graph = layer.capture(x, lg, combine=mode)
    graph_us = _rate_us(graph.replay, reps)
    del graph
    return eager_us, graph_us


def _bits(a, bf16=True):
    import numpy as np
    import torch
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def time_uniform(packed, steps, warmup):
    """The 12288-token layer with uniform routing (N(0,1) logits, no Zipf bias):
    every expert gets about T*k/E routes, so the expert GEMMs see full tiles; the
    reference case for their MFMA fraction."""
    import torch
    import combine_moe_route_topk_amd as moe
    import moe_workloads as mw
    w = mw.WORKLOADS["layer12288"].scaled(name="layer12288_uniform", zipf=False)
    ro, rs, sp, sl = mw.identity_map(w)
    layer = moe.MoeLayer(moe.geom_of(w), w.gating, torch.from_numpy(sp).cuda(),
                         torch.from_numpy(sl).cuda(), weights=packed, I=w.I)
    x, lg = _bits(mw.hidden(w)), _bits(mw.logits(w))
    ms, per, dist = time_gpu(layer, x, lg, steps, warmup)
    A = algorithmic(w)
    gu = A["gateup_ops"] / (per["gateup"] * 1e-3) / 1e12
    dn = A["down_ops"] / (per["down"] * 1e-3) / 1e12
    del layer
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
            "stages_us": {k: round(v * 1e3, 2) for k, v in per.items()},
            "gateup_TOPS": round(gu, 1), "gateup_frac_int8_peak": round(gu / INT8_PEAK_TOPS, 4),
            "down_TOPS": round(dn, 1), "down_frac_int8_peak": round(dn / INT8_PEAK_TOPS, 4),
            "note": "N(0,1) logits without the Zipf bias: about 384 routes per expert"}


def time_decode96(reps):
    """Decode-size dispatch and combine latency: 96 tokens of one source to 256
    partitions of one expert each (identity experts, INT8 combine to fp32)."""
    import torch
    import combine_moe_route_topk_amd as moe
    import moe_workloads as mw
    w = mw.WORKLOADS["decode96"]
    ro, rs, sp, sl = mw.identity_map(w)
    layer = moe.MoeLayer(moe.geom_of(w), w.gating, torch.from_numpy(sp).cuda(),
                         torch.from_numpy(sl).cuda(), out_dtype=torch.float32)
    x, lg = _bits(mw.hidden(w)), _bits(mw.logits(w))
    layer.route(lg)
    route_us = _median_us(lambda: layer.route(lg), reps)
    disp_us = _median_us(lambda: layer.dispatch(x), reps)
    comb_us = _median_us(lambda: layer.combine("q8"), reps)
    step_us, graph_us = time_graph(layer, x, lg, "q8", reps)
    T, H, k = w.T, w.H, w.k
    db = T * H * 2 + T * k * 4 + T * k * (H + 16) + 3 * T * k * 4 + w.D * w.S * 16
    cb = T * k * (H + 4) + T * k * 8 + T * H * 4
    del layer
    torch.cuda.empty_cache()
    return {"route_us": round(route_us, 2), "dispatch_us": round(disp_us, 2),
            "combine_us": round(comb_us, 2),
            "dispatch_plus_combine_us": round(disp_us + comb_us, 2),
            "step_us": {"eager": round(step_us, 2), "graph": round(graph_us, 2),
                        "note": "route + dispatch + combine issued back to back, mean per "
                                "step: eager (one host call per kernel) and replayed as one "
                                "HIP graph (MoeLayer.capture)"},
            "bytes": {"dispatch": db, "combine": cb},
            "frac_hbm_peak": round((db + cb) / ((disp_us + comb_us) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "latency-bound (about 6.9 MB per call pair, cache-resident); median of "
                    f"{reps} launches each"}


def time_eplb4096(packed, steps, warmup):
    """The 4096-token layer with the redundant-expert plan: the calibration batch is
    routed on the GPU, its per-expert counts (the collect histogram) go to the
    planner (moe_eplb_build_map, 32 redundant slots on partitions 256-287), and the
    step runs through the replica map.  The expert FFN is bound by its weight bytes
    here, so its HBM fraction is the figure to read."""
    import numpy as np
    import torch
    import combine_moe_route_topk_amd as moe
    import moe_workloads as mw
    w = mw.WORKLOADS["eplb4096"]
    bias = torch.from_numpy(mw.zipf_bias(w)).cuda()
    ro, rs, sp, sl = mw.identity_map(w.scaled(P=w.E, D=w.E))
    cal = moe.MoeLayer(moe.geom(w.calib_tokens, w.H, w.E, w.E, w.k, w.E, 1, 1, w.calib_tokens),
                       w.gating, torch.from_numpy(sp).cuda(), torch.from_numpy(sl).cuda(), bias=bias)
    counts = []
    for i in range(w.calib_slices):
        cal.route(_bits(mw.logits(w, i)))
        counts.append(cal.buf.expert_counts.cpu().numpy().astype(np.int64))
    del cal
    primary = np.arange(w.E, dtype=np.int32)
    free = np.r_[np.zeros(w.E), np.ones(w.P - w.E)].astype(np.int32)
    ro, rs, sp, sl, _ = moe.moe_eplb_build_map(np.stack(counts), w.P - w.E, w.D, primary, free)
    layer = moe.MoeLayer(moe.geom_of(w), w.gating, torch.from_numpy(sp).cuda(),
                         torch.from_numpy(sl).cuda(), torch.from_numpy(ro).cuda(),
                         torch.from_numpy(rs).cuda(), bias=bias, weights=packed, I=w.I)
    x, lg = _bits(mw.hidden(w)), _bits(mw.logits(w))
    ms, per, dist = time_gpu(layer, x, lg, steps, warmup)
    active = int((layer.buf.expert_counts.cpu().numpy() > 0).sum())
    R = w.T * w.k
    # FFN bytes the method must move: each routed expert's three INT8 projections
    # once, the message rows in, the INT8 intermediate (codes + scale) out and
    # back, the bf16 return rows out
    wbytes = active * 3 * w.H * w.I
    ffn_bytes = wbytes + R * (w.H + 16) + 2 * R * (w.I + 4) + R * w.H * 2
    ffn_ms = per["gateup"] + per["down"]
    A = algorithmic(w)
    del layer
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
            "stages_us": {k: round(v * 1e3, 2) for k, v in per.items()},
            "active_experts": active, "ffn_bytes": ffn_bytes,
            "ffn_GBps": round(ffn_bytes / (ffn_ms * 1e-3) / 1e9, 1),
            "ffn_frac_hbm_peak": round(ffn_bytes / (ffn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "ffn_TOPS": round((A["gateup_ops"] + A["down_ops"]) / (ffn_ms * 1e-3) / 1e12, 1),
            "note": "replica map planned from four 1024-token calibration slices routed on the "
                    "GPU; HBM-bound on the routed experts' weights"}


def time_twohop46080(reps):
    """The 46080-token disaggregated shape: 160 sources to 288 partitions, the routes
    to partitions 160-287 through relays (A2E: dispatch with the second hop; E2A:
    the relay hop of the returns and the combine).  Synthetic returns."""
    import numpy as np
    import torch
    import combine_moe_route_topk_amd as moe
    import moe_workloads as mw
    w = mw.WORKLOADS["twohop46080"]
    ro, rs, sp, sl = mw.first32_map(w)
    layer = moe.MoeLayer(moe.geom_of(w), w.gating, torch.from_numpy(sp).cuda(),
                         torch.from_numpy(sl).cuda(), torch.from_numpy(ro).cuda(),
                         torch.from_numpy(rs).cuda())
    x, lg = _bits(mw.hidden(w)), _bits(mw.logits(w))
    layer.route(lg)
    layer.buf.ret.zero_()
    a2e_us = _median_us(lambda: layer.dispatch(x), reps)
    e2a_us = _median_us(lambda: layer.combine("bf16"), reps)
    T, H, k = w.T, w.H, w.k
    R = T * k
    n_rel = int((sp[layer.buf.phys.cpu().numpy()] >= w.relays).sum())
    # A2E: read x and the ids, write every message once, the relayed ones twice
    # (second hop: read + write); E2A: the relayed return rows copied through the
    # staging (read + write), the combine's gather and its output
    a2e = T * H * 2 + R * 4 + R * (H + 16) + 2 * n_rel * (H + 16) + 3 * R * 4 + w.D * w.S * 16
    e2a = 2 * n_rel * H * 2 + R * H * 2 + R * 8 + T * H * 2
    del layer
    torch.cuda.empty_cache()
    return {"a2e_us": round(a2e_us, 1), "e2a_us": round(e2a_us, 1), "relayed_routes": n_rel,
            "a2e_bytes": a2e, "e2a_bytes": e2a,
            "a2e_GBps": round(a2e / (a2e_us * 1e-6) / 1e9, 1),
            "e2a_GBps": round(e2a / (e2a_us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round((a2e + e2a) / ((a2e_us + e2a_us) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "note": f"median of {reps} launches each; the pages' A2E 172 us / E2A 193 us are "
                    "cross-chip figures (context only)"}


def attainable(w, reps=5):
    """Attainable rates on this GPU, for context next to the published peaks: a
    plain 1 GiB device copy (HBM); the int8 matrix-core rate with nothing but
    MFMAs in flight (moe_probe_mfma_i8: 8 workgroups of 4 wavefronts per CU, each
    wavefront four independent chains of v_mfma_i32_32x32x32_i8, about as long as
    the gate/up launch); and the vendor library's dense INT8 GEMM (torch._int_mm)
    with the gate/up projection's total ops, i.e. all T*k rows against one
    expert's [2I][H] weights (one B matrix, full reuse)."""
    import torch
    import combine_moe_route_topk_amd as moe
    out = {}
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)

    def best(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return min(ms)

    ms = best(lambda: dst.copy_(src))
    out["copy_GBps"] = round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1)
    # one-direction ceilings: a 1 GiB fill (writes only) and a 1 GiB sum (reads only);
    # the dispatch writes 4x what it reads, the combine reads 8x what it writes
    ms = best(lambda: dst.fill_(2.0))
    out["write_GBps"] = round(COPY_BYTES / (ms * 1e-3) / 1e9, 1)
    ms = best(lambda: src.sum())
    out["read_GBps"] = round(COPY_BYTES / (ms * 1e-3) / 1e9, 1)
    del src, dst
    blocks, iters = 8 * 256, 4096
    probe = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    ms = best(lambda: moe.moe_probe_mfma_i8(blocks, iters, probe))
    mfma_ops = blocks * 4 * iters * 4 * 2 * 32 * 32 * 32
    out["mfma_i8_TOPS"] = round(mfma_ops / (ms * 1e-3) / 1e12, 1)
    out["mfma_i8"] = (f"moe_probe_mfma_i8: {blocks} workgroups x 4 wavefronts x {4 * iters} "
                      f"v_mfma_i32_32x32x32_i8, {ms:.3f} ms")
    del probe
    M, K, N = w.T * w.k, w.H, 2 * w.I
    try:
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda")
        wt = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda")
        ms = best(lambda: torch._int_mm(a, wt.t()))
        out["int8_gemm_TOPS"] = round(2 * M * N * K / (ms * 1e-3) / 1e12, 1)
        out["int8_gemm"] = f"torch._int_mm [{M}x{K}] x [{K}x{N}] (dense, one weight matrix)"
        del a, wt
    except Exception as e:  # the library path is context only
        out["int8_gemm_TOPS"] = None
        out["int8_gemm"] = f"unavailable: {type(e).__name__}"
    torch.cuda.empty_cache()
    return out


def host_cpu():
    """The host's CPU model and shape (sockets x cores per socket x threads per core),
    from lscpu, and the logical CPUs this process may run on."""
    import subprocess
    info = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                info[k.strip()] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    return {"model": info.get("Model name", ""), "sockets": info.get("Socket(s)"),
            "cores_per_socket": info.get("Core(s) per socket"),
            "threads_per_core": info.get("Thread(s) per core"),
            "logical_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(w, budget_s=12.0, threads=None):
    """The oracle, as it stands, on the host cores: route, quantization, dispatch
    layout and messages, and combine over the whole batch; the expert FFN on a
    seeded sample of routes (the hottest expert first), scaled by route count.
    `threads` OpenMP threads (default: every CPU this process may use); the
    oracle's results are the same for any thread count."""
    import numpy as np

    import moe_workloads as mw
    import oracle

    if threads is None:
        threads = len(os.sched_getaffinity(0))
        if os.environ.get("OMP_NUM_THREADS"):
            threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    oracle.set_threads(threads)
    x, lg, bias = mw.hidden(w), mw.logits(w), mw.zipf_bias(w)
    ro, rs, sp, sl = mw.identity_map(w)
    t = {}
    c0 = time.perf_counter()
    ids, sc, tw = oracle.route_topk(lg, w.k, w.gating, bias, logits_bf16=True)
    phys = oracle.eplb_phys(ids, w.LB, w.E)
    t["route"] = time.perf_counter() - c0
    c0 = time.perf_counter()
    q, s = oracle.quant_tokens(x, True)
    lay = oracle.dispatch_layout(w, phys, sp, 1)
    rows = oracle.dispatch_rows(w, q, s, phys, lay["slot_local"], 1)
    t["dispatch"] = time.perf_counter() - c0
    del rows
    rets = np.full((w.T * w.k, w.H), 0x3F80, np.uint16)  # timing does not depend on the values
    ident = np.arange(w.T * w.k, dtype=np.int32).reshape(w.T, w.k)
    c0 = time.perf_counter()
    oracle.combine(rets, ident, tw.astype(np.float32), w.k, w.H, "bf16", True)
    t["combine"] = time.perf_counter() - c0
    del rets
    # expert FFN: seeded sample of routes of one expert at a time, grown to fill the budget
    rng = np.random.default_rng(0)
    logical = sl[phys.ravel()]
    hot = int(np.bincount(logical).argmax())
    n_done, ffn_s, experts = 0, 0.0, []
    spent = sum(t.values())
    n = 16
    while ffn_s < max(2.0, budget_s - spent) and n_done < w.T * w.k:
        e = hot if not experts else int(rng.choice(np.unique(logical)))
        sel = np.nonzero(logical == e)[0]
        sel = rng.choice(sel, min(n, len(sel)), replace=False)
        wgu, sgu, wd, sd = mw.expert_weights(w, e)
        toks = sel // w.k
        c0 = time.perf_counter()
        oracle.expert_ffn(q[toks], s[toks], wgu, sgu, wd, sd)
        ffn_s += time.perf_counter() - c0
        n_done += len(sel)
        experts.append(e)
        n *= 2
    t["ffn"] = ffn_s / n_done * w.T * w.k
    total = sum(t.values())
    return {
        "value": w.T / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "sample": (f"route, quantization, dispatch layout + messages and combine over all "
                   f"{w.T} tokens; expert FFN on {n_done} sampled routes of {len(experts)} "
                   f"experts (hottest first), scaled by route count to {w.T * w.k} routes"),
        "seconds": {k: round(v, 3) for k, v in t.items()},
        "ffn_sample_seconds": round(ffn_s, 3),
    }


def copy_calibration(reps=5):
    """A plain copy of known size (1 GiB fp32 -> 1 GiB), for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) that rocprofv3 reports per dispatch."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                                           "launches": reps}}), flush=True)


def measured_traffic():
    """HBM bytes per launch of the gate/up GEMM from the committed counter summary,
    or None if the kernel source changed since the counters were taken."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    if kv.get("source_sha256") != sha:
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="layer12288")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attainable", action="store_true",
                    help="skip the device-copy and library-GEMM reference rates")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the decode96, eplb4096, twohop46080 and uniform-routing lines")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline step (for counter runs: every launch of a "
                         "kernel then has the headline shape)")
    ap.add_argument("--router-only", action="store_true",
                    help="time only the gate logits (moe_router_logits, moe_router_topk) on "
                         "the workload's hidden states: every gate launch then has that shape")
    ap.add_argument("--config-only", choices=("layer12288_uniform", "eplb4096", "decode96",
                                              "twohop46080", "batch_overlap"),
                    help="time only this workload's line of the configs (for profiling runs: "
                         "every launch then belongs to it); prints {workload, config}")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the 1 GiB copy used to scale rocprofv3 byte counters")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the MoE layer; runs on more than one GPU "
              "are not part of this build (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_workloads as mw
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    w = mw.WORKLOADS[args.workload]
    if args.config_only:
        name = args.config_only
        if name == "decode96":
            r = time_decode96(200)
        elif name == "twohop46080":
            r = time_twohop46080(max(5, args.steps // 5))
        elif name == "batch_overlap":
            layer, x, lg = build_layer(w)
            r = time_batch_overlap(layer, x, lg, w, args.steps, args.warmup)
        else:
            # both take the headline layer's packed expert weights
            layer, x, lg = build_layer(w)
            packed = layer.weights
            del layer, x, lg
            torch.cuda.empty_cache()
            r = (time_uniform if name == "layer12288_uniform" else time_eplb4096)(
                packed, args.steps, args.warmup)
        print(json.dumps({"workload": name, "config": r}), flush=True)
        return
    A = algorithmic(w)
    layer, x, lg = build_layer(w)
    if args.router_only:
        r = time_router(layer, x, w, args.steps, args.warmup)
        log(f"[bench] router logits: {r['us']:.1f} us")
        print(json.dumps({"workload": w.name, "router": r}), flush=True)
        return
    ms, per, dist = time_gpu(layer, x, lg, args.steps, args.warmup)
    log(f"[bench] {ms:.3f} ms/step " + " ".join(f"{k}={v * 1e3:.1f}us" for k, v in per.items()))

    dc_bytes = A["dispatch_bytes"] + A["combine_bytes"]
    dc_ms = per["dispatch"] + per["combine"]
    dc_gbs = dc_bytes / (dc_ms * 1e-3) / 1e9
    gu_tops = A["gateup_ops"] / (per["gateup"] * 1e-3) / 1e12
    dn_tops = A["down_ops"] / (per["down"] * 1e-3) / 1e12
    stages = {
        "route": {"us": per["route"] * 1e3,
                  "GBps": A["route_bytes"] / (per["route"] * 1e-3) / 1e9},
        "dispatch": {"us": per["dispatch"] * 1e3,
                     "GBps": A["dispatch_bytes"] / (per["dispatch"] * 1e-3) / 1e9},
        "gateup": {"us": per["gateup"] * 1e3, "TOPS": gu_tops},
        "down": {"us": per["down"] * 1e3, "TOPS": dn_tops},
        "combine": {"us": per["combine"] * 1e3,
                    "GBps": A["combine_bytes"] / (per["combine"] * 1e-3) / 1e9},
    }
    for v in stages.values():
        for kk in list(v):
            v[kk] = round(v[kk], 2)
    for name in ("route", "dispatch", "combine"):
        stages[name]["frac_hbm_peak"] = round(stages[name]["GBps"] / HBM_PEAK_GBS, 4)
    for name in ("gateup", "down"):
        stages[name]["frac_int8_peak"] = round(stages[name]["TOPS"] / INT8_PEAK_TOPS, 4)
    result = {
        "metric": "MoE dispatch+combine GB/s (% of HBM peak) and MoE-layer tokens/s, T=12288 H=7168 k=8",
        "value": round(w.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "k": w.k, "I": w.I,
                   "sources": f"{w.S}x{w.LB}", "partitions": f"{w.D}x{w.Epp}",
                   "routing": "sigmoid(bf16 logit + log-Zipf(1.1) bias)",
                   "parallelism": "one GPU, virtual partitions"},
        "step_ms": {k: round(v, 4) for k, v in dist.items()},
        "dispatch_combine": {"GBps": round(dc_gbs, 1), "frac_hbm_peak": round(dc_gbs / HBM_PEAK_GBS, 4),
                             "bytes": dc_bytes, "us": round(dc_ms * 1e3, 2)},
        "stages": stages,
        "roofline": {"kernel": "ffn_gemm_kernel<GATEUP> (moe_expert_gateup_q8)",
                     "bound": "mfma", "achieved": round(gu_tops, 1), "peak": INT8_PEAK_TOPS,
                     "unit": "TFLOP/s", "ops": "int8 multiply-adds x 2",
                     "frac": round(gu_tops / INT8_PEAK_TOPS, 4), "traffic": measured_traffic(),
                     "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE)"},
    }
    if args.headline_only:
        print(json.dumps(result), flush=True)
        return
    # the same step with cold caches: 1 GiB written between steps (outside the stages)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    msc, perc, distc = time_gpu(layer, x, lg, max(5, args.steps // 2), args.warmup, flush=flush)
    del flush
    dcc_ms = perc["dispatch"] + perc["combine"]
    result["cold_cache"] = {
        "ms_per_step": round(msc, 4), "tokens_per_s": round(w.T / (msc * 1e-3), 1),
        "step_ms": {k: round(v, 4) for k, v in distc.items()},
        "stages_us": {k: round(v * 1e3, 2) for k, v in perc.items()},
        "dispatch_combine": {"GBps": round(dc_bytes / (dcc_ms * 1e-3) / 1e9, 1),
                             "frac_hbm_peak": round(dc_bytes / (dcc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "note": "a 1 GiB buffer is overwritten before every step (outside the timed stages), "
                "so each step starts with its inputs out of the caches; the headline figures "
                "above are hot-cache (steps back to back)"}
    log(f"[bench] cold caches: {msc:.3f} ms/step")
    # the INT8 return paths (XDS P089), timed the same way, beside the bf16 one
    for mode, note in (("q8blocks", "expert returns quantized to INT8 in the down "
                                    "projection's epilogue, one fp32 scale per 256 columns"),
                       ("q8rows", "token-wise INT8 expert returns: one fp32 scale per row, "
                                  "quantized by moe_quant_returns_q8 after the down "
                                  "projection (the send side of the return path)")):
        ms8, per8, dist8 = time_gpu(layer, x, lg, args.steps, args.warmup, returns=mode)
        log(f"[bench] INT8 returns ({mode}): {ms8:.3f} ms/step " +
            " ".join(f"{k}={v * 1e3:.1f}us" for k, v in per8.items()))
        cb = A["combine_q8_bytes"] if mode == "q8blocks" else \
            w.T * w.k * (w.H + 4) + w.T * w.k * 8 + w.T * w.H * 2
        dc8_bytes = A["dispatch_bytes"] + cb
        dc8_ms = per8["dispatch"] + per8["combine"]
        result["int8_returns" if mode == "q8blocks" else "int8_returns_tokenwise"] = {
            "tokens_per_s": round(w.T / (ms8 * 1e-3), 1), "ms_per_step": round(ms8, 4),
            "stages_us": {k: round(v * 1e3, 2) for k, v in per8.items()},
            "combine_GBps": round(cb / (per8["combine"] * 1e-3) / 1e9, 1),
            "dispatch_combine": {"GBps": round(dc8_bytes / (dc8_ms * 1e-3) / 1e9, 1),
                                 "bytes": dc8_bytes, "us": round(dc8_ms * 1e3, 2)},
            "note": note + "; not the headline configuration (bf16 returns)"}
    # the microbatch pipeline: two halves of the sources on two streams
    result["microbatch_pipeline"] = time_pipeline(layer, x, lg, w, args.steps, args.warmup)
    log(f"[bench] 2-microbatch pipeline: {result['microbatch_pipeline']['ms_per_step']:.3f} ms/step")
    result["batch_overlap"] = time_batch_overlap(layer, x, lg, w, args.steps, args.warmup)
    log(f"[bench] whole batches in flight: {result['batch_overlap']['ms_per_batch']:.3f} ms/batch "
        f"(one at a time {result['batch_overlap']['one_at_a_time_ms_per_batch']:.3f})")
    # whole steps replayed as one captured HIP graph, beside the same steps issued eagerly
    eg_us, gr_us = time_graph(layer, x, lg, "bf16", args.steps)
    result["graph_replay"] = {
        "ms_per_step": round(gr_us * 1e-3, 4), "tokens_per_s": round(w.T / (gr_us * 1e-6), 1),
        "eager_ms_per_step": round(eg_us * 1e-3, 4),
        "note": "MoeLayer.capture: the step captured once, replayed back to back; eager = the "
                "same steps issued back to back without per-stage events"}
    log(f"[bench] graph replay: {gr_us * 1e-3:.3f} ms/step (eager back to back "
        f"{eg_us * 1e-3:.3f})")
    # the gate's logits from the hidden states (bf16 MFMA), timed alone:
    # the headline step starts from the logits, as the workload defines
    result["router"] = time_router(layer, x, w, args.steps, args.warmup)
    log(f"[bench] router logits: {result['router']['us']:.1f} us")
    packed = layer.weights
    del layer, x, lg
    torch.cuda.empty_cache()
    if not args.no_configs:
        # the other workloads, each on its own (their figures are context, not the headline)
        cfg = {}
        cfg["layer12288_uniform"] = time_uniform(packed, args.steps, args.warmup)
        log(f"[bench] uniform routing: {cfg['layer12288_uniform']['ms_per_step']:.3f} ms/step")
        cfg["eplb4096"] = time_eplb4096(packed, args.steps, args.warmup)
        log(f"[bench] eplb4096: {cfg['eplb4096']['ms_per_step']:.3f} ms/step")
        del packed
        torch.cuda.empty_cache()
        cfg["decode96"] = time_decode96(200)
        log(f"[bench] decode96: dispatch {cfg['decode96']['dispatch_us']} us, "
            f"combine {cfg['decode96']['combine_us']} us, step {cfg['decode96']['step_us']['eager']} "
            f"us eager / {cfg['decode96']['step_us']['graph']} us graph")
        cfg["twohop46080"] = time_twohop46080(max(5, args.steps // 5))
        log(f"[bench] twohop46080: A2E {cfg['twohop46080']['a2e_us']} us, "
            f"E2A {cfg['twohop46080']['e2a_us']} us")
        result["configs"] = cfg
    else:
        del packed
    if not args.no_attainable:
        log("[bench] attainable rates: device copy, MFMA-only int8 rate, library INT8 GEMM")
        att = attainable(w)
        result["attainable"] = att
        result["roofline"]["frac_of_mfma_attainable"] = round(gu_tops / att["mfma_i8_TOPS"], 4)
        if att.get("int8_gemm_TOPS"):
            result["roofline"]["frac_of_attainable"] = round(gu_tops / att["int8_gemm_TOPS"], 4)
        result["dispatch_combine"]["frac_of_copy"] = round(dc_gbs / att["copy_GBps"], 4)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample: all threads, then one")
        allc = cpu_baseline(w, args.cpu_budget)
        one = cpu_baseline(w, args.cpu_budget * 0.75, threads=1)
        allc["modes"] = {f"{allc['cores']}_threads": {k: allc[k] for k in ("value", "seconds")},
                         "1_thread": {k: one[k] for k in ("value", "seconds", "sample")}}
        allc["host"] = host_cpu()
        result["cpu_baseline"] = allc
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
