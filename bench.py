#!/usr/bin/env python3
"""Benchmark of the routed-attention layer on one MI355X.

One step = one forward pass of the layer's hot path over one batch of
synthetic input already resident in HBM: rt_route (normalise + score + top-w)
-> rt_routed_attn (in-cluster causal attention + scatter-add) ->
rt_centroid_update (EMA) for the routed heads, plus rt_local_attn for the
local heads.  The default workload is the long-sequence layer: batch 1, 8
routed heads (k=64 centroids, w=128) and 4 local heads (window 512), n=8192,
d=128, bfloat16.

The steps are launched eagerly on one stream (--graph replays a captured HIP
graph of the step instead).  Prints one JSON line: the metric and its value,
the per-call timings, the roofline of the dominant kernel and, beside them, the
fp64 oracle timed on the host cores on full steps of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthetic as S  # noqa: E402

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s

# HBM traffic of the in-cluster attention kernel at the long workload, from two rocprofv3
# --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by the same counter's
# reading for a plain 256 MiB device copy in the same run (--copy-calibration 256).  Valid only
# for the kernel sources with this digest: after any change the bench reports traffic null.
CLUSTER_TRAFFIC = {
    "workload": "long",
    "sources": ["content_sparse_attention_unit_amd/csrc/cluster_attn.hip",
                "content_sparse_attention_unit_amd/csrc/rt_common.hpp"],
    "sha256": "e63b17b1c985c28d854e13173c5f455a41fc1fbc642f25c8d2d5c8d8f41a4320",
    "fetch_kib": 11013.253, "write_kib": 28480.546,
    "fetch_scale": 262144.0 / 131088.438, "write_scale": 262144.0 / 262144.0,
}


def measured_traffic(rec, workload):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch, or None when the kernel's
    sources have changed since the counters were taken (or the workload differs)."""
    import hashlib
    if workload != rec["workload"] or not rec["sha256"]:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec["sha256"]:
        return None
    return 1024.0 * (rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"])

# GPU clock cycles per microsecond of torch's spin kernel (torch.cuda._sleep),
# calibrated at start-up.
_SPIN_CYCLES_PER_US = 2370.0


def calibrate_gpu_ahead():
    global _SPIN_CYCLES_PER_US
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    a.record()
    torch.cuda._sleep(400000)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3
    if us > 0:
        _SPIN_CYCLES_PER_US = 400000.0 / us


def gpu_ahead(us):
    """Keep the current stream busy for about `us` microseconds, so that the host
    has enqueued the calls timed next before the GPU reaches them: back-to-back
    and per-call times then measure the GPU, not the host's launch rate (the
    binding's marshalling is several microseconds a call)."""
    torch.cuda._sleep(max(1, int(us * _SPIN_CYCLES_PER_US)))


WORKLOADS = {
    "long": "long: B=1, 8 routed heads (k=64, w=128) + 4 local heads (window 512), "
            "n=8192, d=128, bf16, causal, shared QK, EMA lambda=0.999",
    "mixed": "mixed: B=2, 8 routed heads (k=64, w=64) + 8 local heads (window 256), "
             "n=4096, d=64, bf16",
    "routed": "routed: B=4, 8 routed heads (k=32, w=32), n=1024, d=64, bf16",
    "tiny": "tiny: B=1, 1 routed head (k=4, w=16), n=64, d=16, float32",
    "stress": "stress: B=1, 8 routed heads (k=128, w=256) + 8 local (window 256), "
              "n=32768, d=64, bf16, 10% skewed tokens, forward + in-cluster backward",
}


def dev(t):
    st = t.storage
    if t.dtype == "bf16":
        return torch.from_numpy(st.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(st).cuda()


def algorithmic(cfg):
    """Algorithmic HBM bytes and flops per step, per call (minimum traffic:
    every input read once, every output written once)."""
    B, R, L, n, d, k, w = cfg.B, cfg.R, cfg.L, cfg.n, cfg.d, cfg.k, cfg.w
    e = 2 if cfg.dtype == "bf16" else 4
    tok = B * R * n * d * e                      # one [B,R,n,d] token tensor
    route_bytes = tok + R * k * d * 4 + B * R * n * 4 + B * R * k * w * 4
    attn_bytes = 2 * tok + tok + B * R * k * w * 4 + B * R * n * 4   # qk, v gathered; out; idx; inv
    ema_bytes = tok + B * R * k * w * 4 + 2 * R * k * d * 4 + B * R * n * 4
    local_bytes = 4 * B * L * n * d * e
    attn_flops_tile = 4.0 * B * R * k * w * w * d           # QK^T and PV over full w x w tiles
    attn_flops_causal = 4.0 * B * R * k * (w * (w + 1) / 2) * d
    route_flops = 2.0 * B * R * n * k * d
    lw = min(cfg.window, n)
    local_flops = 4.0 * B * L * d * (lw * (lw + 1) / 2 + max(0, n - lw) * lw)
    # backward: qk, v, dO gathered once, lse/idx; dq_hat, dk_hat, dv written once in fp32;
    # five w x w x d products per cluster (S, dP, dV, dQ, dK)
    bwd_bytes = 3 * tok + 2 * B * R * k * w * 4 + 3 * B * R * n * d * 4
    bwd_flops_tile = 10.0 * B * R * k * w * w * d
    bwd_flops_causal = 10.0 * B * R * k * (w * (w + 1) / 2) * d
    # the scatter's own reads (membership bits); the rows it completes are
    # counted with the attention's output
    scatter_bytes = B * R * n * ((k + 31) // 32) * 4
    return dict(bwd_bytes=bwd_bytes, bwd_flops_tile=bwd_flops_tile,
                bwd_flops_causal=bwd_flops_causal, scatter_bytes=scatter_bytes,
                route_bytes=route_bytes, attn_bytes=attn_bytes, ema_bytes=ema_bytes,
                local_bytes=local_bytes, attn_flops_tile=attn_flops_tile,
                attn_flops_causal=attn_flops_causal, route_flops=route_flops,
                local_flops=local_flops)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_routed_step(oracle, cfg, inp, scale, threads):
    """The routed heads' step on the oracle: route, routed attention and the
    centroid update (and the in-cluster backward for the stress workload)."""
    qk = inp["qk"].value
    _, idx, _, _ = oracle.route(qk, inp["mu"], cfg.w, nthreads=threads)
    oracle.routed_attn(qk, qk, inp["v"].value, idx, scale, True, True, nthreads=threads)
    oracle.centroid_update(inp["mu"], qk, qk, idx, cfg.lam)
    if cfg.backward:
        oracle.routed_attn_bwd(qk, qk, inp["v"].value, idx, inp["dout"].value, scale, True,
                               nthreads=threads)


def cpu_baseline(cfg, inp, scale, min_seconds=10.0):
    """The oracle (fp64, as written: never tuned) on the routed step of the
    workload, on the host cores, repeated until about `min_seconds` have passed;
    plus single-thread times of one step of the tiny and routed workloads."""
    import oracle
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle_routed_step(oracle, cfg, inp, scale, threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    single = {}
    for name in ("tiny", "routed"):
        c = S.CONFIGS[name]
        ci = S.make_inputs(c)
        t1 = time.perf_counter()
        oracle_routed_step(oracle, c, ci, 1.0 / math.sqrt(c.d), 1)
        single[name] = time.perf_counter() - t1
    return {"value": reps * cfg.B * cfg.n / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "seconds": dt, "steps": reps, "cpu_model": cpu_model(),
            "single_thread_s_per_step": single,
            "sample": f"{reps} routed step(s) of the {cfg.name} workload (route, routed "
                      f"attention, centroid update{', in-cluster backward' if cfg.backward else ''}"
                      f"; the metric's step), fp64, {threads} threads; single-thread: one step "
                      f"of the tiny and routed workloads"}


def time_stack(rt, sc, reps=5, use_graph=False):
    """The stack of sc.layers layers (x -> in_proj -> route -> routed attention
    (+member sums) -> centroid update -> local attention -> out_proj, residual in
    place), launched eagerly on one stream or captured as one HIP graph;
    returns timings and rates."""
    B, n, dm, d, R, L, k, w = sc.B, sc.n, sc.dm, sc.d, sc.R, sc.L, sc.k, sc.w
    scale = 1.0 / math.sqrt(d)
    x0 = dev(S.stack_x(sc))
    layers = []
    for l in range(sc.layers):
        lw = S.stack_layer(sc, l)
        layers.append((dev(lw["w_in"]), dev(lw["w_o"]),
                       torch.from_numpy(lw["mu"].astype(np.float32)).cuda()))
    bf = dict(dtype=torch.bfloat16, device="cuda")
    qk, v = torch.empty((B, R, n, d), **bf), torch.empty((B, R, n, d), **bf)
    ql, kl, vl = (torch.empty((B, L, n, d), **bf) for _ in range(3))
    o_r, o_l = torch.empty((B, R, n, d), **bf), torch.empty((B, L, n, d), **bf)
    inv = torch.empty((B, R, n), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, R, k, w), dtype=torch.int32, device="cuda")
    mask = torch.empty((B, R, n, rt.mask_words(k)), dtype=torch.int32, device="cuda")
    sum_q = torch.empty((B, R, k, d), dtype=torch.float32, device="cuda")
    ws_r = torch.empty(rt.workspace_bytes("route", B, R, n, d, k, w), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(rt.workspace_bytes("routed_attn_update", B, R, n, d, k, w),
                       dtype=torch.uint8, device="cuda")
    xs = (torch.empty_like(x0), torch.empty_like(x0))   # layer outputs, alternating

    def forward():
        x = x0                                            # every forward starts from x0
        for l, (w_in, w_o, mu) in enumerate(layers):
            rt.in_proj(x, w_in, R, L, d, out=(qk, v, ql, kl, vl))
            rt.route(qk, mu, w, out=(inv, idx, mask), ws=ws_r)
            rt.routed_attn_update_(qk, qk, v, idx, inv, inv, mu, sc.lam, scale=scale, mask=mask,
                                   out=o_r, ws=ws_a)
            rt.local_attn(ql, kl, vl, sc.window, scale=scale, out=o_l)
            rt.out_proj(o_r, o_l, w_o, x=x, out=xs[l % 2])
            x = xs[l % 2]
        return x

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        x = forward()
        torch.cuda.synchronize()
        finite = bool(torch.isfinite(x.float()).all())
        run = forward
        if use_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                forward()
            run = graph.replay
        torch.cuda.synchronize()
        for _ in range(2):
            run()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
    # the two projections alone (per call, back to back)
    w_in, w_o, _ = layers[0]
    per = {}
    flops_in = 2.0 * B * n * dm * (2 * R + 3 * L) * d
    flops_out = 2.0 * B * n * (R + L) * d * dm
    y = torch.empty((B, n, dm), **bf)
    with torch.cuda.stream(stream):
        for name, fn in (("rt_in_proj", lambda: rt.in_proj(x, w_in, R, L, d, out=(qk, v, ql, kl, vl))),
                         ("rt_out_proj", lambda: rt.out_proj(o_r, o_l, w_o, x=x, out=y))):
            for _ in range(3):
                fn()
            a.record(stream)
            for _ in range(20):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            per[name] = a.elapsed_time(b) / 20
    bwd = time_layer_bwd(rt, sc, stream, layers[0], x0, dict(qk=qk, v=v, ql=ql, kl=kl, vl=vl,
                                                          inv=inv, idx=idx, mask=mask, o_r=o_r,
                                                          o_l=o_l, ws_r=ws_r, ws_a=ws_a))
    return {"layers": sc.layers, "d_model": dm, "ms_per_forward": ms, "graph": use_graph,
            "backward": bwd,
            "tokens_per_s": B * n / (ms * 1e-3), "us_per_layer": ms * 1e3 / sc.layers,
            "finite": finite,
            "proj_ms": per,
            "proj_tflops": {"rt_in_proj": flops_in / (per["rt_in_proj"] * 1e-3) / 1e12,
                            "rt_out_proj": flops_out / (per["rt_out_proj"] * 1e-3) / 1e12},
            "proj_mfma_frac": {"rt_in_proj": flops_in / (per["rt_in_proj"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                               "rt_out_proj": flops_out / (per["rt_out_proj"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
            "workload": f"{sc.layers}-layer stack, d_model={dm}, {R} routed + {L} local heads of "
                        f"{d}, n={n}, B={B}, random-init weights N(0, 1/fan_in)"}


def time_layer_bwd(rt, sc, stream, layer, x0, t, reps=10):
    """The layer's backward at the stack's shapes (one layer, membership held
    fixed): rt_out_proj_bwd -> rt_routed_attn_bwd + rt_normalize_bwd on the
    routed heads, rt_local_attn_bwd on the local heads -> rt_in_proj_bwd.  Each
    call timed back to back (HIP events); the sum is one layer's backward."""
    B, n, dm, d, R, L, k, w = sc.B, sc.n, sc.dm, sc.d, sc.R, sc.L, sc.k, sc.w
    scale = 1.0 / math.sqrt(d)
    w_in, w_o, mu = layer
    f32 = dict(dtype=torch.float32, device="cuda")
    bf = dict(dtype=torch.bfloat16, device="cuda")
    dy = dev(S.normal_tensor(1000 * sc.cfg_id + 60, (B, n, dm), "bf16"))
    lse = torch.empty((B, R, k, w), **f32)
    do_r, do_l = torch.empty((B, R, n, d), **bf), torch.empty((B, L, n, d), **bf)
    dw_o = torch.empty((dm, (R + L) * d), **f32)
    dqh, dv, dqk = (torch.empty((B, R, n, d), **f32) for _ in range(3))
    dq_l, dk_l, dv_l = (torch.empty((B, L, n, d), **f32) for _ in range(3))
    dx = torch.empty((B, n, dm), **f32)
    dw_in = torch.empty(((2 * R + 3 * L) * d, dm), **f32)
    ws_b = torch.empty(rt.workspace_bytes("routed_attn_bwd", B, R, n, d, k, w), dtype=torch.uint8,
                       device="cuda")
    ws_l = torch.empty(rt.workspace_bytes("local_attn_bwd", B, L, n, d, 1, 1), dtype=torch.uint8,
                       device="cuda")
    ws_p = rt.proj_bwd_workspace(B, n, dm, d, R, L, "cuda")    # split weight gradients
    T, NO, NC = B * n, (R + L) * d, (2 * R + 3 * L) * d
    band = L * B * (n * sc.window - sc.window * (sc.window - 1) / 2)   # (query, key) pairs
    calls = {
        "rt_out_proj_bwd": (lambda: rt.out_proj_bwd(dy, t["o_r"], t["o_l"], w_o,
                                                    out=(do_r, do_l, dw_o), ws=ws_p),
                            2 * 2.0 * T * dm * NO),
        "rt_routed_attn_bwd": (lambda: rt.routed_attn_bwd(t["qk"], t["qk"], t["v"], t["idx"], lse,
                                                          do_r, t["inv"], t["inv"], scale=scale,
                                                          mask=t["mask"], out=(dqh, None, dv),
                                                          ws=ws_b, sum_qk=True),
                               10.0 * B * R * k * (w * (w + 1) / 2) * d),
        "rt_normalize_bwd": (lambda: rt.normalize_bwd(t["qk"], t["inv"], dqh, None, out=dqk), 0.0),
        "rt_local_attn_bwd": (lambda: rt.local_attn_bwd(t["ql"], t["kl"], t["vl"], do_l,
                                                        sc.window, scale=scale,
                                                        out=(dq_l, dk_l, dv_l), ws=ws_l),
                              10.0 * band * d),
        "rt_in_proj_bwd": (lambda: rt.in_proj_bwd(x0, w_in, dqk, dv, dq_l, dk_l, dv_l, dres=dy,
                                                  out=(dx, dw_in), ws=ws_p),
                           2 * 2.0 * T * NC * dm),
    }
    per, tfl = {}, {}
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        # forward state of one layer (with the softmax statistics the routed backward needs)
        rt.in_proj(x0, w_in, R, L, d, out=(t["qk"], t["v"], t["ql"], t["kl"], t["vl"]))
        rt.route(t["qk"], mu, w, out=(t["inv"], t["idx"], t["mask"]), ws=t["ws_r"])
        rt.routed_attn(t["qk"], t["qk"], t["v"], t["idx"], t["inv"], t["inv"], scale=scale,
                       mask=t["mask"], out=t["o_r"], lse=lse, ws=t["ws_a"])
        rt.local_attn(t["ql"], t["kl"], t["vl"], sc.window, scale=scale, out=t["o_l"])
        for name, (fn, flops) in calls.items():
            for _ in range(3):
                fn()
            gpu_ahead(30 * reps)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            per[name] = a.elapsed_time(b) / reps
            if flops:
                tfl[name] = flops / (per[name] * 1e-3) / 1e12
    finite = all(bool(torch.isfinite(g).all()) for g in (dx, dw_in, dw_o))
    total = sum(per.values())
    return {"ms_per_layer": total, "tokens_per_s": B * n / (total * 1e-3), "per_call_ms": per,
            "tflops": tfl, "finite": finite,
            "note": "one layer's backward (membership fixed), the sum of back-to-back call "
                    "times; tflops on the algorithmic products (routed and local attention: "
                    "5 products per visible pair; the routed backward returns dq_hat + dk_hat)"}


def time_variants(rt, cfg, inp, reps=20):
    """The variants at the workload's shapes: blocked local attention (blocks of
    the window, one block of look-back) on the local heads, partition-style
    routing and the nearest-centroid update on the routed heads."""
    B, R, L, n, d, k = cfg.B, cfg.R, cfg.L, cfg.n, cfg.d, cfg.k
    scale = 1.0 / math.sqrt(d)
    qk = dev(inp["qk"])
    ql, kl, vl = dev(inp["q_local"]), dev(inp["k_local"]), dev(inp["v_local"])
    mu = torch.from_numpy(inp["mu"].astype(np.float32)).cuda()
    out_l = torch.empty_like(ql)
    inv = torch.empty((B, R, n), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, R, k, n // k), dtype=torch.int32, device="cuda")
    ws_p = torch.empty(rt.workspace_bytes("route_partition", B, R, n, d, k, 1), dtype=torch.uint8,
                       device="cuda")
    ws_e = torch.empty(rt.workspace_bytes("centroid_update_argmax", B, R, n, d, k, 1),
                       dtype=torch.uint8, device="cuda")
    # separately routed queries and keys: a distinct key tensor of the routed heads' shape
    kd = dev(S.normal_tensor(5_000_000, (B, R, n, d), "bf16"))
    vd = dev(inp["v"])
    q_inv, idx_q, q_mask = rt.route(qk, mu, cfg.w, want_mask=True)
    k_inv, idx_k = rt.route(kd, mu, cfg.w)
    out_s = torch.empty_like(qk)
    ws_s = torch.empty(rt.workspace_bytes("routed_attn", B, R, n, d, k, cfg.w), dtype=torch.uint8,
                       device="cuda")
    # the Jensen-Shannon diagnostic: routed head h against local head h (the first L heads)
    qk_js = qk[:, :L].contiguous()
    inv_js, idx_js = rt.route(qk_js, mu[:L].contiguous(), cfg.w)
    js_out = torch.empty((B, L, k, cfg.w), dtype=torch.float32, device="cuda")
    ws_js = torch.empty(rt.workspace_bytes("attn_js", B, L, n, d, k, cfg.w), dtype=torch.uint8,
                        device="cuda")
    calls = {
        "rt_attn_js": lambda: rt.attn_js(qk_js, inv_js, idx_js, ql, kl, cfg.window, scale_r=scale,
                                         scale_l=scale, out=js_out, ws=ws_js),
        "rt_local_attn_blocked": lambda: rt.local_attn_blocked(ql, kl, vl, cfg.window, 1,
                                                               scale=scale, out=out_l),
        "rt_routed_attn_split": lambda: rt.routed_attn_split(qk, kd, vd, idx_q, idx_k, q_inv,
                                                             k_inv, scale=scale, q_mask=q_mask,
                                                             out=out_s, ws=ws_s),
        "rt_route_partition": lambda: rt.route_partition(qk, mu, out=(inv, idx), ws=ws_p),
        "rt_centroid_update_argmax": lambda: rt.centroid_update_argmax_(mu, qk, lam=cfg.lam,
                                                                        ws=ws_e),
    }
    per = {}
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, fn in calls.items():
        for _ in range(3):
            fn()
        gpu_ahead(30 * reps)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        per[name] = a.elapsed_time(b) / reps
    return {"per_call_ms": per,
            "note": f"blocked local: blocks of {cfg.window}, one block of look-back, {L} heads; "
                    f"partition: n/k = {n // k} tokens a cluster, {R} heads; nearest-centroid "
                    f"update: shared q/k, {R} heads; split routing: distinct q and k each "
                    f"routed (k={k}, w={cfg.w}), {R} heads, non-causal; JS diagnostic: "
                    f"{L} routed heads against the {L} local heads, incl. the local pass "
                    f"for their denominators",
            "js_mean": float(js_out.mean())}


def time_decode(rt, cfg, inp, group=16, reps=20):
    """Incremental decode after a prefill of the workload's n tokens: caches
    filled from the prefill's routing, then steps of one new token per
    sequence (the routed step on the routed heads and, concurrently on a second
    stream, the local step on the local heads), captured as HIP graphs of
    `group` consecutive steps."""
    B, R, L, n, d, k, w = cfg.B, cfg.R, cfg.L, cfg.n, cfg.d, cfg.k, cfg.w
    scale = 1.0 / math.sqrt(d)
    qk, v = dev(inp["qk"]), dev(inp["v"])
    kl, vl = dev(inp["k_local"]), dev(inp["v_local"])
    mu = torch.from_numpy(inp["mu"].astype(np.float32)).cuda()
    inv, idx = rt.route(qk, mu, w)
    cap = w + group * (2 * reps + 8)
    cache = rt.decode_fill(qk, v, inv, idx, cap)
    rk, rv = rt.decode_ring_fill(kl, vl, cfg.window)
    new = [dev(S.normal_tensor(4_000_000 + i, (group, B, H_, d), "bf16"))
           for i, H_ in enumerate((R, R, L, L, L))]
    out_r = torch.empty((group, B, R, d), dtype=torch.bfloat16, device="cuda")
    lab = torch.empty((group, B, R), dtype=torch.int32, device="cuda")
    out_l = torch.empty((group, B, L, d), dtype=torch.bfloat16, device="cuda")

    def routed(g):
        rt.decode_routed(cache, new[0][g], new[1][g], n + g, mu, scale=scale, out=out_r[g],
                         label=lab[g])

    def local(g):
        rt.decode_local(rk, rv, new[2][g], new[3][g], new[4][g], n + g, scale=scale,
                        out=out_l[g])

    stream, side = torch.cuda.Stream(), torch.cuda.Stream()

    def step(g):
        """Both kinds of heads of one token: the local heads on a second stream."""
        side.wait_stream(stream)
        routed(g)
        with torch.cuda.stream(side):
            local(g)
        stream.wait_stream(side)

    parts = {"routed": routed, "local": local, "step": step}
    per = {}
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        for name, fn in parts.items():
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for g in range(group):
                    fn(g)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps // 2):
                graph.replay()
            b.record(stream)
            torch.cuda.synchronize()
            per[name] = a.elapsed_time(b) / (reps // 2) / group
    assert int(cache["len"].max()) <= cap and bool((lab >= 0).all()), "decode cache overflow"
    return {"ms_per_token_step": per["step"], "tokens_per_s": B / (per["step"] * 1e-3),
            "per_call_ms": {"rt_decode_routed": per["routed"], "rt_decode_local": per["local"]},
            "note": f"after a prefill of {n} tokens: {R} routed heads (k={k} caches of {w}+ "
                    f"entries), {L} local heads (window {cfg.window}) on a second stream; graphs of "
                    f"{group} steps"}


def sweep_configs(only=None):
    """The long layer's shape (B=1, 8 routed + 4 local heads of width 128, window
    512) at n = 1K .. 64K with k = sqrt(n) rounded down to a power of two and
    w = n/k (``only``: the subset of n to keep)."""
    out = []
    for i, lg in enumerate(range(10, 17)):
        n = 1 << lg
        if only and n not in only:
            continue
        k = 1 << (lg // 2)
        out.append(S.Config(80 + i, f"sweep_n{n}", "bf16", 1, 8, 4, n, 128, k, n // k, 512))
    return out


def run_sweep(rt, reps=20, only=None):
    """Per-call times of the layer's entry points across sequence lengths, and
    the fitted growth of the routed heads' time with n (the pages' O(n^1.5 d)
    at k = sqrt(n)) and the routed/local ratio (the pages' ~1.7x on TPUv3)."""
    pts = []
    for cfg in sweep_configs(only):
        inp = S.make_inputs(cfg)
        B, R, n, d, k, w = cfg.B, cfg.R, cfg.n, cfg.d, cfg.k, cfg.w
        scale = 1.0 / math.sqrt(d)
        qk, v = dev(inp["qk"]), dev(inp["v"])
        ql, kl, vl = dev(inp["q_local"]), dev(inp["k_local"]), dev(inp["v_local"])
        mu = torch.from_numpy(inp["mu"].astype(np.float32)).cuda()
        del inp
        inv = torch.empty((B, R, n), dtype=torch.float32, device="cuda")
        idx = torch.empty((B, R, k, w), dtype=torch.int32, device="cuda")
        mask = torch.empty((B, R, n, rt.mask_words(k)), dtype=torch.int32, device="cuda")
        sum_q = torch.empty((B, R, k, d), dtype=torch.float32, device="cuda")
        out, out_l = torch.empty_like(qk), torch.empty_like(ql)
        ws_r = torch.empty(rt.workspace_bytes("route", B, R, n, d, k, w), dtype=torch.uint8,
                           device="cuda")
        ws_a = torch.empty(rt.workspace_bytes("routed_attn", B, R, n, d, k, w), dtype=torch.uint8,
                           device="cuda")
        calls = {
            "rt_route": lambda: rt.route(qk, mu, w, out=(inv, idx, mask), ws=ws_r),
            "rt_routed_attn": lambda: rt.routed_attn(qk, qk, v, idx, inv, inv, scale=scale,
                                                     mask=mask, sums=(sum_q, None), out=out,
                                                     ws=ws_a),
            "rt_centroid_update_sums": lambda: rt.centroid_update_sums_(mu, sum_q, cfg.lam),
            "rt_local_attn": lambda: rt.local_attn(ql, kl, vl, cfg.window, scale=scale, out=out_l),
        }
        us = {}
        for name, fn in calls.items():
            for _ in range(3):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            gpu_ahead(30 * reps)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            us[name] = a.elapsed_time(b) / reps * 1e3
        routed = us["rt_route"] + us["rt_routed_attn"] + us["rt_centroid_update_sums"]
        pts.append({"n": n, "k": k, "w": w, "us": us, "routed_us": routed,
                    "routed_over_local": routed / us["rt_local_attn"],
                    "routed_tokens_per_s": B * n / (routed * 1e-6),
                    "routed_gflop": (6.0 * n * k * d + 4.0 * k * w * w * d) * R * B / 1e9})
        del qk, v, ql, kl, vl, ws_r, ws_a, out, out_l
        torch.cuda.empty_cache()
    if len(pts) < 3:
        return {"metric": "routed-attention call times vs n at k = sqrt(n) (long layer shape)",
                "points": pts}
    ln = np.log([p["n"] for p in pts])
    fit = lambda ys: float(np.polyfit(ln, np.log(ys), 1)[0])
    big = [p for p in pts if p["n"] >= 8192]
    lnb = np.log([p["n"] for p in big])
    return {"metric": "routed-attention call times vs n at k = sqrt(n) (long layer shape)",
            "points": pts,
            "exponent_routed_time_all": fit([p["routed_us"] for p in pts]),
            "exponent_routed_time_n_ge_8192": float(np.polyfit(lnb, np.log([p["routed_us"] for p in big]), 1)[0]),
            "exponent_routed_flops": fit([p["routed_gflop"] for p in pts]),
            "exponent_local_time": fit([p["us"]["rt_local_attn"] for p in pts])}


def event_stats(fn, reps, stream, flush=None):
    """p10/p50/p90/mean (ms) of `reps` calls of fn(), each bracketed by its own
    HIP event pair on `stream` (back to back, so warm); with `flush` (cold) a
    write of that buffer (512 MB: beyond the 256 MB MALL) precedes every call,
    outside its events."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        if flush is not None:
            flush.fill_(1.0)
        gpu_ahead(40)
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return {"p10": float(np.percentile(t, 10)), "p50": float(np.percentile(t, 50)),
            "p90": float(np.percentile(t, 90)), "mean": float(t.mean()), "reps": reps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long", choices=sorted(WORKLOADS))
    ap.add_argument("--reps", type=int, default=200, help="calls per entry point for the "
                    "p10/p50/p90 timing, warm and cold")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="skip timing the 22-layer stack of "
                    "the long workload (reported apart from the per-layer metric)")
    ap.add_argument("--no-extras", action="store_true", help="skip timing the variants and the "
                    "decode steps of the long workload (reported apart from the metric)")
    ap.add_argument("--graph", action="store_true", help="replay a captured HIP graph of the "
                    "step (and of the stack) instead of launching eagerly on one stream; graph "
                    "replay measured slower here")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly (the default)")
    ap.add_argument("--concurrent-local", action="store_true", help="in the whole-layer step, "
                    "run the local heads concurrently on a second stream")
    ap.add_argument("--sweep", action="store_true", help="instead of the benchmark step, time "
                    "the entry points at n = 1K..64K with k = sqrt(n) and print that as one JSON "
                    "line")
    ap.add_argument("--sweep-n", default="", help="with --sweep: comma-separated subset of the "
                    "lengths (powers of two, 1024 .. 65536)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before timing, copy a MIB-mebibyte device buffer once (a plain copy "
                    "of known size that scales the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs and is measured on one GPU; --gpus must be 1 "
                                   "(no sharding or collectives are implemented)"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)

    import content_sparse_attention_unit_amd as rt
    rt._load()
    calibrate_gpu_ahead()

    if args.sweep:
        only = {int(x) for x in args.sweep_n.split(",") if x}
        print(json.dumps(run_sweep(rt, only=only)), flush=True)
        return

    cfg = S.CONFIGS[args.workload]
    inp = S.make_inputs(cfg)
    scale = 1.0 / math.sqrt(cfg.d)
    qk, v = dev(inp["qk"]), dev(inp["v"])
    mu0 = torch.from_numpy(inp["mu"].astype(np.float32)).cuda()
    mu = mu0.clone()
    B, R, n, d, k, w = cfg.B, cfg.R, cfg.n, cfg.d, cfg.k, cfg.w
    f32 = dict(dtype=torch.float32, device="cuda")
    inv = torch.empty((B, R, n), **f32)
    idx = torch.empty((B, R, k, w), dtype=torch.int32, device="cuda")
    mask = torch.empty((B, R, n, rt.mask_words(k)), dtype=torch.int32, device="cuda")
    sum_q = torch.empty((B, R, k, d), **f32)
    out = torch.empty_like(qk)
    ws_route = torch.empty(rt.workspace_bytes("route", B, R, n, d, k, w), dtype=torch.uint8,
                           device="cuda")
    ws_attn = torch.empty(rt.workspace_bytes("routed_attn", B, R, n, d, k, w), dtype=torch.uint8,
                          device="cuda")
    ws_upd = torch.empty(rt.workspace_bytes("routed_attn_update", B, R, n, d, k, w),
                         dtype=torch.uint8, device="cuda")
    if cfg.L > 0:
        ql, kl, vl = dev(inp["q_local"]), dev(inp["k_local"]), dev(inp["v_local"])
        out_l = torch.empty_like(ql)
    lse = None
    if cfg.backward:
        # the forward keeps its softmax statistics; the backward takes a seeded dO
        lse = torch.empty((B, R, k, w), **f32)
        dout = dev(inp["dout"])
        # shared q/k: the backward returns dq_hat + dk_hat (what the normalisation's
        # gradient consumes) and dv
        grads = (torch.empty((B, R, n, d), **f32), None, torch.empty((B, R, n, d), **f32))
        ws_bwd = torch.empty(rt.workspace_bytes("routed_attn_bwd", B, R, n, d, k, w),
                             dtype=torch.uint8, device="cuda")

    def do_route():
        rt.route(qk, mu, w, out=(inv, idx, mask), ws=ws_route)

    def do_cluster():
        rt.cluster_attn(qk, qk, v, idx, inv, inv, mask, scale=scale, out=out, lse=lse,
                        sums=(sum_q, None), ws=ws_attn)

    def do_scatter_update():
        rt.scatter_rows(mask, out, ws_attn, k, w, in_dtype=qk.dtype, mu=mu, sum_q=sum_q,
                        lam=cfg.lam)

    def do_scatter():
        rt.scatter_rows(mask, out, ws_attn, k, w, in_dtype=qk.dtype)

    def do_attn_update():
        """Both stages in one call (the same two kernels)."""
        rt.routed_attn_update_(qk, qk, v, idx, inv, inv, mu, cfg.lam, scale=scale, mask=mask,
                               out=out, lse=lse, ws=ws_upd)

    def do_bwd():
        rt.routed_attn_bwd(qk, qk, v, idx, lse, dout, inv, inv, scale=scale, mask=mask,
                           out=grads, ws=ws_bwd, sum_qk=True)

    def do_local():
        rt.local_attn(ql, kl, vl, cfg.window, scale=scale, out=out_l)

    stream = torch.cuda.Stream()
    side = torch.cuda.Stream()          # local heads: independent of the routed heads
    cl_ev = []                          # HIP events around rt_cluster_attn in the timed steps

    def routed_step(timed=False):
        """The routed heads' forward (route, in-cluster attention, scatter-add and the
        centroid update), plus the in-cluster backward for the stress workload."""
        do_route()
        if timed:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            do_cluster()
            b.record(stream)
            cl_ev.append((a, b))
        else:
            do_cluster()
        do_scatter_update()
        if cfg.backward:
            do_bwd()

    def layer_step():
        """routed_step plus the local heads (after it, or concurrently)."""
        if cfg.L > 0 and args.concurrent_local:
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                do_local()
        routed_step()
        if cfg.L > 0:
            if not args.concurrent_local:
                do_local()
            else:
                stream.wait_stream(side)

    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    use_graph = args.graph and not args.no_graph

    def timed_loop(fn, steps, graph=None):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        ev0.record(stream)
        for _ in range(steps):
            if graph is not None:
                graph.replay()
            else:
                fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps, time.perf_counter() - t_wall

    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup)):
            layer_step()
        torch.cuda.synchronize()
        graph = None
        if use_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                routed_step()
            torch.cuda.synchronize()
            for _ in range(3):
                graph.replay()
            torch.cuda.synchronize()

        # The timed region: K routed steps (the metric).  The centroids evolve
        # step by step as in training; they start from the same state each run.
        mu.copy_(mu0)
        ms_per_step, t_wall = timed_loop(routed_step, args.steps, graph)
        # The same steps again with an event pair around each rt_cluster_attn (an
        # event drains the stream, so this pass is kept out of the metric): the
        # kernel's duration inside the step sequence, launch latency included.
        mu.copy_(mu0)
        timed_loop(lambda: routed_step(timed=True), args.steps)
        cluster_in_step_ms = float(np.mean([a.elapsed_time(b) for a, b in cl_ev]))

        # The whole layer (routed + local heads), the same number of steps.
        mu.copy_(mu0)
        layer_ms, _ = timed_loop(layer_step, args.steps)

        # Per call: amortised over back-to-back calls, and p10/p50/p90 per call,
        # warm and cold (events on the stream the kernels are launched on).
        calls = [("rt_route", do_route), ("rt_cluster_attn", do_cluster),
                 ("rt_scatter_rows", do_scatter), ("rt_scatter_rows+update", do_scatter_update),
                 ("rt_routed_attn_update", do_attn_update)]
        if cfg.L > 0:
            calls.append(("rt_local_attn", do_local))
        if cfg.backward:
            calls.append(("rt_routed_attn_bwd", do_bwd))
        flush = torch.empty((512 << 20) // 4, **f32)
        per_call, per_call_stats = {}, {}
        for name, fn in calls:
            fn()                        # a first launch loads the kernel's code
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(20, args.steps)
            gpu_ahead(30 * reps)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            per_call[name] = a.elapsed_time(b) / reps
            per_call_stats[name] = {"warm": event_stats(fn, args.reps, stream),
                                    "cold": event_stats(fn, args.reps, stream, flush)}
        del flush
        mu.copy_(mu0)

        # The floor of one dependent launch on the GPU: a captured graph of 100
        # one-element kernels, each waiting for the one before, replayed (so the
        # host's launch rate is out of it).
        tiny = torch.zeros(1, **f32)
        tiny_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(tiny_graph, stream=stream):
            for _ in range(100):
                tiny.add_(1.0)
        for _ in range(3):
            tiny_graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(5):
            tiny_graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        launch_floor_ms = a.elapsed_time(b) / 500
        del tiny_graph

    alg = algorithmic(cfg)
    tokens = B * n

    def rate(nbytes, flops, ms):
        s_ = ms * 1e-3
        r = {"ms": ms, "GB/s": nbytes / s_ / 1e9, "hbm_frac": nbytes / s_ / 1e9 / PEAK_HBM_GBS}
        if flops:
            r["TFLOP/s"] = flops / s_ / 1e12
            r["mfma_frac"] = flops / s_ / 1e12 / PEAK_BF16_TFLOPS
        return r

    stages = {
        "rt_route": rate(alg["route_bytes"], 0, per_call["rt_route"]),
        "rt_cluster_attn": rate(alg["attn_bytes"], alg["attn_flops_causal"],
                                per_call["rt_cluster_attn"]),
        "rt_scatter_rows+update": rate(alg["scatter_bytes"] + alg["ema_bytes"], 0,
                                       per_call["rt_scatter_rows+update"]),
        "rt_routed_attn_update": rate(alg["attn_bytes"] + alg["ema_bytes"],
                                      alg["attn_flops_causal"], per_call["rt_routed_attn_update"]),
    }
    stages["rt_route"]["scoring_TFLOP/s"] = alg["route_flops"] / (per_call["rt_route"] * 1e-3) / 1e12
    if cfg.backward:
        stages["rt_routed_attn_bwd"] = rate(alg["bwd_bytes"], alg["bwd_flops_causal"],
                                            per_call["rt_routed_attn_bwd"])
    if cfg.L > 0:
        stages["rt_local_attn"] = rate(alg["local_bytes"], alg["local_flops"],
                                       per_call["rt_local_attn"])
    # The dominant kernel of the routed step is the in-cluster attention:
    # rt_cluster_attn launches exactly cluster_attn_bf16_kernel, so its per-call
    # time (HIP events on its stream around back-to-back calls) is that kernel's
    # average launch duration.  Its intensity
    # (causal-useful flops over the bytes it must move, about w/3 flop/B) is far
    # below the ridge point, so HBM bounds it; its fraction of the bf16 MFMA peak
    # (the metric's second half) rides along.
    t = per_call["rt_cluster_attn"] * 1e-3
    achieved = alg["attn_bytes"] / t / 1e9
    roofline = {"bound": "hbm", "kernel": "cluster_attn_bf16_kernel (rt_cluster_attn)",
                "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS,
                "traffic": measured_traffic(CLUSTER_TRAFFIC, args.workload),
                "algorithmic_bytes": alg["attn_bytes"],
                "launch_ms": t * 1e3,
                "launch_ms_in_step": cluster_in_step_ms,
                "mfma_frac": alg["attn_flops_causal"] / t / 1e12 / PEAK_BF16_TFLOPS,
                "mfma_TFLOP/s": alg["attn_flops_causal"] / t / 1e12,
                "flops": alg["attn_flops_causal"],
                "flops_note": "causal-useful: 4 d (w (w+1)/2) per cluster (QK^T and PV over the "
                              "visible pairs)",
                "mfma_frac_hbm_ceiling": min(1.0, alg["attn_flops_causal"] / alg["attn_bytes"]
                                             * PEAK_HBM_GBS / 1e3 / PEAK_BF16_TFLOPS),
                "route_stage": {"entry": "rt_route", "algorithmic_bytes": alg["route_bytes"],
                                "ms": per_call["rt_route"],
                                "hbm_frac": stages["rt_route"]["hbm_frac"]}}
    routed_ceiling = tokens / ((alg["route_bytes"] + alg["attn_bytes"] + alg["ema_bytes"])
                               / (PEAK_HBM_GBS * 1e9))
    res = {
        "metric": "routed-attention tokens/sec/layer at n=8192 fwd; % bf16 MFMA peak",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded SplitMix64/Box-Muller inputs of the workload's shapes)",
        "config": {"workload": WORKLOADS[args.workload], "batch": B, "seq_len": n,
                   "routed_heads": R, "local_heads": cfg.L, "d_head": d, "k": k, "w": w,
                   "window": cfg.window, "graph": use_graph, "backward": cfg.backward,
                   "step": "rt_route -> rt_cluster_attn -> rt_scatter_rows (+ centroid update)"
                           + (" -> rt_routed_attn_bwd" if cfg.backward else "")},
        "roofline": roofline,
        "launch_floor": {
            "us_per_launch": launch_floor_ms * 1e3,
            "launches_per_step": 4 + (2 if cfg.backward else 0),
            "us_per_step": (4 + (2 if cfg.backward else 0)) * launch_floor_ms * 1e3,
            "share_of_step": (4 + (2 if cfg.backward else 0)) * launch_floor_ms / ms_per_step,
            "note": "a replayed graph of dependent one-element kernels: the least a dependent "
                    "launch costs on the GPU; the step makes 4 (scoring, top-w, in-cluster attention, "
                    "scatter with the centroid update)" + (" plus 2 for the backward"
                                                           if cfg.backward else "")},
        "hbm_bound_ceiling_tokens_per_s": routed_ceiling,
        "frac_of_hbm_ceiling": tokens / (ms_per_step * 1e-3) / routed_ceiling,
        "layer": {"ms_per_step": layer_ms, "tokens_per_s": tokens / (layer_ms * 1e-3),
                  "local_heads_stream": "concurrent" if args.concurrent_local else "same",
                  "note": "routed step plus the local heads' rt_local_attn"},
        "per_call_ms": per_call,
        "per_call_stats_ms": per_call_stats,
        "stages": stages,
        "routed_over_local_time": (ms_per_step / per_call["rt_local_attn"]
                                   if "rt_local_attn" in per_call and not cfg.backward else None),
        "wall_s_timed": t_wall,
    }
    if args.workload == "long" and not args.no_stack:
        res["stack"] = time_stack(rt, S.STACKS["long_stack"], use_graph=use_graph)
    if args.workload == "long" and not args.no_extras:
        res["variants"] = time_variants(rt, cfg, inp)
        res["decode"] = time_decode(rt, cfg, inp)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, scale)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
