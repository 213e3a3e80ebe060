#!/usr/bin/env python3
"""Benchmark of the projected-attention forward on one MI355X.

One step = one spa_attn_fwd call (projection launch + attention launch) over the headline
workload, B=2 H=16 N=8192 d=128 m=32 dv=128, causal, bf16 inputs and output, with the inputs
resident in HBM. Prints one JSON line (see the keys below).

  python bench.py [--steps K] [--warmup W] [--workload c3] [--no-cpu-baseline]
  python bench.py --calibrate-copy      # a plain 1 GiB device copy, for counter scaling

Flops are algorithmic (the projection 4 N d m, scores 2 N^2 m, weights x V 2 N^2 dv per head,
the N^2 terms halved under the causal mask); the exact-attention work the method avoids is
not counted. The timed steps are the product call alone. A second pass of the same number of
steps, after the timed region, records HIP events around each launch on the launch stream:
that gives the per-launch split and the dominant kernel's duration for the roofline.
Measured matrix-core and fp32 VALU rates with the engine clock (rate probes of the library)
are reported beside the published peaks.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import jl_feature_projected_amd as spa  # noqa: E402
from jl_feature_projected_amd import accounting, inputs  # noqa: E402

METRIC = "projected-attention fwd TFLOP/s and % bf16 MFMA peak at N=8192,d=128,m=32"
# The attention kernel's source: the kernel file and the device helpers it includes.
ATTN_SRCS = [os.path.join(ROOT, "jl_feature_projected_amd", "csrc", f)
             for f in ("spa_attn_bf16.hip", "spa_device.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_c3_hbm_traffic.md")


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name: str):
    """HBM bytes per attention launch from the committed counter summary, if it was taken on
    this exact kernel source and workload; otherwise None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"kernel source sha256\[:16\]:\s*`?([0-9a-f]{16})", text)
    m_wl = re.search(r"workload:\s*`?([\w.-]+)", text)
    m_b = re.search(r"hbm bytes per launch:\s*`?([0-9.eE+]+)", text)
    if not (m_hash and m_wl and m_b):
        return None
    if m_hash.group(1) != source_hash(ATTN_SRCS) or m_wl.group(1) != workload_name:
        return None
    return float(m_b.group(1))


def cpu_baseline(w: inputs.Workload, x: inputs.Inputs, budget_s: float = 12.0) -> dict:
    """The CPU oracle timed on a bounded sample of the same workload: whole heads, all rows."""
    import numpy as np

    import oracle

    BH = w.B * w.H
    Q = x.Q.reshape(BH, 1, w.N, w.d)
    K = x.K.reshape(BH, 1, w.N, w.d)
    V = x.V.reshape(BH, 1, w.N, w.dv)
    P = x.P.double().numpy()

    def heads(n):
        # heads 0..n-1 of the flattened (batch, head) axis, each with its own P[h]
        idx = list(range(n))
        q = np.concatenate([Q[i:i + 1].double().numpy() for i in idx], axis=1)
        k = np.concatenate([K[i:i + 1].double().numpy() for i in idx], axis=1)
        v = np.concatenate([V[i:i + 1].double().numpy() for i in idx], axis=1)
        p = np.stack([P[i % w.H] for i in idx])
        return q, k, v, p

    q, k, v, p = heads(1)
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, p, w.scale, w.causal)
    t1 = time.perf_counter() - t0
    n = max(1, min(BH, int(budget_s / max(t1, 1e-3))))
    if n > 1:
        q, k, v, p = heads(n)
        t0 = time.perf_counter()
        oracle.attn_fwd(q, k, v, p, w.scale, w.causal)
        t1 = time.perf_counter() - t0
    flops = accounting.work(1, n, w.N, w.d, w.m, w.dv, w.causal).total_flops
    return {"value": round(flops / t1 / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{n} of {BH} heads, all {w.N} rows each ({flops / 1e9:.1f} GFLOP, "
                      f"{t1:.2f} s, float64)"}


def time_backward(w, x, Q, K, V, P, steps, warmup, dev) -> dict:
    """spa_attn_bwd on the forward's own output and lse, dO a seeded N(0, 1) draw; steps
    calls timed between events on the launch stream after warmup calls."""
    f32 = Q.dtype == torch.float32  # the fp32 path: fp32 O, dO and gradients
    O, lse = spa.spa_attn_fwd(Q, K, V, P, w.scale, w.causal,
                              out_dtype=torch.float32 if f32 else torch.bfloat16, return_lse=True)
    dO = inputs.draw_grad_output(w, seed=w.seed + 1).to(dev)
    ws = torch.empty(spa.spa_attn_bwd_workspace_bytes(w.B, w.H, w.N, w.d, w.m, w.dv, Q.dtype),
                     dtype=torch.uint8, device=dev)

    def timed(grad_dtype) -> float:
        def bstep():
            spa.spa_attn_bwd(Q, K, V, P, O, dO, lse, w.scale, w.causal, grad_dtype=grad_dtype,
                             workspace=ws)

        for _ in range(warmup):
            bstep()
        stream = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            bstep()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    bw = accounting.bwd_work(w.B, w.H, w.N, w.d, w.m, w.dv, w.causal)
    peak = accounting.PEAK_FP32_VECTOR_TFLOPS if f32 else accounting.PEAK_BF16_DENSE_TFLOPS
    ms = timed(torch.float32)
    tf = bw.total_flops / (ms * 1e-3) / 1e12
    res = {"ms_per_call": round(ms, 5), "value": round(tf, 3), "unit": "TFLOP/s",
           "dtype": "f32" if f32 else "bf16",
           "pct_of_peak": round(100.0 * tf / peak, 2),
           "peak": peak, "flops_per_call": bw.total_flops,
           "executed_n2_flops_per_call": bw.executed_n2_flops, "grad_dtype": "f32"}
    if not f32:
        # the same calls writing dQ, dK and dV in bf16, the inputs' dtype (what spa_attention
        # hands to autograd); the arithmetic is the same, only the stores are narrower
        ms16 = timed(torch.bfloat16)
        tf16 = bw.total_flops / (ms16 * 1e-3) / 1e12
        res["bf16_grads"] = {"ms_per_call": round(ms16, 5), "value": round(tf16, 3),
                             "pct_of_peak": round(100.0 * tf16 / peak, 2)}
    return res


def time_decode(w, x, P, steps, warmup, dev, nq: int = 1) -> dict:
    """One decode step per call: the last nq queries of every head against the whole cache
    of projected keys (fp16) and values, spa_attn_decode timed between events on the launch
    stream. The reported rate is the cache bytes read per second (the bound at few queries);
    the flops of the step are reported beside it."""
    K, V = x.K.to(dev), x.V.to(dev)
    cache = torch.empty((w.B, w.H, w.N, w.m), dtype=torch.float16, device=dev)
    spa.spa_kcache_append(K, P, cache, 0)
    Q = x.Q[:, :, -nq:].contiguous().to(dev)
    ws = torch.empty(spa.spa_attn_decode_workspace_bytes(w.B, w.H, nq, w.N, w.dv),
                     dtype=torch.uint8, device=dev)

    def dstep():
        spa.spa_attn_decode(Q, cache, V, P, w.N, w.scale, w.causal, workspace=ws)

    for _ in range(warmup):
        dstep()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        dstep()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    cache_bytes = w.B * w.H * w.N * (2 * w.m + 2 * w.dv)
    gbs = cache_bytes / (ms * 1e-3) / 1e9
    # every query against all N keys (the causal mask drops about nq^2 / 2 of those pairs)
    flops = w.B * w.H * nq * w.N * (2 * w.m + 2 * w.dv)
    return {"ms_per_step": round(ms, 5), "cache_bytes": cache_bytes,
            "value": round(gbs, 1), "unit": "GB/s", "frac_of_hbm_peak": round(gbs / 8000.0, 4),
            "k_cache_vs_k_bytes": round(w.m / w.d, 4), "queries_per_head": nq,
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}


def time_sfa(w, Q, K, V, topk, steps, warmup, dev) -> dict:
    """spa_sfa_fwd on the workload's Q, K, V with topk features per row, timed between
    events on the launch stream. Its attention kernel runs the score MFMA over all d
    features (the zeros included), so the rate is quoted on c N^2 (2d + 2dv) flops per head."""
    O = torch.empty((w.B, w.H, w.N, w.dv), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(spa.spa_sfa_fwd_workspace_bytes(w.B, w.H, w.N, w.d, w.dv),
                     dtype=torch.uint8, device=dev)

    def sstep():
        spa.spa_sfa_fwd(Q, K, V, topk, w.scale, w.causal, out_dtype=torch.bfloat16,
                        workspace=ws)

    for _ in range(warmup):
        sstep()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        sstep()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    c = 0.5 if w.causal else 1.0
    # executed: the score MFMAs run over all d features, zeros included
    flops = c * w.N * w.N * (2 * w.d + 2 * w.dv) * w.B * w.H
    # the method's own work: a query and a key with k of d features each share k^2/d features
    # on average, two flops each, plus the weights times V
    method = c * w.N * w.N * (2.0 * topk * topk / w.d + 2 * w.dv) * w.B * w.H
    tf = flops / (ms * 1e-3) / 1e12
    tm = method / (ms * 1e-3) / 1e12
    return {"topk": topk, "ms_per_call": round(ms, 5), "unit": "TFLOP/s",
            "executed_tflops": round(tf, 3), "executed_flops_per_call": flops,
            "method_tflops": round(tm, 3), "method_flops_per_call": method,
            "method_pct_of_bf16_peak": round(100.0 * tm / accounting.PEAK_BF16_DENSE_TFLOPS, 2)}


def calibrate_copy(dev) -> None:
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=inputs.HEADLINE, choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="also time one decode step (spa_attn_decode, the last query of every "
                         "head against the whole cache) and report it in a 'decode' object")
    ap.add_argument("--decode-queries", type=int, default=1,
                    help="queries per head of the decode step (more than four take the "
                         "matrix-core kernel when m is a multiple of 8)")
    ap.add_argument("--sfa", type=int, default=0, metavar="K",
                    help="also time sparse feature attention (spa_sfa_fwd) with K features "
                         "per row and report it in an 'sfa' object")
    ap.add_argument("--backward", action="store_true",
                    help="also time spa_attn_bwd (bf16 workloads) and report it in a "
                         "'backward' object")
    args = ap.parse_args()
    if not 1 <= args.decode_queries <= inputs.WORKLOADS[args.workload].N:
        ap.error("--decode-queries must be between 1 and the workload's N")

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every (batch, head) is independent, and the library "
              "has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(dev)
        return 0

    w = inputs.WORKLOADS[args.workload]
    x = inputs.draw(w)
    Q, K, V, P = (t.to(dev) for t in (x.Q, x.K, x.V, x.P))
    out_dtype = w.torch_dtype
    O = torch.empty((w.B, w.H, w.N, w.dv), dtype=out_dtype, device=dev)
    ws = torch.empty(spa.spa_attn_fwd_workspace_bytes(w.B, w.H, w.N, w.d, w.m, w.dv, w.torch_dtype),
                     dtype=torch.uint8, device=dev)

    def step():
        spa.spa_attn_fwd(Q, K, V, P, w.scale, w.causal, out=O, workspace=ws, out_dtype=out_dtype)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)

    # Launch split: the same number of steps again, with the library's HIP events around
    # each launch on the launch stream (outside the timed region: the events themselves add
    # a few microseconds per launch).
    spa.profile_begin(args.steps)
    for _ in range(args.steps):
        step()
    proj_ms, attn_ms, calls = spa.profile_end()

    # Distribution of single calls (after the timed region, not part of it): each call
    # bracketed by its own events on the launch stream.
    per_call = []
    for _ in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        per_call.append(e0.elapsed_time(e1))
    per_call.sort()

    work = accounting.work(w.B, w.H, w.N, w.d, w.m, w.dv, w.causal)
    ms_per_step = max(wall * 1e3, ev_ms) / args.steps
    value = work.total_flops / (ms_per_step * 1e-3) / 1e12
    peak = accounting.PEAK_BF16_DENSE_TFLOPS if w.dtype == "bf16" else accounting.PEAK_FP32_VECTOR_TFLOPS
    attn_avg_ms = attn_ms / calls
    plan = spa.spa_attn_fwd_plan(w.B, w.H, w.N, w.d, w.m, w.dv, spa.SPA_BF16 if w.dtype == "bf16"
                                 else spa.SPA_F32, w.causal)
    q_in_attn = plan > 0 and bool(plan & spa.SPA_PLAN_QUERIES_IN_ATTENTION)
    # the attention launch's work: scores and weights x V, plus the query projection when it
    # runs there
    attn_work = work.attn_flops + (work.project_flops / 2 if q_in_attn else 0.0)
    achieved = attn_work / (attn_avg_ms * 1e-3) / 1e12
    bytes_ = accounting.path_bytes(w.B, w.H, w.N, w.d, w.m, w.dv,
                                   elem=2 if w.dtype == "bf16" else 4,
                                   out_elem=2 if w.dtype == "bf16" else 4,
                                   queries_in_attention=q_in_attn)
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "m": w.m,
                   "dv": w.dv, "causal": w.causal, "out_dtype": w.dtype,
                   "flops_per_step": work.total_flops},
        "pct_of_bf16_peak": round(100.0 * value / accounting.PEAK_BF16_DENSE_TFLOPS, 2),
        "launch_ms": {"project": round(proj_ms / calls, 5), "attn": round(attn_avg_ms, 5)},
        "call_ms": {"median": round(per_call[len(per_call) // 2], 5),
                    "min": round(per_call[0], 5),
                    "p90": round(per_call[int(0.9 * (len(per_call) - 1))], 5),
                    "calls": len(per_call)},
        "roofline": {
            "kernel": "attn_bf16_kernel" if w.dtype == "bf16" else "attn_f32_kernel",
            "bound": "mfma" if w.dtype == "bf16" else "alu",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(w.name),
            "algorithmic_bytes": bytes_["attn"],
        },
    }
    # Measured rates behind the published peaks (pure-MFMA and fp32-FMA probes).
    rates = spa.probe_rates(dev)
    res["measured_rates"] = {k: round(v, 3) for k, v in rates.items()}
    res["roofline"]["frac_of_measured_mfma"] = (
        round(achieved / rates["mfma_bf16_tflops"], 4) if w.dtype == "bf16" else None)
    if args.backward:
        res["backward"] = time_backward(w, x, Q, K, V, P, args.steps, args.warmup, dev)
    if args.sfa and w.dtype == "bf16":
        res["sfa"] = time_sfa(w, Q, K, V, args.sfa, args.steps, args.warmup, dev)
    if args.decode and w.dtype == "bf16":
        res["decode"] = time_decode(w, x, P, args.steps, args.warmup, dev, args.decode_queries)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
