#!/usr/bin/env python3
"""Benchmark of the block-quantized MoE hot path on one MI355X.

Headline workload: one top-6 MoE decode layer, q = 1 (hidden 4096, 256 routed
experts, inter 2048; gate/up ROCmFP2 with 4-entry per-expert codebooks, down
ROCmFP3 with 8-entry codebooks; router fp16 N(0, 0.02), softmax over the top 6;
SwiGLU; x fp32 N(0, 1)). A step is one qmoe_decode_layer call on one token;
64 pre-generated tokens rotate so that consecutive calls route to different
experts (the 2.28 GB of packed experts do not fit in the 256 MB last-level
cache, so weights stream from HBM).

value = effective packed-weight GB/s = packed bytes of the experts a call
touches (6 x 8,912,896 B) / wall time per call (router time included, router
bytes not counted).

Also reported (the other rows of the hot path): q = 4 decode with forced expert
overlap, 8K-token prefill with Zipf-skewed routing, the dense FP4 + FP3/H32 mix
at batch 1 and 4, and the FP2 512x256 matvec latency.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_MFMA_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, published (TOPS)
# HBM bytes per launch of the dominant decode q=1 kernel (k_gateup1<2>), from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs scaled by a 256 MiB device copy (profiles/hbm_traffic_decode_q1_prefill_8k.md). Must be
# re-measured (or set to None) whenever that kernel changes.
DOMINANT_Q1_TRAFFIC_BYTES = 31819695

WORKLOAD = ("MoE decode layer q=1: hidden 4096, 256 routed experts, expert intermediate 2048, router W fp16 "
            "N(0,0.02) with softmax top-6, gate/up ROCmFP2 (4-entry per-expert codebooks), down ROCmFP3 "
            "(8-entry codebooks), SwiGLU, x fp32 N(0,1)")
METRIC = "effective packed-weight GB/s + MoE layer tokens/s (q=1, q=4, 8K prefill), % roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="only the q=1 headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=256)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before the benchmark, copy MIB MiB device-to-device once (a plain copy of known size, "
                         "for scaling memory-traffic counters)")
    ap.add_argument("--prefill-only", action="store_true", help="only the 8K-token prefill (for profiling)")
    ap.add_argument("--quantize-only", action="store_true", help="only the weight quantizer (for profiling)")
    ap.add_argument("--decode-q4-only", action="store_true", help="only the q=4 decode (for profiling)")
    ap.add_argument("--dense-only", action="store_true", help="only the dense FP4 + FP3/H32 mix (for profiling)")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the warm q=1 calls and their kernel times (for the kernel-trace profile)")
    ap.add_argument("--prefill-small-sweep", action="store_true",
                    help="only: prefill time against the small-expert threshold over batch sizes")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timer:
    """HIP events on the current (launch) stream around a block of calls."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.torch.cuda.synchronize()
        self.ms = self.a.elapsed_time(self.b)


def kernel_avg_ms(qm, name):
    tot, n = qm.qmoe_timing_read(name)
    return (tot / n if n else None), n


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_block_quantized_rocmfp2_amd as qm
    from synth import gen

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    spec = gen.LayerSpec.full()
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read + {n} bytes written")
        del src, dst
    t0 = time.time()
    dl = qm.device.DeviceLayer(spec, seed=0)
    per_expert = dl.packed_bytes_per_expert()
    log(f"built full layer ({per_expert * spec.n_experts:,} packed bytes) in {time.time() - t0:.1f}s")
    gateup_bytes = qm.qmoe_packed_bytes(2, spec.inter, spec.hidden) * 2
    if args.prefill_only:
        res = bench_prefill(torch, qm, gen, spec, dl, dev)
        print(json.dumps({"prefill_8k": res}), flush=True)
        return
    if args.prefill_small_sweep:
        print(json.dumps({"prefill_small_sweep": bench_prefill_small_sweep(torch, qm, gen, spec, dl, dev)}), flush=True)
        return
    if args.quantize_only:
        print(json.dumps({"quantize_fp2": bench_quantize(torch, qm, gen, dev),
                          "quantize_fp3": bench_quantize(torch, qm, gen, dev, fmt=3, rows=4096, k=2048)}), flush=True)
        return
    if args.dense_only:
        res = {}
        bench_dense(args, torch, qm, gen, dev, res)
        print(json.dumps(res), flush=True)
        return
    ws = dl.workspace(4)
    if args.decode_q4_only:
        print(json.dumps(bench_q4(args, torch, qm, gen, spec, dl, ws, per_expert, dev)[0]), flush=True)
        return
    toks = torch.from_numpy(gen.tokens(64, spec.hidden, seed=0, stream=7)).to(dev)
    out = torch.empty((4, spec.hidden), dtype=torch.float32, device=dev)

    def decode_q1(i):
        qm.qmoe_decode_layer(dl.desc, toks[i % 64: i % 64 + 1], out[:1], ws)

    # ---------------------------------------------------------------- q = 1 headline
    for i in range(args.warmup):
        decode_q1(i)
    K = args.steps
    with Timer(torch) as t:
        for i in range(K):
            decode_q1(i)
    ms = t.ms / K
    bytes_q1 = spec.topk * per_expert
    value = bytes_q1 / (ms * 1e-3) / 1e9
    log(f"decode q=1: {ms * 1e3:.2f} us/call, {value:.1f} GB/s effective")
    if args.headline_only:
        K_only = K

        def kernel_times_only(names):
            qm.qmoe_timing_enable(True)
            for i in range(K_only):
                decode_q1(i)
            torch.cuda.synchronize()
            kt = {name: kernel_avg_ms(qm, name)[0] for name in names}
            qm.qmoe_timing_enable(False)
            return kt
        kern = kernel_times_only(("route", "gateup", "down"))
        log("decode q=1 kernels (us): " + ", ".join(f"{k}={v * 1e3:.2f}" for k, v in kern.items()))
        print(json.dumps({"decode_q1_us_per_call": round(ms * 1e3, 2),
                          "kernel_us": {k: round(v * 1e3, 2) for k, v in kern.items()}}), flush=True)
        return
    # per-call distribution: a pair of events around each of K back-to-back calls
    evk = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        evk[i][0].record()
        decode_q1(i)
        evk[i][1].record()
    torch.cuda.synchronize()
    per_call = np.array([a.elapsed_time(b) for a, b in evk]) * 1e3
    pct = {f"p{p}": round(float(np.percentile(per_call, p)), 2) for p in (10, 50, 90)}
    log(f"decode q=1 per-call events (us): {pct}")

    # cold-cache variant: before each call a 512 MiB device write (not timed)
    # evicts the 256 MB last-level cache and the L2s, then the call alone is
    # timed with events on the stream
    # (the same single-call timing after a 4 KiB write separates the cost of
    # timing a call alone from the cost of the cold cache)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(64)]

    def single_calls(nbytes, read_only=False):
        buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
        acc = torch.zeros(1, dtype=torch.int32, device=dev)
        t_ = []
        for rep in range(2):
            for i in range(64):
                if read_only:
                    torch.amax(buf, dim=0, keepdim=True, out=acc)   # reads the buffer, writes 4 bytes
                else:
                    buf.fill_(rep + i)
                ev[i][0].record()
                decode_q1(i)
                ev[i][1].record()
            torch.cuda.synchronize()
            t_ += [a.elapsed_time(b) for a, b in ev]
        del buf
        return float(np.mean(t_[64:]))
    ms_cold = single_calls(512 << 20)
    ms_cold_r = single_calls(512 << 20, read_only=True)
    ms_single = single_calls(4096)
    log(f"decode q=1 single calls: {ms_cold * 1e3:.2f} us after a 512 MiB write, {ms_cold_r * 1e3:.2f} us after a "
        f"512 MiB read, {ms_single * 1e3:.2f} us after a 4 KiB write (mean of 64)")

    # the same calls captured once as a HIP graph (64 calls, one per rotating
    # token) and replayed: the steady state of a decode loop that replays its
    # layer launches
    g_stream = torch.cuda.Stream()
    g_stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(g_stream):
        for i in range(64):
            decode_q1(i)
    torch.cuda.current_stream().wait_stream(g_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(64):
            decode_q1(i)
    for _ in range(2):
        graph.replay()
    reps = max(1, K // 64)
    with Timer(torch) as tg:
        for _ in range(reps):
            graph.replay()
    ms_graph = tg.ms / (reps * 64)
    log(f"decode q=1 graph replay: {ms_graph * 1e3:.2f} us/call, "
        f"{bytes_q1 / (ms_graph * 1e-3) / 1e9:.1f} GB/s effective")
    del graph

    # dominant kernel, timed with HIP events on the launch stream over K calls
    def kernel_times(names):
        qm.qmoe_timing_enable(True)
        for i in range(K):
            decode_q1(i)
        torch.cuda.synchronize()
        kt = {}
        for name in names:
            avg, n = kernel_avg_ms(qm, name)
            if avg:
                kt[name] = avg
        qm.qmoe_timing_enable(False)
        return kt
    kern = kernel_times(("route", "gateup", "down"))
    log("decode q=1 kernels (us): " + ", ".join(f"{k}={v * 1e3:.2f}" for k, v in kern.items()))
    dom_ms, dom_bytes = kern["gateup"], spec.topk * gateup_bytes
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": DOMINANT_Q1_TRAFFIC_BYTES,
                "kernel": "k_gateup1<2> (6 experts x gate+up FP2 = 31,457,280 algorithmic bytes per launch)",
                "kernel_us": round(dom_ms * 1e3, 2)}
    down_gbs = spec.topk * qm.qmoe_packed_bytes(3, spec.hidden, spec.inter) / (kern["down"] * 1e-3) / 1e9

    # measured HBM read peak: the library's read-only streaming probe over 1 GiB
    # (the best of several grid sizes); a 1 GiB device copy is kept beside it
    probes = bench_probes(torch, qm, dev)
    read_gbs = probes["stream_read"]["peak_GBps"]
    router_bytes = spec.n_experts * spec.hidden * 2
    roofline["measured_stream_peak"] = round(read_gbs, 1)
    roofline["measured_stream_peak_kind"] = "read-only stream, 1 GiB (qmoe_probe_read)"
    roofline["frac_of_measured_stream_peak"] = round(achieved / read_gbs, 4)

    extra = {"decode_q1": {"us_per_call": round(ms * 1e3, 2), "tokens_per_s": round(1.0 / (ms * 1e-3), 1),
                           "us_per_call_events": pct,
                           "effective_GBps_with_router": round((bytes_q1 + router_bytes) / (ms * 1e-3) / 1e9, 1),
                           "frac_of_measured_stream_peak": round(value / read_gbs, 4),
                           "effective_GBps": round(value, 1), "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
                           "kernel_us": {k: round(v * 1e3, 2) for k, v in kern.items() if v},
                           "down_kernel_GBps": round(down_gbs, 1),
                           "single_call_after_512MiB_write_us": round(ms_cold * 1e3, 2),
                           "single_call_after_512MiB_read_us": round(ms_cold_r * 1e3, 2),
                           "single_call_warm_us": round(ms_single * 1e3, 2),
                           "graph_replay_us_per_call": round(ms_graph * 1e3, 2),
                           "graph_replay_GBps": round(bytes_q1 / (ms_graph * 1e-3) / 1e9, 1)},
             "probes": probes}

    if not args.no_extra:
        extra.update(bench_extra(args, torch, qm, gen, spec, dl, ws, per_expert, dev))
        pf = extra.get("prefill_8k", {})
        if pf.get("gemm_int8_TOPS"):
            mf = probes["mfma_int8"]
            pf["gemm_frac_of_measured_mfma_16x16x32"] = round(pf["gemm_int8_TOPS"] / mf["k16x16x32_TOPS"], 4)
            pf["gemm_frac_of_valu_epilogue_ceiling"] = round(pf["gemm_int8_TOPS"] / probes["valu_epilogue"]
                                                             ["int8_TOPS_ceiling"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, spec, dl, per_expert, extra)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8 dot / fp32 accumulate (ROCmFP2/FP3 weights)", "data": "synthetic",
        "config": {"workload": WORKLOAD, "q": 1, "seed": 0, "rotating_tokens": 64, "packed_bytes_per_call": bytes_q1,
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)


def bench_q4(args, torch, qm, gen, spec, dl, ws, per_expert, dev):
    """q = 4 decode on groups of four tokens whose top-6 sets overlap (at most 12
    distinct experts, at least half of them shared by two or more tokens)."""
    res = {}
    K = max(20, args.steps // 2)
    groups, U = [], []
    idx = torch.empty((4, spec.topk), dtype=torch.int32, device=dev)
    gw = torch.empty((4, spec.topk), dtype=torch.float32, device=dev)
    variant = 0
    while len(groups) < 16 and variant < 400:
        x = torch.from_numpy(gen.q4_group(spec.hidden, seed=0, variant=variant)).to(dev)
        qm.qmoe_route(dl.desc, x, idx, gw, ws)
        ids, counts = np.unique(idx.cpu().numpy().ravel(), return_counts=True)
        if len(ids) <= 12 and 2 * np.sum(counts >= 2) >= len(ids):
            groups.append(x)
            U.append(len(ids))
        variant += 1
    out = torch.empty((4, spec.hidden), dtype=torch.float32, device=dev)
    for i in range(10):
        qm.qmoe_decode_layer(dl.desc, groups[i % len(groups)], out, ws)
    with Timer(torch) as t:
        for i in range(K):
            qm.qmoe_decode_layer(dl.desc, groups[i % len(groups)], out, ws)
    ms = t.ms / K
    mean_bytes = float(np.mean([U[i % len(groups)] for i in range(K)])) * per_expert
    gbs = mean_bytes / (ms * 1e-3) / 1e9
    qm.qmoe_timing_enable(True)
    for i in range(K):
        qm.qmoe_decode_layer(dl.desc, groups[i % len(groups)], out, ws)
    torch.cuda.synchronize()
    kern = {}
    for name in ("route", "gateup", "down"):
        avg, _ = kernel_avg_ms(qm, name)
        if avg:
            kern[name] = round(avg * 1e3, 2)
    qm.qmoe_timing_enable(False)
    res["decode_q4"] = {"us_per_call": round(ms * 1e3, 2), "tokens_per_s": round(4 / (ms * 1e-3), 1),
                        "mean_distinct_experts": round(float(np.mean(U)), 2), "effective_GBps": round(gbs, 1),
                        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "groups": len(groups), "kernel_us": kern}
    log(f"decode q=4: {ms * 1e3:.2f} us/call, U={np.mean(U):.2f}, {gbs:.1f} GB/s; kernels (us): "
        + ", ".join(f"{k}={v}" for k, v in kern.items()))
    return res, groups, out, ms


def bench_extra(args, torch, qm, gen, spec, dl, ws, per_expert, dev):
    K = max(20, args.steps // 2)
    res, groups, out, ms = bench_q4(args, torch, qm, gen, spec, dl, ws, per_expert, dev)

    # ablation: the same four columns decoded one call per column (each expert
    # block decoded once per routed column instead of once per group)
    cols = [[g[t:t + 1] for t in range(4)] for g in groups]
    for i in range(10):
        for t in range(4):
            qm.qmoe_decode_layer(dl.desc, cols[i % len(groups)][t], out[t:t + 1], ws)
    with Timer(torch) as t_pc:
        for i in range(K):
            for t in range(4):
                qm.qmoe_decode_layer(dl.desc, cols[i % len(groups)][t], out[t:t + 1], ws)
    ms_pc = t_pc.ms / K
    res["decode_q4_per_column"] = {"us_per_4_tokens": round(ms_pc * 1e3, 2),
                                   "tokens_per_s": round(4 / (ms_pc * 1e-3), 1),
                                   "decode_once_speedup": round(ms_pc / ms, 3),
                                   "packed_bytes_read": 4 * spec.topk * per_expert}
    log(f"decode q=4 as four q=1 calls: {ms_pc * 1e3:.2f} us ({ms_pc / ms:.2f}x the decode-once call)")

    # ablation: the same groups with the expert products on the int8 matrix
    # cores (qmoe_decode_layer_mfma: the 4 tokens as the MFMA's 4 columns)
    for i in range(10):
        qm.qmoe_decode_layer_mfma(dl.desc, groups[i % len(groups)], out, ws)
    with Timer(torch) as t_mx:
        for i in range(K):
            qm.qmoe_decode_layer_mfma(dl.desc, groups[i % len(groups)], out, ws)
    ms_mx = t_mx.ms / K
    qm.qmoe_timing_enable(True)
    for i in range(K):
        qm.qmoe_decode_layer_mfma(dl.desc, groups[i % len(groups)], out, ws)
    torch.cuda.synchronize()
    kern_mx = {}
    for name in ("route", "gateup_mx", "down_mx"):
        avg, _ = kernel_avg_ms(qm, name)
        if avg:
            kern_mx[name] = round(avg * 1e3, 2)
    qm.qmoe_timing_enable(False)
    res["decode_q4_mfma"] = {"us_per_call": round(ms_mx * 1e3, 2), "tokens_per_s": round(4 / (ms_mx * 1e-3), 1),
                             "vs_dot4_call": round(ms_mx / ms, 3), "kernel_us": kern_mx,
                             "entry_point": "qmoe_decode_layer_mfma"}
    log(f"decode q=4 with the products on v_mfma_i32_4x4x4_16b_i8: {ms_mx * 1e3:.2f} us ({ms_mx / ms:.2f}x the "
        f"dot4 call); kernels (us): " + ", ".join(f"{k}={v}" for k, v in kern_mx.items()))

    # routing variant: the same layer with top-4 routing, q = 1
    desc4 = qm.make_layer(spec.hidden, spec.inter, spec.n_experts, 4, spec.fmt_gate, spec.fmt_up, spec.fmt_down,
                          spec.rot_gateup, spec.rot_down, dl.w_router, None, dl.gate, dl.up, dl.down, dl.cb_gate,
                          dl.cb_up, dl.cb_down)
    toks = torch.from_numpy(gen.tokens(64, spec.hidden, seed=0, stream=7)).to(dev)
    for i in range(10):
        qm.qmoe_decode_layer(desc4, toks[i % 64: i % 64 + 1], out[:1], ws)
    with Timer(torch) as t4:
        for i in range(K):
            qm.qmoe_decode_layer(desc4, toks[i % 64: i % 64 + 1], out[:1], ws)
    ms4 = t4.ms / K
    gbs4 = 4 * per_expert / (ms4 * 1e-3) / 1e9
    res["decode_q1_top4"] = {"us_per_call": round(ms4 * 1e3, 2), "effective_GBps": round(gbs4, 1),
                             "frac_hbm_peak": round(gbs4 / HBM_PEAK_GBS, 4)}
    log(f"decode q=1 top-4: {ms4 * 1e3:.2f} us/call, {gbs4:.1f} GB/s")

    # format variant: the same layer with FP2 down projections (2.5 bits per weight
    # everywhere), q = 1; gate/up and the router are shared with the FP3-down layer
    spec2 = gen.LayerSpec.full(fmt_down=2)
    down2, cb_down2 = qm.device.pack_experts(spec2, "down", 0, dev)
    desc2 = qm.make_layer(spec2.hidden, spec2.inter, spec2.n_experts, spec2.topk, spec2.fmt_gate, spec2.fmt_up,
                          spec2.fmt_down, spec2.rot_gateup, spec2.rot_down, dl.w_router, None, dl.gate, dl.up, down2,
                          dl.cb_gate, dl.cb_up, cb_down2)
    qm.qmoe_layer_check(desc2)
    per_expert2 = (qm.qmoe_packed_bytes(2, spec2.inter, spec2.hidden) * 2
                   + qm.qmoe_packed_bytes(2, spec2.hidden, spec2.inter))
    for i in range(10):
        qm.qmoe_decode_layer(desc2, toks[i % 64: i % 64 + 1], out[:1], ws)
    with Timer(torch) as t2:
        for i in range(K):
            qm.qmoe_decode_layer(desc2, toks[i % 64: i % 64 + 1], out[:1], ws)
    ms2 = t2.ms / K
    gbs2 = spec2.topk * per_expert2 / (ms2 * 1e-3) / 1e9
    res["decode_q1_fp2_down"] = {"us_per_call": round(ms2 * 1e3, 2), "effective_GBps": round(gbs2, 1),
                                 "frac_hbm_peak": round(gbs2 / HBM_PEAK_GBS, 4),
                                 "packed_bytes_per_call": spec2.topk * per_expert2}
    log(f"decode q=1 FP2 down: {ms2 * 1e3:.2f} us/call, {gbs2:.1f} GB/s")
    del down2, cb_down2

    # ---------------------------------------------------------------- a stack of distinct layers
    try:
        res["decode_q1_layer_stack"] = bench_layer_stack(torch, qm, gen, spec, per_expert, dev)
    except RuntimeError as e:   # e.g. out of device memory
        res["decode_q1_layer_stack"] = {"status": f"not run: {e}"}

    # ---------------------------------------------------------------- prefill 8K (Zipf)
    try:
        res["prefill_8k"] = bench_prefill(torch, qm, gen, spec, dl, dev)
    except qm.QmoeError as e:
        res["prefill_8k"] = {"status": f"not run: {e}"}

    # ---------------------------------------------------------------- dense FP4 + FP3/H32 mix
    fp4, fp3 = bench_dense(args, torch, qm, gen, dev, res)

    # ---------------------------------------------------------------- fused versus expand-then-multiply
    fp3_big = gen.matvec_case(3, 4096, 16384, ncols=1, seed=0, rot=1)
    for name, fmt_x, c in (("fp3_4096x2048_h32", 3, fp3), ("fp3_4096x16384_h32", 3, fp3_big),
                           ("fp4_4096x16384", 4, fp4)):
        m = qm.device.DeviceMatrix(c)
        x1 = torch.from_numpy(c.x[:1]).to(dev)
        y1 = torch.empty((1, c.rows), dtype=torch.float32, device=dev)
        ws_f = m.workspace(1)
        ws_x = torch.empty(qm.qmoe_matvec_expanded_workspace_bytes(c.rows, c.k, 1), dtype=torch.uint8, device=dev)
        t_ = {}
        for label, fn, w_ in (("fused", qm.qmoe_matvec, ws_f), ("expand_then_multiply", qm.qmoe_matvec_expanded, ws_x)):
            for _ in range(10):
                fn(fmt_x, c.rows, c.k, m.w, m.cb, c.rot, x1, y1, w_)
            with Timer(torch) as tm:
                for _ in range(K):
                    fn(fmt_x, c.rows, c.k, m.w, m.cb, c.rot, x1, y1, w_)
            t_[label] = tm.ms / K * 1e3
        res[f"matvec_fusion_{name}"] = {"fused_us": round(t_["fused"], 2),
                                         "expand_then_multiply_us": round(t_["expand_then_multiply"], 2),
                                         "fused_speedup": round(t_["expand_then_multiply"] / t_["fused"], 2)}
        log(f"matvec {name} q=1: fused {t_['fused']:.2f} us, expand-then-multiply "
            f"{t_['expand_then_multiply']:.2f} us ({t_['expand_then_multiply'] / t_['fused']:.2f}x)")

    # ---------------------------------------------------------------- weight quantizer
    res["quantize_fp2"] = bench_quantize(torch, qm, gen, dev)
    res["quantize_fp3"] = bench_quantize(torch, qm, gen, dev, fmt=3, rows=4096, k=2048)

    # ---------------------------------------------------------------- FP2 512x256 matvec latency
    c = gen.fp2_matvec(0)
    m = qm.device.DeviceMatrix(c)
    x = torch.from_numpy(c.x).to(dev)
    y = torch.empty((1, 512), dtype=torch.float32, device=dev)
    w = m.workspace(1)
    for _ in range(10):
        qm.qmoe_matvec(2, 512, 256, m.w, m.cb, 0, x, y, w)
    with Timer(torch) as t:
        for _ in range(K):
            qm.qmoe_matvec(2, 512, 256, m.w, m.cb, 0, x, y, w)
    res["fp2_matvec_512x256"] = {"us_per_call": round(t.ms / K * 1e3, 2)}
    return res


def bench_dense(args, torch, qm, gen, dev, res):
    """The dense FP4 4096x16384 + FP3/H32 4096x2048 mix at 1 and 4 columns: one
    qmoe_matvec_group call (one launch at one column: every workgroup quantizes
    its matrix's input into LDS; two at four: both inputs quantized, then both
    matrices' rows), and as the ablation one qmoe_matvec per matrix (three
    launches: the 16384-long input is quantized in a launch of its own).
    Returns the last (FP4, FP3) cases."""
    K = max(20, args.steps // 2)
    for ncols in (1, 4):
        fp4, fp3 = gen.dense_mix(ncols, seed=0)
        mats = [qm.device.DeviceMatrix(c) for c in (fp4, fp3)]
        xs = [torch.from_numpy(c.x).to(dev) for c in (fp4, fp3)]
        ys = [torch.empty((ncols, c.rows), dtype=torch.float32, device=dev) for c in (fp4, fp3)]
        wss = [m.workspace(ncols) for m in mats]
        items = [(c.fmt, c.rows, c.k, m.w, m.cb, c.rot, x, y) for c, m, x, y in zip((fp4, fp3), mats, xs, ys)]
        arr = qm.matvec_items(items)   # marshalled once: the timed loop is the C call alone
        gws = torch.empty(qm.qmoe_matvec_group_workspace_bytes(items, ncols), dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream().cuda_stream

        def step():
            st = qm.LIB.qmoe_matvec_group(arr, len(items), ncols, gws.data_ptr(), gws.numel(), stream)
            if st:
                raise qm.QmoeError(st, "qmoe_matvec_group", qm.LIB.qmoe_last_error().decode())

        def step_per_matrix():
            for m, c, x, y, w in zip(mats, (fp4, fp3), xs, ys, wss):
                qm.qmoe_matvec(c.fmt, c.rows, c.k, m.w, m.cb, c.rot, x, y, w)
        nbytes = sum(m.w.numel() for m in mats)
        out = {}
        for name, f in (("group", step), ("per_matrix", step_per_matrix)):
            for _ in range(10):
                f()
            with Timer(torch) as t:
                for _ in range(K):
                    f()
            out[name] = t.ms / K
        ms = out["group"]
        gbs = nbytes / (ms * 1e-3) / 1e9
        qm.qmoe_timing_enable(True)
        for _ in range(K):
            step()
        torch.cuda.synchronize()
        kern = {}
        for n in ("group_fq", "group_quant", "group_mvl", "group_mv"):   # one launch (group_fq) or two
            avg, cnt = kernel_avg_ms(qm, n)
            if cnt:
                kern[n] = round(avg * 1e3, 2)
        qm.qmoe_timing_enable(False)
        res[f"dense_mix_q{ncols}"] = {"us_per_step": round(ms * 1e3, 2), "effective_GBps": round(gbs, 1),
                                      "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "packed_bytes": nbytes,
                                      "kernel_us": kern, "entry_point": "qmoe_matvec_group",
                                      "per_matrix_calls_us": round(out["per_matrix"] * 1e3, 2)}
        log(f"dense mix q={ncols}: {ms * 1e3:.2f} us, {gbs:.1f} GB/s (one qmoe_matvec per matrix: "
            f"{out['per_matrix'] * 1e3:.2f} us); kernels (us): " + ", ".join(f"{k}={v}" for k, v in kern.items()))

    return fp4, fp3


def bench_probes(torch, qm, dev):
    """Measured denominators from the library's probe kernels (qmoe_probe_*):
    the sustained read-only HBM rate, the cost of one cold streaming launch of B
    bytes (fitted as latency + B / rate), the int8 matrix-core rate alone (both
    MFMA forms) and the vector-ALU rate of the prefill GEMMs' per-block epilogue
    (convert + fused multiply-add), which bounds those GEMMs at
    64 int8 ops per epilogue element-block."""
    res = {}
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    n = 1 << 30
    buf = torch.ones(n // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    best, per_grid = 0.0, {}
    for grid in (cu, 2 * cu, 4 * cu, 8 * cu, 16 * cu):
        for _ in range(2):
            qm.qmoe_probe_read(buf, grid, sink)
        with Timer(torch) as t:
            for _ in range(10):
                qm.qmoe_probe_read(buf, grid, sink)
        gbs = 10 * n / (t.ms * 1e-3) / 1e9
        per_grid[str(grid)] = round(gbs, 1)
        best = max(best, gbs)
    # the same over a 1 GiB device copy (bytes read + written), for reference
    dst = torch.empty_like(buf)
    dst.copy_(buf)
    with Timer(torch) as t:
        for _ in range(10):
            dst.copy_(buf)
    copy_gbs = 2 * 10 * n / (t.ms * 1e-3) / 1e9
    del dst
    res["stream_read"] = {"peak_GBps": round(best, 1), "bytes": n, "GBps_by_grid": per_grid,
                          "frac_hbm_peak": round(best / HBM_PEAK_GBS, 4),
                          "device_copy_read_plus_write_GBps": round(copy_gbs, 1)}
    log(f"probe: read-only stream {best:.1f} GB/s (by grid {per_grid}); 1 GiB copy {copy_gbs:.1f} GB/s")

    # one cold launch per size: a 512 MiB read of another buffer first evicts the
    # last-level cache (clean lines), then one probe launch reads B bytes at a
    # fresh offset; the kernel's own time from in-dispatch events
    flush = torch.ones((512 << 20) // 4, dtype=torch.int32, device=dev)
    sizes = [2097152, 5242880, 22020096, 31457280, 53477376, 134217728]
    pts = []
    for B in sizes:
        ts = []
        for rep in range(6):
            off = ((rep * 7 + 3) * (64 << 20)) % (n - B) // 256 * 64   # int32 elements, 256-byte aligned
            view = buf[off: off + B // 4]
            qm.qmoe_probe_read(flush, 0, sink)
            qm.qmoe_timing_enable(True)
            qm.qmoe_probe_read(view, 0, sink)
            torch.cuda.synchronize()
            ms, cnt = qm.qmoe_timing_read("probe_read")
            qm.qmoe_timing_enable(False)
            ts.append(ms / cnt)
        pts.append((B, float(np.median(ts))))
    del flush
    A = np.array([[1.0, b] for b, _ in pts])
    y = np.array([t for _, t in pts]) * 1e-3
    (lat, inv_bw), *_ = np.linalg.lstsq(A, y, rcond=None)
    res["cold_launch_read"] = {"us_by_bytes": {str(b): round(t * 1e3, 2) for b, t in pts},
                               "fit_latency_us": round(lat * 1e6, 2), "fit_GBps": round(1.0 / inv_bw / 1e9, 1),
                               "grid": 4 * cu}
    log(f"probe: one cold read launch = {lat * 1e6:.2f} us + B / {1.0 / inv_bw / 1e9:.1f} GB/s "
        f"({ {b: round(t * 1e3, 2) for b, t in pts} } us)")

    # int8 matrix cores alone, and the epilogue's vector-ALU rate
    grid = 4 * cu
    sink2 = torch.empty(grid * 256, dtype=torch.int32, device=dev)
    mf = {}
    for kind, name, mnk in ((0, "k16x16x32", 16 * 16 * 32), (1, "k32x32x32", 32 * 32 * 32)):
        iters = 256
        qm.qmoe_probe_mfma(kind, iters, grid, sink2)
        with Timer(torch) as t:
            for _ in range(5):
                qm.qmoe_probe_mfma(kind, iters, grid, sink2)
        ops = 5 * grid * 4 * iters * 4 * 2 * mnk
        mf[f"{name}_TOPS"] = round(ops / (t.ms * 1e-3) / 1e12, 1)
    mf["frac_spec_peak_k16x16x32"] = round(mf["k16x16x32_TOPS"] / INT8_MFMA_PEAK_TOPS, 4)
    mf["frac_spec_peak_k32x32x32"] = round(mf["k32x32x32_TOPS"] / INT8_MFMA_PEAK_TOPS, 4)
    res["mfma_int8"] = mf
    iters = 8192
    qm.qmoe_probe_valu(iters, grid, sink2)
    with Timer(torch) as t:
        for _ in range(5):
            qm.qmoe_probe_valu(iters, grid, sink2)
    eb = 5 * grid * 256 * iters * 16 / (t.ms * 1e-3)
    res["valu_epilogue"] = {"element_blocks_per_s": round(eb, 1),
                            "fp32_vector_TFLOPs": round(eb * 2 * 2 / 1e12, 1),   # convert + FMA (2 flops)
                            "int8_TOPS_ceiling": round(eb * 64 / 1e12, 1)}
    log(f"probe: int8 MFMA {mf}; epilogue {eb:.3e} element-blocks/s -> ceiling {eb * 64 / 1e12:.1f} TOPS")
    del buf, sink, sink2
    return res


def bench_layer_stack(torch, qm, gen, spec, per_expert, dev, n_layers=8, reps=25):
    """Decode q=1 through n_layers distinct full-size layers (each its own seeded
    weights and its own token), all captured in one HIP graph and replayed: the
    steady state of a model whose layers stream their experts from HBM one after
    another (nothing is reused across layers: 8 x 2.28 GB of experts)."""
    layers = [qm.device.DeviceLayer(spec, seed=200 + i) for i in range(n_layers)]
    xs = [torch.from_numpy(gen.tokens(1, spec.hidden, seed=200 + i, stream=13)).to(dev) for i in range(n_layers)]
    outs = [torch.empty_like(x) for x in xs]
    ws = layers[0].workspace(1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for dl, x, o in zip(layers, xs, outs):
            qm.qmoe_decode_layer(dl.desc, x, o, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for dl, x, o in zip(layers, xs, outs):
            qm.qmoe_decode_layer(dl.desc, x, o, ws)
    for _ in range(3):
        g.replay()
    with Timer(torch) as t:
        for _ in range(reps):
            g.replay()
    us_layer = t.ms / (reps * n_layers) * 1e3
    gbs = spec.topk * per_expert / (us_layer * 1e-6) / 1e9
    # the same layers called eagerly, back to back
    with Timer(torch) as te:
        for _ in range(reps):
            for dl, x, o in zip(layers, xs, outs):
                qm.qmoe_decode_layer(dl.desc, x, o, ws)
    us_eager = te.ms / (reps * n_layers) * 1e3
    del g, layers
    torch.cuda.empty_cache()
    log(f"decode q=1, {n_layers} distinct layers in one graph: {us_layer:.2f} us/layer ({gbs:.1f} GB/s); "
        f"eager {us_eager:.2f} us/layer")
    return {"layers": n_layers, "us_per_layer_graph": round(us_layer, 2), "us_per_layer_eager": round(us_eager, 2),
            "effective_GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "distinct_packed_bytes": n_layers * spec.n_experts * per_expert}


def bench_quantize(torch, qm, gen, dev, fmt=2, n=16, rows=2048, k=4096, iters=8):
    """qmoe_quantize of n fp32 matrices (N(0, 0.02) with 0.1% outliers), 8 Lloyd
    iterations: FP2 on the gate and up matrices of 8 experts (16 x 2048 x 4096),
    FP3 on the down matrices of 16 experts (16 x 4096 x 2048). Algorithmic HBM
    bytes per weight: norm 4 (fp32 in) + 2 (int16 out) + 1/16 (scale); assign 2
    per iteration; pack 2 + 1/16 in, block bytes / 32 out."""
    bb = {2: 10, 3: 14, 4: 17}[fmt]
    w = torch.from_numpy(gen.float_matrices(n, rows, k, seed=0)).to(dev)
    out = torch.empty((n, rows, (k // 32) * bb), dtype=torch.uint8, device=dev)
    cb = torch.empty((n, 1 << fmt), dtype=torch.int8, device=dev)
    ws = torch.empty(qm.qmoe_quantize_workspace_bytes(n, rows, k), dtype=torch.uint8, device=dev)
    qm.qmoe_quantize(fmt, w, iters, out, cb, ws)
    torch.cuda.synchronize()
    reps = 5
    with Timer(torch) as t:
        for _ in range(reps):
            qm.qmoe_quantize(fmt, w, iters, out, cb, ws)
    ms = t.ms / reps
    qm.qmoe_timing_enable(True)
    for _ in range(reps):
        qm.qmoe_quantize(fmt, w, iters, out, cb, ws)
    torch.cuda.synchronize()
    nw = n * rows * k
    per_w = {"qz_norm": 4 + 2 + 2 / 32, "qz_assign": 2.0, "qz_pack": 2 + 2 / 32 + bb / 32}
    kern = {}
    for name in ("qz_norm", "qz_assign", "qz_update", "qz_pack"):
        avg, _ = kernel_avg_ms(qm, name)
        if avg:
            e = {"us": round(avg * 1e3, 2)}
            if name in per_w:
                gbs = per_w[name] * nw / (avg * 1e-3) / 1e9
                e.update({"GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
            kern[name] = e
    qm.qmoe_timing_enable(False)
    res = {"ms_per_call": round(ms, 3), "matrices": n, "shape": [rows, k], "iters": iters,
           "weights_per_s": round(nw / (ms * 1e-3), 1), "fp32_input_GBps": round(4 * nw / (ms * 1e-3) / 1e9, 1),
           "kernels": kern}
    log(f"quantize FP{fmt} {n}x{rows}x{k}, {iters} iters: {ms:.3f} ms; kernels: {kern}")
    del w, out, ws
    return res


def bench_prefill(torch, qm, gen, spec, dl, dev):
    T = 8192
    bias = gen.zipf_bias(spec.n_experts)
    bias_d = torch.from_numpy(bias).to(dev)
    desc = qm.make_layer(spec.hidden, spec.inter, spec.n_experts, spec.topk, spec.fmt_gate, spec.fmt_up,
                         spec.fmt_down, spec.rot_gateup, spec.rot_down, dl.w_router, bias_d, dl.gate, dl.up,
                         dl.down, dl.cb_gate, dl.cb_up, dl.cb_down)
    x = torch.from_numpy(gen.tokens(T, spec.hidden, seed=0, stream=9)).to(dev)
    out = torch.empty_like(x)
    ws = torch.zeros(qm.qmoe_workspace_bytes(desc, T), dtype=torch.uint8, device=dev)
    qm.qmoe_prefill_layer(desc, x, out, ws)
    torch.cuda.synchronize()
    reps = 5
    with Timer(torch) as t:
        for _ in range(reps):
            qm.qmoe_prefill_layer(desc, x, out, ws)
    ms = t.ms / reps
    ops = 2.0 * T * spec.topk * 3 * spec.hidden * spec.inter
    tops = ops / (ms * 1e-3) / 1e12
    qm.qmoe_timing_enable(True)
    for _ in range(reps):
        qm.qmoe_prefill_layer(desc, x, out, ws)
    torch.cuda.synchronize()
    kern = {}
    for name in ("quant_act", "router", "topk", "group_count", "group_scan", "group_scatter", "gateup_mfma",
                 "down_mfma", "gateup_small", "down_small", "combine"):
        avg, _ = kernel_avg_ms(qm, name)
        if avg:
            kern[name] = round(avg * 1e3, 1)
    qm.qmoe_timing_enable(False)
    # the expert products of both branches: MFMA tiles and the matvec path of the
    # experts with at most four pairs
    gemm_ms = sum(kern.get(k, 0) for k in ("gateup_mfma", "down_mfma", "gateup_small", "down_small")) / 1e3
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None
    lay = qm.qmoe_workspace_layout(desc, T)
    E = spec.n_experts
    counts = ws[lay["group"]: lay["group"] + 4 * E].cpu().numpy().view(np.int32)
    th = qm.PREFILL_SMALL_DEFAULT
    small = (counts >= 1) & (counts <= th)
    branches = {"small_threshold": th, "mfma_experts": int(np.count_nonzero(counts > th)),
                "mfma_pairs": int(counts[counts > th].sum()), "small_experts": int(np.count_nonzero(small)),
                "small_pairs": int(counts[small].sum()), "mfma_tiles_of_64": int(np.sum((counts[counts > th] + 63) // 64))}
    log(f"prefill 8K: {ms:.3f} ms, {T / (ms * 1e-3):.0f} tok/s, {tops:.1f} TOPS; kernels (us): "
        + ", ".join(f"{k}={v}" for k, v in kern.items()))
    return {"ms_per_call": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1), "int8_TOPS": round(tops, 2),
            "frac_int8_mfma_peak": round(tops / INT8_MFMA_PEAK_TOPS, 4), "kernel_us": kern,
            "gemm_int8_TOPS": round(gemm_tops, 2) if gemm_tops else None, "branches": branches,
            "gemm_frac_int8_mfma_peak": round(gemm_tops / INT8_MFMA_PEAK_TOPS, 4) if gemm_tops else None}


def bench_prefill_small_sweep(torch, qm, gen, spec, dl, dev):
    """Prefill time against qmoe_prefill_layer_ex's small-expert threshold (0 = all
    experts on MFMA tiles) for 32 .. 8192 tokens, with and without the Zipf(1.1)
    router bias. The thresholds are timed in rounds that alternate their order
    (medians of 6 rounds), since the first timing after a change of input runs
    slow."""
    bias = torch.from_numpy(gen.zipf_bias(spec.n_experts)).to(dev)
    rows = []
    for zipf in (True, False):
        desc = qm.make_layer(spec.hidden, spec.inter, spec.n_experts, spec.topk, spec.fmt_gate, spec.fmt_up,
                             spec.fmt_down, spec.rot_gateup, spec.rot_down, dl.w_router, bias if zipf else None,
                             dl.gate, dl.up, dl.down, dl.cb_gate, dl.cb_up, dl.cb_down)
        for T in (32, 128, 512, 2048, 8192):
            x = torch.from_numpy(gen.tokens(T, spec.hidden, seed=0, stream=9)).to(dev)
            out = torch.empty_like(x)
            ws = torch.zeros(qm.qmoe_workspace_bytes(desc, T), dtype=torch.uint8, device=dev)
            thresholds = (0, 1, 2, 4)
            samples = {sp: [] for sp in thresholds}
            for _ in range(3):
                qm.qmoe_prefill_layer_ex(desc, x, out, ws, 0)
            for rnd in range(6):
                for sp in (thresholds if rnd % 2 == 0 else thresholds[::-1]):
                    reps = 10 if T <= 2048 else 3
                    qm.qmoe_prefill_layer_ex(desc, x, out, ws, sp)
                    with Timer(torch) as t:
                        for _ in range(reps):
                            qm.qmoe_prefill_layer_ex(desc, x, out, ws, sp)
                    samples[sp].append(t.ms / reps * 1e3)
            lay = qm.qmoe_workspace_layout(desc, T)
            counts = ws[lay["group"]: lay["group"] + 4 * spec.n_experts].cpu().numpy().view(np.int32)
            row = {"zipf": zipf, "tokens": T, "us_median_by_threshold": {sp: round(float(np.median(v)), 1)
                                                                         for sp, v in samples.items()},
                   "experts_1_to_4_pairs": int(((counts >= 1) & (counts <= 4)).sum()),
                   "experts_over_4_pairs": int((counts > 4).sum())}
            log(f"prefill small-expert sweep: {row}")
            rows.append(row)
    return rows


def oracle_threads():
    """Host threads for the oracle: the process's CPU affinity, at most 16 (one
    GPU's share of the host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _pmap(fn, items, n):
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(n) as ex:
        return list(ex.map(fn, items))


def cpu_baseline(args, spec, dl, per_expert, extra):
    """The oracle (numpy, fp64; never tuned) timed on bounded samples of the
    benchmark's workloads. Tokens (and the columns of a dense call) are
    independent, so the multi-threaded legs hand whole tokens to a thread pool
    of the affinity core count; numpy's array arithmetic releases the
    interpreter lock. Input generation is not timed. The headline leg (q=1
    decode, the same layer and tokens as the GPU headline) is the returned
    baseline; the others go to extra["cpu_oracle"]."""
    from threadpoolctl import threadpool_limits

    from oracle import dots, moe, router
    from synth import gen

    nt = oracle_threads()
    n = args.cpu_sample_tokens
    cache = {}

    def get(name, e):
        if (name, e) not in cache:
            t = gen.expert_tensor(spec, name, e, 0)
            cache[(name, e)] = (t.fmt, t.codes, t.scales, t.cb)
        return cache[(name, e)]

    def prepare(L, xs):
        idx, _, _ = router.route(L.w_router, xs, L.bias, spec.topk)
        _pmap(lambda ne: get(*ne), sorted({(nm, int(e)) for e in np.unique(idx) for nm in ("gate", "up", "down")}), nt)

    def run_tokens(L, xs, threads):
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            if threads == 1:
                moe.moe_tokens(L, xs)
            else:
                _pmap(lambda t: moe.moe_tokens(L, xs[t:t + 1]), range(xs.shape[0]), threads)
            return time.perf_counter() - t0

    legs = {}
    # q = 1 decode: the headline layer and its rotating tokens
    L = moe.Layer(spec.hidden, spec.inter, spec.n_experts, spec.topk, dl.w_router_host, get)
    # the GPU headline rotates the first 64 of these tokens; the sample continues the same stream
    x = gen.tokens(max(64, n), spec.hidden, seed=0, stream=7)[:n]
    n = x.shape[0]
    n1 = max(1, n // 8)
    prepare(L, x)
    dt = run_tokens(L, x, nt)
    dt1 = run_tokens(L, x[:n1], 1)
    gbs = n * spec.topk * per_expert / dt / 1e9
    gbs1 = n1 * spec.topk * per_expert / dt1 / 1e9
    legs["decode_q1"] = {"GBps": round(gbs, 5), "threads": nt, "tokens": n, "s": round(dt, 2),
                         "single_thread_GBps": round(gbs1, 5), "single_thread_tokens": n1,
                         "single_thread_s": round(dt1, 2)}
    log(f"cpu oracle: decode q=1 {n} tokens on {nt} threads {dt:.1f}s ({gbs:.4f} GB/s); "
        f"{n1} tokens on 1 thread {dt1:.1f}s ({gbs1:.4f} GB/s)")
    # q = 4 decode: two forced-overlap groups (each token independent)
    groups = [gen.q4_group(spec.hidden, seed=0, variant=v) for v in range(2)]
    xg = np.concatenate(groups)
    prepare(L, xg)
    dt = run_tokens(L, xg, nt)
    legs["decode_q4"] = {"tokens_per_s": round(xg.shape[0] / dt, 3), "threads": nt, "groups": len(groups),
                         "s": round(dt, 2)}
    # 8K prefill: a sample of the Zipf-biased batch's tokens through the per-token oracle
    bias = gen.zipf_bias(spec.n_experts)
    Lb = moe.Layer(spec.hidden, spec.inter, spec.n_experts, spec.topk, dl.w_router_host, get, bias)
    xp = gen.tokens(8192, spec.hidden, seed=0, stream=9)[::256]
    prepare(Lb, xp)
    dt = run_tokens(Lb, xp, nt)
    legs["prefill_8k_sample"] = {"tokens_per_s": round(xp.shape[0] / dt, 3), "threads": nt,
                                 "sample": f"{xp.shape[0]} of the 8192 tokens (every 256th), per-token oracle",
                                 "s": round(dt, 2)}
    cache.clear()
    # dense mix q = 1 and q = 4: the oracle matvec, one column per thread
    for ncols in (1, 4):
        mats = gen.dense_mix(ncols, seed=0)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            for c in mats:
                _pmap(lambda j: dots.matvec(c.fmt, c.codes, c.scales, c.cb, c.x[j:j + 1], c.rot), range(ncols),
                      min(nt, ncols))
            dt = time.perf_counter() - t0
        nbytes = sum(c.rows * (c.k // 32) * {2: 10, 3: 14, 4: 17}[c.fmt] for c in mats)
        legs[f"dense_mix_q{ncols}"] = {"GBps": round(nbytes / dt / 1e9, 5), "threads": min(nt, ncols),
                                       "s": round(dt, 2)}
        del mats
    log("cpu oracle legs: " + json.dumps(legs))
    extra["cpu_oracle"] = legs
    h = legs["decode_q1"]
    return {"value": h["GBps"], "unit": "GB/s", "cores": nt, "kind": "oracle",
            "sample": f"{n} q=1 decode tokens of the same layer (routing + 6 experts each) on a pool of {nt} "
                      f"threads, {h['s']} s; numpy int64/fp64; single thread: {h['single_thread_GBps']} GB/s "
                      f"on {h['single_thread_tokens']} tokens"}


if __name__ == "__main__":
    main()
