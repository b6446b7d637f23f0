#!/usr/bin/env python3
"""Benchmark of the W4A16 MoE hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
routing align (topk_ids -> sorted_ids / expert_ids / num_tokens_padded), the
gate/up W4A16 GEMM (per routed slot), and the down W4A16 GEMM with the
top-k-weighted combine.  Inputs and packed weights are resident in HBM before
the timed region.  Default workload: the EP8 decode share of a Kimi K2.x MoE
layer (48 of 384 experts, top-8, 576 tokens, hidden 7168, intermediate 2048).

Prints one JSON line (rank 0).  `value` is the step's weight+scale bytes
(experts touched by the batch, both projections) over the step time, in GB/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA
# Measured HBM traffic of the gate/up GEMM (rocprofv3 FETCH_SIZE / WRITE_SIZE
# per dispatch, scaled by a copy of known size); valid only for the kernel
# sources it was taken on, identified by their hash.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "moe_gemm_ep8_decode_traffic.md")
KERNEL_SOURCES = ["w4a16_int4_mixture_moe_amd/csrc/gemm.hip", "w4a16_int4_mixture_moe_amd/csrc/tile_common.hpp",
                  "w4a16_int4_mixture_moe_amd/csrc/device_common.hpp",
                  "w4a16_int4_mixture_moe_amd/csrc/launch.hpp", "w4a16_int4_mixture_moe_amd/build.py"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(n_touched: int, N: int, K: int) -> int:
    """Packed INT4 weights (K/2 bytes per row) + bf16 group-32 scales."""
    return n_touched * (N * K // 2 + N * (K // 32) * 2)


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, cfg_tag: str):
    """HBM bytes per gate/up launch from the committed counter summary, or
    None when there is none for this workload and config or the kernel
    sources changed since the counters were taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    import re
    m = re.search(r"<!-- traffic: (\{.*?\}) -->", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("workload") != workload or rec.get("config") != cfg_tag:
        return None
    if rec.get("sources_sha256") != kernel_sources_sha256():
        return None
    return int(round(rec["fetch_kib"] * 1024 * rec["fetch_factor"] + rec["write_kib"] * 1024 * rec["write_factor"]))


def copy_calibration() -> int:
    """A plain device copy of 1 GiB, three times: the reference that scales
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    x = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": x.numel() * 4, "copies": 3}), flush=True)
    return 0


def cpu_baseline(sh, ids, wts, x, a, c1, s1, c2, s2, n_experts: int) -> dict:
    """The oracle's fp32 path (dequantise, sgemm, combine), untuned, on the
    first `n_experts` local experts and all rows routed to them."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    S = n_experts
    t0 = time.perf_counter()
    O.indexed_gate_up_fp32(x, c1[:S], s1[:S], ids, sh.first, S)
    t1 = time.perf_counter()
    O.indexed_down_combine_fp32(a, c2[:S], s2[:S], ids, wts, sh.first, S)
    t2 = time.perf_counter()
    dt = t2 - t0
    flat = ids.reshape(-1)
    rows = int(((flat >= sh.first) & (flat < sh.first + S)).sum())
    b = weight_bytes(S, sh.N1, sh.K1) + weight_bytes(S, sh.N2, sh.K2)
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3), "gate_up_seconds": round(t1 - t0, 3), "down_combine_seconds": round(t2 - t1, 3),
            "sample": f"gate/up + down+combine for local experts 0..{S - 1} of {sh.E_loc} "
                      f"({rows} routed rows), same inputs as the GPU step; GB/s of weight+scale bytes"}


def mx_weight_bytes(n_touched: int, N: int, K: int) -> int:
    """MXFP4 weights (K/2 bytes per row) + one E8M0 byte per 32 K."""
    return n_touched * (N * K // 2 + N * (K // 32))


def cpu_baseline_mx(sh, ids, wts, x, a, w1, s1, w2, s2, n_experts: int) -> dict:
    """The MXFP4 oracle as it stands (quantise the step's activation rows,
    dequantise, float64 matmul, combine) on the first `n_experts` local
    experts and all rows routed to them."""
    from oracle import mx_oracle as X
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    S = n_experts
    t0 = time.perf_counter()
    xq = X.mx_quantize(x)
    aq = X.mx_quantize(a)
    t1 = time.perf_counter()
    X.mx_indexed_gate_up(*xq, X.unpack_nibbles(w1[:S]), s1[:S], ids, sh.first, S)
    t2 = time.perf_counter()
    X.mx_indexed_down_combine(*aq, X.unpack_nibbles(w2[:S]), s2[:S], ids, wts, sh.first, S)
    t3 = time.perf_counter()
    dt = t3 - t0
    flat = ids.reshape(-1)
    rows = int(((flat >= sh.first) & (flat < sh.first + S)).sum())
    b = mx_weight_bytes(S, sh.N1, sh.K1) + mx_weight_bytes(S, sh.N2, sh.K2)
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "quantise_seconds": round(t1 - t0, 3), "gate_up_seconds": round(t2 - t1, 3),
            "down_combine_seconds": round(t3 - t2, 3),
            "sample": f"A4W4: quantise all activation rows, gate/up + down+combine for local experts "
                      f"0..{S - 1} of {sh.E_loc} ({rows} routed rows), same inputs as the GPU step; "
                      f"GB/s of MXFP4 weight+scale bytes"}


def bench_grouped(args, sh, M, W, dev) -> int:
    """The grouped gate/up GEMMs on skewed routing: the contiguous layout
    (each expert's rows padded to 128, m_indices -1 on padding) and the
    masked one ([E, max_m, K] with masked_m counts).  A step is one call of
    each, replayed as a HIP graph; the metric is MFMA TFLOP/s on valid rows,
    the gate/up weights being read once per 128-row block (prefill side)."""
    import torch

    t_gen = time.perf_counter()
    ids, _ = W.routing_for(sh)
    x = W.activations(sh.seed, "x", sh.T, sh.K1)
    c1 = W.weight_codes(sh.seed, "w1_codes", sh.E_loc, sh.N1, sh.K1)
    s1 = W.weight_scales(sh.seed, "w1_scales", sh.E_loc, sh.N1, sh.K1)
    A, mi, _ = W.contiguous_layout(ids, x, sh.first, sh.E_loc, pad=128, pad_fill=0)
    A3, mm, _, dropped = W.masked_layout(ids, x, sh.first, sh.E_loc, sh.max_m, pad_fill=0)
    log(f"inputs generated in {time.perf_counter() - t_gen:.1f}s")

    def bf(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)

    p1 = M.pack_w4(torch.from_numpy(c1).to(dev), bf(s1))
    d_A, d_A3 = bf(A), bf(A3)
    d_mi = torch.from_numpy(mi.astype(np.int32)).to(dev)
    d_mm = torch.from_numpy(mm.astype(np.int32)).to(dev)
    expected_m = max(1, int(round(float(mm.mean()))))
    out_c = torch.empty(A.shape[0], sh.N1, dtype=torch.bfloat16, device=dev)
    out_m = torch.empty(A3.shape[0] * A3.shape[1], sh.N1, dtype=torch.bfloat16, device=dev)

    def contiguous():
        M.grouped_contiguous(d_A, p1, d_mi, out=out_c)

    def masked():
        M.grouped_masked(d_A3, p1, d_mm, expected_m, out=out_m)

    def step():
        contiguous()
        masked()

    def graph_of(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        return g

    stream = torch.cuda.current_stream(dev)

    def replay_us(g, reps, per):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        g.replay()
        torch.cuda.synchronize()
        for a_, b_ in ev:
            a_.record(stream)
            g.replay()
            b_.record(stream)
        torch.cuda.synchronize()
        t = np.array([a_.elapsed_time(b_) * 1e3 / per for a_, b_ in ev])
        return float(t.mean()), float(np.median(t)), float(t.min()), float(np.percentile(t, 90))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    g_step = graph_of(step, 1)
    for _ in range(args.warmup):
        g_step.replay()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        g_step.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    inner = 4
    st_c = replay_us(graph_of(contiguous, inner), max(4, args.steps // 4), inner)
    st_m = replay_us(graph_of(masked, inner), max(4, args.steps // 4), inner)

    # cold calls: a 1 GiB read before each leaves no useful line in any cache
    flush_buf = torch.zeros(1 << 28, dtype=torch.int32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.int32, device=dev)

    def cold(fn, reps=10):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a_, b_ in ev:
            torch.amax(flush_buf, dim=0, out=flush_sink)
            a_.record(stream)
            fn()
            b_.record(stream)
        torch.cuda.synchronize()
        t = np.array([a_.elapsed_time(b_) * 1e3 for a_, b_ in ev])
        return float(np.median(t)), float(t.min()), float(np.percentile(t, 90))
    cold_c, cold_m = cold(contiguous), cold(masked)
    del flush_buf

    fl_row = 2.0 * sh.N1 * sh.K1
    valid_c = int((mi >= 0).sum())
    valid_m = int(mm.sum())
    tf = lambda rows, us: rows * fl_row / (us * 1e-6) / 1e12
    tf_c = tf(valid_c, st_c[0])
    value = (valid_c + valid_m) * fl_row / (ms_step * 1e-3) / 1e12
    out = {
        "metric": "MFMA TFLOP/s on valid rows of the grouped gate/up GEMMs (contiguous and masked layouts, "
                  "one call each per step), with us/call",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "timing": "HIP graph replay of the step",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": sh.name, "variant": "w4a16", "T": sh.T, "topk": sh.topk, "E_glob": sh.E_glob,
                   "E_loc": sh.E_loc, "K1": sh.K1, "N1": sh.N1, "contiguous_rows": int(A.shape[0]),
                   "contiguous_valid_rows": valid_c, "masked_max_m": int(sh.max_m), "masked_valid_rows": valid_m,
                   "masked_dropped_rows": int(dropped), "expected_m": expected_m,
                   "zero_row_experts": int((mm == 0).sum())},
        "per_call_us": {"contiguous": round(st_c[0], 2), "masked": round(st_m[0], 2)},
        "per_call_stats_us": {name: {"median": round(v[1], 2), "min": round(v[2], 2), "p90": round(v[3], 2)}
                              for name, v in (("contiguous", st_c), ("masked", st_m))},
        "per_call_cold_us": {name: {"median": round(v[0], 2), "min": round(v[1], 2), "p90": round(v[2], 2)}
                             for name, v in (("contiguous", cold_c), ("masked", cold_m))},
        "gemm_rates": {
            "contiguous_TFLOPs": round(tf_c, 2),
            "contiguous_TFLOPs_padded_rows": round(tf(int(A.shape[0]), st_c[0]), 2),
            "masked_TFLOPs": round(tf(valid_m, st_m[0]), 2),
            "masked_TFLOPs_all_rows": round(tf(int(A3.shape[0] * A3.shape[1]), st_m[0]), 2),
        },
        "roofline": {"kernel": "moe_gemm_kernel (grouped contiguous gate/up)", "bound": "mfma",
                     "achieved": round(tf_c, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf_c / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops": valid_c * fl_row},
    }
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 warmup steps (about 60 ms of GPU work at the decode size): with only a
    # few, the timed region starts before the GPU's clocks have ramped to
    # their steady level and every figure reads 10-20 % slow
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="ep8_decode")
    ap.add_argument("--block-m", type=int, default=0, help="override the selector's block_m")
    ap.add_argument("--nr", type=int, default=0, help="override the selector's weight tiles per wave")
    ap.add_argument("--waves", type=int, default=0, help="override the selector's waves per workgroup")
    ap.add_argument("--split-k", type=int, default=-1, help="override: 0 stream-K, 1 one workgroup per tile")
    ap.add_argument("--stages", type=int, default=0, help="override: K chunks of weights in flight per wave")
    ap.add_argument("--cpu-experts", type=int, default=20, help="experts in the CPU-baseline sample (0: skip)")
    ap.add_argument("--eager", action="store_true", help="launch the step eagerly instead of replaying a HIP graph")
    ap.add_argument("--fused", action="store_true",
                    help="chained layer: gate/up with the SiLU activation fused, written in sorted order, "
                         "read as is by the down projection (instead of a synthetic per-slot down input)")
    ap.add_argument("--mx", action="store_true",
                    help="A4W4 variant: MXFP4 weights, activations quantised to MXFP4 on the device "
                         "inside the step (quantise x, gate/up, quantise the down input, down+combine)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB three times (reference for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(collectives and sharding are out of scope); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import w4a16_int4_mixture_moe_amd as M
    from synth import workloads as W

    sh = W.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    if sh.name == "grouped_skewed":
        if args.mx or args.fused:
            print("the grouped layouts run the W4A16 gate/up GEMM only (no --mx / --fused)", file=sys.stderr)
            return 2
        return bench_grouped(args, sh, M, W, dev)
    t_gen = time.perf_counter()
    ids, wts = W.routing_for(sh)
    x = W.activations(sh.seed, "x", sh.T, sh.K1)
    a = W.activations(sh.seed, "a", sh.T * sh.topk, sh.K2)
    if args.mx:
        c1 = W.mx_weight_codes(sh.seed, "w1_mx_codes", sh.E_loc, sh.N1, sh.K1)
        s1 = W.mx_weight_scales(sh.seed, "w1_mx_scales", sh.E_loc, sh.N1, sh.K1)
        c2 = W.mx_weight_codes(sh.seed, "w2_mx_codes", sh.E_loc, sh.N2, sh.K2)
        s2 = W.mx_weight_scales(sh.seed, "w2_mx_scales", sh.E_loc, sh.N2, sh.K2)
    else:
        c1 = W.weight_codes(sh.seed, "w1_codes", sh.E_loc, sh.N1, sh.K1)
        s1 = W.weight_scales(sh.seed, "w1_scales", sh.E_loc, sh.N1, sh.K1)
        c2 = W.weight_codes(sh.seed, "w2_codes", sh.E_loc, sh.N2, sh.K2)
        s2 = W.weight_scales(sh.seed, "w2_scales", sh.E_loc, sh.N2, sh.K2)
    log(f"inputs generated in {time.perf_counter() - t_gen:.1f}s")

    def bf(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)

    if args.mx:
        p1 = M.pack_mxfp4(torch.from_numpy(c1).to(dev), torch.from_numpy(s1).to(dev), gate_up=args.fused)
        p2 = M.pack_mxfp4(torch.from_numpy(c2).to(dev), torch.from_numpy(s2).to(dev))
    else:
        p1 = M.pack_w4(torch.from_numpy(c1).to(dev), bf(s1), gate_up=args.fused)
        p2 = M.pack_w4(torch.from_numpy(c2).to(dev), bf(s2))
    d_ids = torch.from_numpy(ids).to(dev)
    d_w = torch.from_numpy(wts).to(dev)
    d_x, d_a = bf(x), bf(a)
    # the selector decides block_m, which fixes the routing alignment
    select = M.mxfp4_select if args.mx else M.select
    cfg = select(sh.T, sh.topk, sh.E_glob, sh.E_loc, sh.N1, sh.K1)
    if args.block_m:
        cfg.block_m = args.block_m
    if args.nr:
        cfg.nr = args.nr
    if args.waves:
        cfg.waves = args.waves
    if args.split_k >= 0:
        cfg.split_k = args.split_k
    if args.stages:
        cfg.stages = args.stages
    T, k = sh.T, sh.topk
    cap = M.align_capacity(T, k, sh.E_loc, cfg.block_m)
    sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    expert_ids = torch.empty(cap // cfg.block_m, dtype=torch.int32, device=dev)
    ntp = torch.empty(1, dtype=torch.int32, device=dev)
    routing = M.Routing(sorted_ids, expert_ids, ntp, cfg.block_m, d_ids, sh.E_glob, sh.first, sh.E_loc)
    h = torch.empty(T * k, sh.N1, dtype=torch.bfloat16, device=dev)
    y = torch.empty(T, sh.N2, dtype=torch.bfloat16, device=dev)
    if args.mx:
        # the A4W4 kernels: four weight tiles per wave, four stages for the
        # decode blocks (overrides apply as for the W4A16 kernels)
        cfg = M.mxfp4_config(cfg.block_m, args.nr or 4, args.stages or None)
        ws1 = torch.empty(16, dtype=torch.uint8, device=dev)
        ws2 = torch.empty(max(16, M.mxfp4_workspace_bytes(p2, T, k, True)), dtype=torch.uint8, device=dev)
        qx = M.MXRows(torch.empty(T, sh.K1 // 2, dtype=torch.uint8, device=dev),
                      torch.empty(T, sh.K1 // 32, dtype=torch.uint8, device=dev))
        qa = M.MXRows(torch.empty(T * k, sh.K2 // 2, dtype=torch.uint8, device=dev),
                      torch.empty(T * k, sh.K2 // 32, dtype=torch.uint8, device=dev))
    else:
        ws1 = torch.empty(max(16, M.workspace_bytes(p1, T, k, False, cfg)), dtype=torch.uint8, device=dev)
        ws2 = torch.empty(max(16, M.workspace_bytes(p2, T, k, True, cfg)), dtype=torch.uint8, device=dev)
    L = M.load()
    stream = torch.cuda.current_stream(dev)
    import ctypes

    def align():
        # current stream looked up per call: under graph capture it is the capture stream
        s_ptr = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        M._lib.check(L.w4a16_moe_align(d_ids.data_ptr(), T, k, sh.E_glob, sh.first, sh.E_loc,
                                       cfg.block_m, sorted_ids.data_ptr(), expert_ids.data_ptr(),
                                       ntp.data_ptr(), cap, 0, s_ptr))

    inter = torch.zeros(cap, sh.N1 // 2, dtype=torch.bfloat16, device=dev) if args.fused and not args.mx else None
    inter_mx = (M.MXRows(torch.zeros(cap, sh.N1 // 4, dtype=torch.uint8, device=dev),
                         torch.zeros(cap, sh.N1 // 64, dtype=torch.uint8, device=dev))
                if args.fused and args.mx else None)
    if args.fused and (sh.K2 != sh.N1 // 2 or cfg.split_k != 1 or cfg.nr % 2 or (args.mx and cfg.nr != 4)):
        log("--fused needs K2 = N1 / 2, split_k = 1 and an even nr (4 with --mx)")
        return 2

    def gate_up():
        if args.mx and args.fused:
            M.moe_mxfp4_gate_up_silu(qx, p1, routing, cfg=cfg, out=inter_mx)
        elif args.mx:
            M.moe_mxfp4_gemm(qx, p1, routing, cfg=cfg, out=h)
        elif args.fused:
            M.moe_gate_up_silu(d_x, p1, routing, cfg=cfg, out=inter)
        else:
            M.moe_w4a16_gemm(d_x, p1, routing, cfg=cfg, out=h, workspace=ws1)

    def down():
        if args.mx and args.fused:
            M.moe_mxfp4_gemm(inter_mx, p2, routing, topk_weights=d_w, a_layout="sorted", cfg=cfg, out=y,
                             workspace=ws2)
        elif args.mx:
            M.moe_mxfp4_gemm(qa, p2, routing, topk_weights=d_w, cfg=cfg, out=y, workspace=ws2)
        elif args.fused:
            M.moe_w4a16_gemm(inter, p2, routing, topk_weights=d_w, a_layout="sorted", cfg=cfg, out=y,
                             workspace=ws2)
        else:
            M.moe_w4a16_gemm(d_a, p2, routing, topk_weights=d_w, cfg=cfg, out=y, workspace=ws2)

    def quant():
        # A4W4: the activation rows to MXFP4 (unfused: also the rows of the
        # step's synthetic per-slot down input that the down GEMM reads, those
        # of local slots; fused: the gate/up epilogue quantises the down input
        # itself)
        M.mxfp4_quant(d_x, out=qx)
        if not args.fused:
            M.mxfp4_quant_local_slots(d_a, routing, out=qa)

    def step():
        align()
        if args.mx:
            M.mxfp4_quant(d_x, out=qx)
        gate_up()
        if args.mx and not args.fused:
            M.mxfp4_quant_local_slots(d_a, routing, out=qa)
        down()

    def graph_of(fn, n):
        """Capture n back-to-back calls of fn in one HIP graph (torch's
        capture stream is the current stream inside the context, so the
        library's launches land in the graph)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        return g

    def timed(g, reps, per):
        """Per-call duration: replay g (per calls back to back) `reps` times,
        each replay between two events on the stream the kernels run on.
        Returns (mean, median, min, p90) of the per-call averages, in us."""
        s_ = torch.cuda.current_stream(dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        g.replay()
        torch.cuda.synchronize()
        for a_, b_ in ev:
            a_.record(s_)
            g.replay()
            b_.record(s_)
        torch.cuda.synchronize()
        t = np.array([a_.elapsed_time(b_) * 1e3 / per for a_, b_ in ev])
        return float(t.mean()), float(np.median(t)), float(t.min()), float(np.percentile(t, 90))

    def cold(fn, reps):
        """Per-call duration with every cache cold: before each call a
        1 GiB read (far beyond the 256 MB last-level cache) evicts whatever
        the previous call left, leaving only clean lines (a writing flush
        would leave the call to compete with their write-back); events
        bracket the call alone on its stream.  Returns (median, min, p90)
        in us."""
        s_ = torch.cuda.current_stream(dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a_, b_ in ev:
            torch.amax(flush_buf, dim=0, out=flush_sink)
            a_.record(s_)
            fn()
            b_.record(s_)
        torch.cuda.synchronize()
        t = np.array([a_.elapsed_time(b_) * 1e3 for a_, b_ in ev])
        return float(np.median(t)), float(t.min()), float(np.percentile(t, 90))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    use_graph = not args.eager
    if use_graph:
        g_step = graph_of(step, 1)
        for _ in range(args.warmup):
            g_step.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        if use_graph:
            g_step.replay()
        else:
            step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    # per-kernel averages: each call replayed back to back inside one graph
    inner = 8
    st_align = timed(graph_of(align, inner), max(4, args.steps // 2), inner)
    st_gu = timed(graph_of(gate_up, inner), max(4, args.steps // 2), inner)
    st_dn = timed(graph_of(down, inner), max(4, args.steps // 2), inner)
    st_q = timed(graph_of(quant, inner), max(4, args.steps // 2), inner) if args.mx else None
    us_align, us_gu, us_dn = st_align[0], st_gu[0], st_dn[0]
    flush_buf = torch.zeros(1 << 28, dtype=torch.int32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.int32, device=dev)
    cold_reps = 20
    st_cold = {"align": cold(align, cold_reps), "gate_up": cold(gate_up, cold_reps),
               "down_combine": cold(down, cold_reps)}
    del flush_buf, flush_sink

    # host cost of choosing a config (first call runs the sampled search,
    # later calls hit the memoised result) and of one launch (binding +
    # argument checks + kernel enqueue), no device time
    def host_us(fn, reps):
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        return (time.perf_counter() - t0) / reps * 1e6
    probe_T = T + 1                                        # a shape the run has not selected for yet
    t0 = time.perf_counter()
    M.select(probe_T, k, sh.E_glob, sh.E_loc, sh.N1, sh.K1)
    host_select_first = (time.perf_counter() - t0) * 1e6
    host_select_memo = host_us(lambda: M.select(probe_T, k, sh.E_glob, sh.E_loc, sh.N1, sh.K1), 200)
    host_launch = host_us(gate_up, 50)
    torch.cuda.synchronize()

    flat = ids.reshape(-1)
    local = (flat >= sh.first) & (flat < sh.first + sh.E_loc)
    n_local = int(local.sum())
    touched = int(len(np.unique(flat[local])))
    tokens_with_local = int(local.reshape(T, k).any(1).sum())
    wbytes = mx_weight_bytes if args.mx else weight_bytes
    wb1 = wbytes(touched, sh.N1, sh.K1)
    wb2 = wbytes(touched, sh.N2, sh.K2)
    n_ntp = int(ntp.item())
    # algorithmic bytes per gate/up launch: weights+scales of touched experts,
    # one activation row read and one output row written per routed slot,
    # the routing indices
    # fused: the activation, half the columns (MXFP4 with --mx: codes + scales)
    if args.fused and args.mx:
        out1 = n_local * (sh.N1 // 4 + sh.N1 // 64)
    else:
        out1 = n_local * (sh.N1 // 2 if args.fused else sh.N1) * 2
    row1 = sh.K1 // 2 + sh.K1 // 32 if args.mx else sh.K1 * 2     # MXFP4 row: codes + scales
    alg1 = wb1 + n_local * row1 + out1 + n_ntp * 4 + (n_ntp // cfg.block_m) * 4
    value = (wb1 + wb2) / (ms_step * 1e-3) / 1e9
    cfg_tag = f"bm{cfg.block_m} nr{cfg.nr} waves{cfg.waves} split_k{cfg.split_k} stages{cfg.stages}"
    gu_gbs = alg1 / (us_gu * 1e-6) / 1e9
    flops1 = 2.0 * n_local * sh.N1 * sh.K1
    flops2 = 2.0 * n_local * sh.N2 * sh.K2
    kname = "mx_gemm_kernel (A4W4 gate/up)" if args.mx else "moe_gemm_kernel (gate/up)"
    # the gate/up kernel's bound: HBM below the ridge (routed rows per touched
    # expert where its flops per weight byte reach the matrix peak over 8 TB/s),
    # MFMA above it
    mfma_peak = FP4_PEAK_TFLOPS if args.mx else BF16_PEAK_TFLOPS
    rows_per_expert = n_local / max(touched, 1)
    ridge_rows = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9) * (wb1 / max(touched, 1)) / (2.0 * sh.N1 * sh.K1)
    if rows_per_expert >= ridge_rows:
        tflops1 = flops1 / (us_gu * 1e-6) / 1e12
        roofline = {"kernel": kname, "bound": "mfma", "achieved": round(tflops1, 1), "peak": mfma_peak,
                    "unit": "TFLOP/s", "frac": round(tflops1 / mfma_peak, 4), "traffic": None,
                    "algorithmic_flops": flops1, "rows_per_expert": round(rows_per_expert, 1),
                    "ridge_rows_per_expert": round(ridge_rows, 1)}
    else:
        roofline = {"kernel": kname, "bound": "hbm", "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                    "traffic": None if args.mx else measured_traffic(sh.name, cfg_tag),
                    "algorithmic_bytes": int(alg1), "rows_per_expert": round(rows_per_expert, 1),
                    "ridge_rows_per_expert": round(ridge_rows, 1)}
    out = {
        "metric": ("weight-HBM GB/s of one A4W4 MoE layer step (align + MXFP4 quantisation + gate/up + "
                   "down+combine), with us/call per MXFP4 GEMM") if args.mx else
                  "weight-HBM GB/s of one MoE layer step (align + gate/up + down+combine), "
                  "with us/call per W4A16 GEMM",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "timing": "HIP graph replay of the step" if use_graph else "eager launches",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if args.mx else "bf16",
        "data": "synthetic",
        "config": {"workload": sh.name, "variant": "a4w4-mxfp4" if args.mx else "w4a16",
                   "fused_silu": bool(args.fused), "T": T, "topk": k, "E_glob": sh.E_glob, "E_loc": sh.E_loc,
                   "K1": sh.K1, "N1": sh.N1, "K2": sh.K2, "N2": sh.N2, "block_m": cfg.block_m,
                   "nr": cfg.nr, "waves": cfg.waves, "split_k": cfg.split_k, "stages": cfg.stages, "routed_rows": n_local,
                   "experts_touched": touched, "num_tokens_padded": n_ntp},
        "per_call_stats_us": {name: {"median": round(v[1], 2), "min": round(v[2], 2), "p90": round(v[3], 2)}
                              for name, v in (("align", st_align), ("gate_up", st_gu), ("down_combine", st_dn))},
        "per_call_cold_us": {name: {"median": round(v[0], 2), "min": round(v[1], 2), "p90": round(v[2], 2)}
                             for name, v in st_cold.items()},
        "host_us": {"select_first_call": round(host_select_first, 1), "select_memoised": round(host_select_memo, 2),
                    "gate_up_launch": round(host_launch, 1)},
        "per_call_us": {"align": round(us_align, 2), "gate_up": round(us_gu, 2),
                        "down_combine": round(us_dn, 2)},
        "gemm_rates": {
            "gate_up_weight_GBs": round(wb1 / (us_gu * 1e-6) / 1e9, 1),
            "down_weight_GBs": round(wb2 / (us_dn * 1e-6) / 1e9, 1),
            "gate_up_TFLOPs": round(flops1 / (us_gu * 1e-6) / 1e12, 2),
            "gate_up_TFLOPs_padded_rows": round(2.0 * n_ntp * sh.N1 * sh.K1 / (us_gu * 1e-6) / 1e12, 2),
            "down_TFLOPs": round(flops2 / (us_dn * 1e-6) / 1e12, 2),
        },
        "roofline": roofline,
    }
    if st_q is not None:
        qname = "mxfp4_quant_x" if args.fused else "mxfp4_quant_x_and_a"
        out["per_call_stats_us"][qname] = {"median": round(st_q[1], 2), "min": round(st_q[2], 2),
                                                          "p90": round(st_q[3], 2)}
        out["per_call_us"][qname] = round(st_q[0], 2)
        out["gemm_rates"]["gate_up_fp4_frac"] = round(flops1 / (us_gu * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 4)
    if args.cpu_experts > 0:
        log("timing the CPU oracle baseline ...")
        base = cpu_baseline_mx if args.mx else cpu_baseline
        out["cpu_baseline"] = base(sh, ids, wts, x, a, c1, s1, c2, s2, args.cpu_experts)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
