#!/usr/bin/env python3
"""Benchmark of the W4A16 MoE hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
routing align (topk_ids -> sorted_ids / expert_ids / num_tokens_padded), the
gate/up W4A16 GEMM (per routed slot), and the down W4A16 GEMM with the
top-k-weighted combine.  Inputs and packed weights are resident in HBM before
the timed region.  The headline workload is the EP8 decode share of a Kimi K2.x
MoE layer (48 of 384 experts, top-8, 576 tokens, hidden 7168, intermediate
2048); `value` is the step's weight+scale bytes (experts touched by the batch,
both projections) over the step time, in GB/s.

Without --workload the JSON line also carries `configs`: one record per
synthetic configuration (tiny; EP8 decode; EP8 prefill; the TP8 token sweep;
the skewed grouped layouts), each GEMM with its us/call, its bound (HBM below
the ridge of rows per expert, MFMA above), achieved rate, fraction of the
roofline and the kernel name the rocprofv3 trace shows.  With --workload NAME
only that workload is measured (profiling runs).

Before any timing, each workload's step is replayed for a fixed wall time
(--ramp-ms, default 200 ms) so the GPU clocks are at their steady level
whatever --warmup says; --warmup steps follow as usual.
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
METRIC = "µs/call + weight-HBM GB/s (decode), MFMA TFLOP/s (prefill) per MoE GEMM"
# Measured HBM traffic of the gate/up GEMM (rocprofv3 FETCH_SIZE / WRITE_SIZE
# per dispatch, scaled by a copy of known size); valid only for the kernel
# sources it was taken on, identified by their hash.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "moe_gemm_ep8_decode_traffic.md")
KERNEL_SOURCES = ["w4a16_int4_mixture_moe_amd/csrc/gemm.hip", "w4a16_int4_mixture_moe_amd/csrc/tile_common.hpp",
                  "w4a16_int4_mixture_moe_amd/csrc/device_common.hpp",
                  "w4a16_int4_mixture_moe_amd/csrc/launch.hpp", "w4a16_int4_mixture_moe_amd/build.py"]
ROUTE_INDEXED, ROUTE_CONTIGUOUS, ROUTE_MASKED = 0, 1, 2
EPI_STORE, EPI_WEIGHTED = 0, 1


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(n_touched: int, N: int, K: int) -> int:
    """Packed INT4 weights (K/2 bytes per row) + bf16 group-32 scales."""
    return n_touched * (N * K // 2 + N * (K // 32) * 2)


def mx_weight_bytes(n_touched: int, N: int, K: int) -> int:
    """MXFP4 weights (K/2 bytes per row) + one E8M0 byte per 32 K."""
    return n_touched * (N * K // 2 + N * (K // 32))


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


def cfg_tag(cfg) -> str:
    return f"bm{cfg.block_m} nr{cfg.nr} waves{cfg.waves} split_k{cfg.split_k} stages{cfg.stages}"


def kernel_name(cfg, route: int, epi: int, K: int, mx: bool = False) -> str:
    """The GEMM kernel's name as the rocprofv3 kernel trace shows it.  nr 1 is
    the tile whose waves split K; the library runs the unsplit 128-row,
    4-tiles-per-wave, 4-wave and 256-row, 2-tiles-per-wave, 8-wave
    configurations on its prefill tiles when K is a multiple of 128, the
    first in its N-tile-loop form for K <= 256 on the grids measured here."""
    if mx:
        if cfg.nr == 1:
            return f"mx_kwave_kernel<{cfg.waves}, {epi}>"
        return f"mx_gemm_kernel<{cfg.block_m // 16}, {cfg.nr}, {cfg.waves}, {cfg.stages}, {epi}>"
    if cfg.nr == 1:
        return f"moe_gemm_kwave_kernel<{cfg.waves}, {epi}>"
    tile = (cfg.block_m, cfg.nr, cfg.waves)
    if tile in ((128, 4, 4), (256, 2, 8)) and cfg.stages == 2 and cfg.split_k <= 1 and K % 128 == 0:
        loop = "true" if K <= 256 and tile == (128, 4, 4) else "false"
        return f"moe_gemm_prefill_kernel<{cfg.block_m // 16}, {cfg.nr}, {cfg.waves}, {route}, {epi}, {loop}>"
    return f"moe_gemm_kernel<{cfg.block_m // 16}, {cfg.nr}, {cfg.waves}, {cfg.stages}, {route}, {epi}>"


def gemm_record(us: float, wbytes: int, flops: float, rows_per_expert: float, kernel: str, cfg,
                total_bytes: int | None = None, peak_tflops: float = BF16_PEAK_TFLOPS, stats=None) -> dict:
    """One GEMM call: its bound from the regime (HBM below the ridge of rows per
    expert at which flops per weight byte reach peak_tflops over 8 TB/s, MFMA
    above), the achieved rate on algorithmic units (weight+scale bytes, or
    flops on valid rows) and the fraction of that roofline."""
    gbs = wbytes / (us * 1e-6) / 1e9
    tfl = flops / (us * 1e-6) / 1e12
    ridge = peak_tflops * 1e12 / (HBM_PEAK_GBS * 1e9) * wbytes / max(flops / max(rows_per_expert, 1e-9), 1e-9)
    hbm = rows_per_expert < ridge
    rec = {"us": round(us, 2), "kernel": kernel, "config": cfg_tag(cfg),
           "bound": "hbm" if hbm else "mfma",
           "achieved": round(gbs if hbm else tfl, 1), "unit": "GB/s" if hbm else "TFLOP/s",
           "peak": HBM_PEAK_GBS if hbm else peak_tflops,
           "frac": round(gbs / HBM_PEAK_GBS if hbm else tfl / peak_tflops, 4),
           "weight_GBs": round(gbs, 1), "TFLOPs": round(tfl, 2),
           "weight_bytes": int(wbytes), "flops": float(flops),
           "rows_per_expert": round(rows_per_expert, 1), "ridge_rows_per_expert": round(ridge, 1)}
    if total_bytes is not None:
        rec["total_bytes"] = int(total_bytes)
        rec["total_GBs"] = round(total_bytes / (us * 1e-6) / 1e9, 1)
    if stats is not None:
        rec["median_us"], rec["min_us"], rec["p90_us"] = (round(v, 2) for v in stats[1:])
    return rec


# ------------------------------------------------------------------ timing

class Timer:
    """HIP-event timing on the stream the library launches on (torch's current
    stream, which the binding passes to every call)."""

    def __init__(self, torch, dev):
        self.torch, self.dev = torch, dev

    def stream(self):
        return self.torch.cuda.current_stream(self.dev)

    def graph_of(self, fn, n):
        """n back-to-back calls of fn in one HIP graph (inside the capture
        context torch's current stream is the capture stream, so the library's
        launches land in the graph)."""
        g = self.torch.cuda.CUDAGraph()
        with self.torch.cuda.graph(g):
            for _ in range(n):
                fn()
        return g

    def ramp(self, g, min_ms: float) -> float:
        """Replay g until min_ms of wall time has passed (clocks to their
        steady level); returns the time spent."""
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < min_ms:
            for _ in range(8):
                g.replay()
            torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3

    def per_call(self, fn, inner: int, reps: int, ramp_ms: float = 60.0):
        """Per-call duration: a graph of `inner` calls, replayed for ramp_ms
        first (the GPU's clocks drop within milliseconds of light work, such
        as a run of small calls, and take as long to come back: timed at once,
        back-to-back decode gate/up calls read 194 us instead of 159), then
        replayed `reps` times, each replay between two events.
        (mean, median, min, p90) in us."""
        torch = self.torch
        g = self.graph_of(fn, inner)
        self.ramp(g, ramp_ms)
        s_ = self.stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        g.replay()
        torch.cuda.synchronize()
        for a_, b_ in ev:
            a_.record(s_)
            g.replay()
            b_.record(s_)
        torch.cuda.synchronize()
        t = np.array([a_.elapsed_time(b_) * 1e3 / inner for a_, b_ in ev])
        del g
        return float(t.mean()), float(np.median(t)), float(t.min()), float(np.percentile(t, 90))

    def cold(self, fn, reps: int, flush_buf, flush_sink):
        """Per-call duration with every cache cold: a read of 1 GiB (far beyond
        the 256 MB last-level cache) before each call leaves only clean lines
        (a writing flush would make the call compete with their write-back).
        (median, min, p90) in us."""
        torch = self.torch
        s_ = self.stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a_, b_ in ev:
            torch.amax(flush_buf, dim=0, out=flush_sink)
            a_.record(s_)
            fn()
            b_.record(s_)
        torch.cuda.synchronize()
        t = np.array([a_.elapsed_time(b_) * 1e3 for a_, b_ in ev])
        return float(np.median(t)), float(t.min()), float(np.percentile(t, 90))


# ------------------------------------------------------------------ indexed workloads

class IndexedStep:
    """Inputs, packed weights, routing buffers, configs and workspaces of one
    indexed workload, with align / gate_up / down callables."""

    def __init__(self, torch, M, W, sh, dev, args, weights=None, T=None):
        import ctypes
        self.torch, self.M, self.sh, self.dev = torch, M, sh, dev
        self.mx, self.fused = bool(args.mx), bool(args.fused)
        T = sh.T if T is None else T
        self.T, k = T, sh.topk
        t_gen = time.perf_counter()
        self.ids, self.wts = W.routing_for(sh, T)
        self.x = W.activations(sh.seed, "x", T, sh.K1)
        self.a = W.activations(sh.seed, "a", T * k, sh.K2)
        if weights is not None:
            self.c1, self.s1, self.c2, self.s2 = weights
        elif self.mx:
            self.c1 = W.mx_weight_codes(sh.seed, "w1_mx_codes", sh.E_loc, sh.N1, sh.K1)
            self.s1 = W.mx_weight_scales(sh.seed, "w1_mx_scales", sh.E_loc, sh.N1, sh.K1)
            self.c2 = W.mx_weight_codes(sh.seed, "w2_mx_codes", sh.E_loc, sh.N2, sh.K2)
            self.s2 = W.mx_weight_scales(sh.seed, "w2_mx_scales", sh.E_loc, sh.N2, sh.K2)
        else:
            self.c1 = W.weight_codes(sh.seed, "w1_codes", sh.E_loc, sh.N1, sh.K1)
            self.s1 = W.weight_scales(sh.seed, "w1_scales", sh.E_loc, sh.N1, sh.K1)
            self.c2 = W.weight_codes(sh.seed, "w2_codes", sh.E_loc, sh.N2, sh.K2)
            self.s2 = W.weight_scales(sh.seed, "w2_scales", sh.E_loc, sh.N2, sh.K2)
        log(f"{sh.name} T={T}: inputs generated in {time.perf_counter() - t_gen:.1f}s")

        def bf(b):
            return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)

        if self.mx:
            self.p1 = M.pack_mxfp4(torch.from_numpy(self.c1).to(dev), torch.from_numpy(self.s1).to(dev),
                                   gate_up=self.fused)
            self.p2 = M.pack_mxfp4(torch.from_numpy(self.c2).to(dev), torch.from_numpy(self.s2).to(dev))
        else:
            self.p1 = M.pack_w4(torch.from_numpy(self.c1).to(dev), bf(self.s1), gate_up=self.fused)
            self.p2 = M.pack_w4(torch.from_numpy(self.c2).to(dev), bf(self.s2))
        self.d_ids = torch.from_numpy(self.ids).to(dev)
        self.d_w = torch.from_numpy(self.wts).to(dev)
        self.d_x, self.d_a = bf(self.x), bf(self.a)
        # the selector decides block_m (which fixes the routing alignment)
        # and, per projection, the rest of the tile
        sel = M.mxfp4_select if self.mx else M.select
        c = sel(T, k, sh.E_glob, sh.E_loc, sh.N1, sh.K1)
        bm = args.block_m or c.block_m
        cap = M.align_capacity(T, k, sh.E_loc, bm)
        self.cap = cap
        self.sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
        self.expert_ids = torch.empty(cap // bm, dtype=torch.int32, device=dev)
        self.ntp = torch.empty(1, dtype=torch.int32, device=dev)
        self.routing = M.Routing(self.sorted_ids, self.expert_ids, self.ntp, bm, self.d_ids, sh.E_glob, sh.first,
                                 sh.E_loc)

        def override(cfg):
            if args.nr:
                cfg.nr = args.nr
            if args.waves:
                cfg.waves = args.waves
            if args.split_k >= 0:
                cfg.split_k = args.split_k
            if args.stages:
                cfg.stages = args.stages
            return cfg

        if self.mx:
            # per projection, as the selector gives it
            c2 = M.mxfp4_select(T, k, sh.E_glob, sh.E_loc, sh.N2, sh.K2)
            nr_of = lambda cc: 4 if cc.nr == 1 and bm != 16 else cc.nr
            self.cfg1 = M.mxfp4_config(bm, args.nr or nr_of(c), args.stages or None)
            self.cfg2 = M.mxfp4_config(bm, args.nr or (4 if c2.nr == 1 and bm != 16 else c2.nr), args.stages or None)
        else:
            self.cfg1 = override(M.indexed_config(self.routing, self.p1))
            self.cfg2 = override(M.indexed_config(self.routing, self.p2))
            self.cfg2.combine_cols = args.combine_cols
            if self.fused:
                self.cfg1.split_k = 1   # what the fused call chooses for itself: whole tiles
        self.h = torch.empty(T * k, sh.N1, dtype=torch.bfloat16, device=dev)
        self.y = torch.empty(T, sh.N2, dtype=torch.bfloat16, device=dev)
        z = lambda n: torch.zeros(max(16, n), dtype=torch.uint8, device=dev)
        if self.mx:
            self.ws1 = z(0)
            self.ws2 = z(M.mxfp4_workspace_bytes(self.p2, T, k, True))
            self.qx = M.MXRows(torch.empty(T, sh.K1 // 2, dtype=torch.uint8, device=dev),
                               torch.empty(T, sh.K1 // 32, dtype=torch.uint8, device=dev))
            self.qa = M.MXRows(torch.empty(T * k, sh.K2 // 2, dtype=torch.uint8, device=dev),
                               torch.empty(T * k, sh.K2 // 32, dtype=torch.uint8, device=dev))
        else:
            self.ws1 = z(M.workspace_bytes(self.p1, self.routing, False, self.cfg1))
            self.ws2 = z(M.workspace_bytes(self.p2, self.routing, True, self.cfg2))
        self.inter = (torch.zeros(cap, sh.N1 // 2, dtype=torch.bfloat16, device=dev)
                      if self.fused and not self.mx else None)
        self.inter_mx = (M.MXRows(torch.zeros(cap, sh.N1 // 4, dtype=torch.uint8, device=dev),
                                  torch.zeros(cap, sh.N1 // 64, dtype=torch.uint8, device=dev))
                         if self.fused and self.mx else None)
        if self.fused and (sh.K2 != sh.N1 // 2 or (self.cfg1.nr % 2 and self.cfg1.nr != 1)
                           or (self.mx and self.cfg1.nr not in (1, 4))):
            raise SystemExit("--fused needs K2 = N1 / 2 and an even nr or 1 (4 or 1 with --mx)")
        self.L = M.load()
        self._ctypes = ctypes

    def align(self):
        # the current stream is looked up per call: under graph capture it is the capture stream
        M, sh, torch = self.M, self.sh, self.torch
        s_ptr = self._ctypes.c_void_p(torch.cuda.current_stream(self.dev).cuda_stream)
        M._lib.check(self.L.w4a16_moe_align(self.d_ids.data_ptr(), self.T, sh.topk, sh.E_glob, sh.first, sh.E_loc,
                                            self.routing.block_m, self.sorted_ids.data_ptr(),
                                            self.expert_ids.data_ptr(), self.ntp.data_ptr(), self.cap, 0, s_ptr))

    def gate_up(self):
        M = self.M
        if self.mx and self.fused:
            M.moe_mxfp4_gate_up_silu(self.qx, self.p1, self.routing, cfg=self.cfg1, out=self.inter_mx)
        elif self.mx:
            M.moe_mxfp4_gemm(self.qx, self.p1, self.routing, cfg=self.cfg1, out=self.h)
        elif self.fused:
            M.moe_gate_up_silu(self.d_x, self.p1, self.routing, cfg=self.cfg1, out=self.inter)
        else:
            M.moe_w4a16_gemm(self.d_x, self.p1, self.routing, cfg=self.cfg1, out=self.h, workspace=self.ws1)

    def down(self):
        M = self.M
        if self.mx and self.fused:
            M.moe_mxfp4_gemm(self.inter_mx, self.p2, self.routing, topk_weights=self.d_w, a_layout="sorted",
                             cfg=self.cfg2, out=self.y, workspace=self.ws2)
        elif self.mx:
            M.moe_mxfp4_gemm(self.qa, self.p2, self.routing, topk_weights=self.d_w, cfg=self.cfg2, out=self.y,
                             workspace=self.ws2)
        elif self.fused:
            M.moe_w4a16_gemm(self.inter, self.p2, self.routing, topk_weights=self.d_w, a_layout="sorted",
                             cfg=self.cfg2, out=self.y, workspace=self.ws2)
        else:
            M.moe_w4a16_gemm(self.d_a, self.p2, self.routing, topk_weights=self.d_w, cfg=self.cfg2, out=self.y,
                             workspace=self.ws2)

    def quant(self):
        # A4W4: the activation rows to MXFP4 (unfused: also the local-slot rows
        # of the step's synthetic per-slot down input; fused: the gate/up
        # epilogue quantises the down input itself)
        self.M.mxfp4_quant(self.d_x, out=self.qx)
        if not self.fused:
            self.M.mxfp4_quant_local_slots(self.d_a, self.routing, out=self.qa)

    def step(self):
        self.align()
        if self.mx:
            self.M.mxfp4_quant(self.d_x, out=self.qx)
        self.gate_up()
        if self.mx and not self.fused:
            self.M.mxfp4_quant_local_slots(self.d_a, self.routing, out=self.qa)
        self.down()

    def stats(self):
        """Routed rows, touched experts and the algorithmic units of each GEMM."""
        sh = self.sh
        flat = self.ids.reshape(-1)
        local = (flat >= sh.first) & (flat < sh.first + sh.E_loc)
        n_local = int(local.sum())
        touched = int(len(np.unique(flat[local])))
        wbytes = mx_weight_bytes if self.mx else weight_bytes
        s = {"routed_rows": n_local, "experts_touched": touched,
             "tokens_with_local_slot": int(local.reshape(self.T, sh.topk).any(1).sum()),
             "num_tokens_padded": int(self.ntp.item()),
             "wb1": wbytes(touched, sh.N1, sh.K1), "wb2": wbytes(touched, sh.N2, sh.K2),
             "flops1": 2.0 * n_local * sh.N1 * sh.K1, "flops2": 2.0 * n_local * sh.N2 * sh.K2,
             "rows_per_expert": n_local / max(touched, 1)}
        ntp = s["num_tokens_padded"]
        # total bytes per gate/up launch: weights+scales, one activation row read
        # and one output row written per routed slot, the routing indices
        if self.fused and self.mx:
            out1 = n_local * (sh.N1 // 4 + sh.N1 // 64)
        else:
            out1 = n_local * (sh.N1 // 2 if self.fused else sh.N1) * 2
        row1 = sh.K1 // 2 + sh.K1 // 32 if self.mx else sh.K1 * 2
        s["total1"] = s["wb1"] + n_local * row1 + out1 + ntp * 4 + (ntp // self.routing.block_m) * 4
        # down + combine: weights+scales, slot rows read, fp32 per-slot partials
        # written and read back, the combined [T, N2] bf16 output
        row2 = sh.K2 // 2 + sh.K2 // 32 if self.mx else sh.K2 * 2
        s["total2"] = (s["wb2"] + n_local * row2 + 2 * n_local * sh.N2 * 4 + self.T * sh.N2 * 2
                       + ntp * 4 + self.T * sh.topk * 8)
        return s

    def records(self, st_gu, st_dn, st_align=None):
        s = self.stats()
        peak = FP4_PEAK_TFLOPS if self.mx else BF16_PEAK_TFLOPS
        rec = {"gate_up": gemm_record(st_gu[0], s["wb1"], s["flops1"], s["rows_per_expert"],
                                      kernel_name(self.cfg1, ROUTE_INDEXED, 3 if self.mx and self.fused else
                                                  (2 if self.fused else EPI_STORE), self.sh.K1, self.mx),
                                      self.cfg1, s["total1"], peak, st_gu),
               "down_combine": gemm_record(st_dn[0], s["wb2"], s["flops2"], s["rows_per_expert"],
                                           kernel_name(self.cfg2, ROUTE_INDEXED, EPI_WEIGHTED, self.sh.K2, self.mx),
                                           self.cfg2, s["total2"], peak, st_dn)}
        if st_align is not None:
            rec["align_us"] = round(st_align[0], 2)
        rec.update({k: s[k] for k in ("routed_rows", "experts_touched", "num_tokens_padded")})
        rec["block_m"] = self.routing.block_m
        return rec, s


def measure_indexed(timer, step: IndexedStep, ramp_ms: float, reps: int, inner: int = 4) -> dict:
    g = timer.graph_of(step.step, 1)
    ramp = timer.ramp(g, ramp_ms)
    del g
    st_al = timer.per_call(step.align, inner, reps)
    st_gu = timer.per_call(step.gate_up, inner, reps)
    st_dn = timer.per_call(step.down, inner, reps)
    rec, _ = step.records(st_gu, st_dn, st_al)
    rec["step_us"] = round(st_al[0] + st_gu[0] + st_dn[0], 2)
    rec["clock_ramp_ms"] = round(ramp, 1)
    return rec


# ------------------------------------------------------------------ grouped workload

class GroupedStep:
    """The configuration-4 grouped gate/up GEMMs on skewed routing: the
    contiguous layout (each expert's rows padded to 128, m_indices -1 on
    padding) and the masked one ([E, max_m, K] with masked_m counts)."""

    def __init__(self, torch, M, W, sh, dev, args=None):
        self.torch, self.M, self.sh = torch, M, sh
        t_gen = time.perf_counter()
        ids, _ = W.routing_for(sh)
        x = W.activations(sh.seed, "x", sh.T, sh.K1)
        self.c1 = W.weight_codes(sh.seed, "w1_codes", sh.E_loc, sh.N1, sh.K1)
        self.s1 = W.weight_scales(sh.seed, "w1_scales", sh.E_loc, sh.N1, sh.K1)
        A, self.mi, _ = W.contiguous_layout(ids, x, sh.first, sh.E_loc, pad=128, pad_fill=0)
        A3, self.mm, _, self.dropped = W.masked_layout(ids, x, sh.first, sh.E_loc, sh.max_m, pad_fill=0)
        log(f"{sh.name}: inputs generated in {time.perf_counter() - t_gen:.1f}s")

        def bf(b):
            return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)

        self.p1 = M.pack_w4(torch.from_numpy(self.c1).to(dev), bf(self.s1))
        self.rows_c = int(A.shape[0])
        self.d_A, self.d_A3 = bf(A), bf(A3)
        del A, A3
        self.d_mi = torch.from_numpy(self.mi.astype(np.int32)).to(dev)
        self.d_mm = torch.from_numpy(self.mm.astype(np.int32)).to(dev)
        self.expected_m = max(1, int(round(float(self.mm.mean()))))
        self.cfg_c = M.select(self.rows_c, 1, 1, sh.E_loc, sh.N1, sh.K1, kind="contiguous")
        self.cfg_m = M.select(sh.max_m, 1, 1, sh.E_loc, sh.N1, sh.K1, kind="masked", expected_m=self.expected_m)
        # --block-m / --nr / --waves overrides: the calls then take the
        # changed configs (block_m on the contiguous layout only where it
        # divides the layout's 128-row segments)
        self.explicit = bool(args is not None and (args.nr or args.waves or args.block_m))
        if self.explicit:
            for c in (self.cfg_c, self.cfg_m):
                if args.block_m and (c is self.cfg_m or 128 % args.block_m == 0):
                    c.block_m = args.block_m
                c.nr = args.nr or c.nr
                c.waves = args.waves or c.waves
        z = lambda n: torch.zeros(max(16, n), dtype=torch.uint8, device=dev)
        self.ws_c = z(M.grouped_workspace_bytes(self.p1, "contiguous", self.rows_c,
                                                cfg=self.cfg_c if self.explicit else None))
        self.ws_m = z(M.grouped_workspace_bytes(self.p1, "masked", sh.max_m, self.expected_m,
                                                cfg=self.cfg_m if self.explicit else None))
        self.out_c = torch.empty(self.rows_c, sh.N1, dtype=torch.bfloat16, device=dev)
        self.out_m = torch.empty(sh.E_loc * sh.max_m, sh.N1, dtype=torch.bfloat16, device=dev)

    def contiguous(self):
        self.M.grouped_contiguous(self.d_A, self.p1, self.d_mi, out=self.out_c, workspace=self.ws_c,
                                  cfg=self.cfg_c if self.explicit else None)

    def masked(self):
        self.M.grouped_masked(self.d_A3, self.p1, self.d_mm, self.expected_m, out=self.out_m, workspace=self.ws_m,
                              cfg=self.cfg_m if self.explicit else None)

    def step(self):
        self.contiguous()
        self.masked()

    def records(self, st_c, st_m):
        sh = self.sh
        fl_row = 2.0 * sh.N1 * sh.K1
        valid_c = int((self.mi >= 0).sum())
        valid_m = int(self.mm.sum())
        touched = int(sum(1 for c in self.mm if c > 0))
        wb = weight_bytes(touched, sh.N1, sh.K1)
        rpe_c = valid_c / max(touched, 1)
        rec_c = gemm_record(st_c[0], wb, valid_c * fl_row, rpe_c, kernel_name(self.cfg_c, ROUTE_CONTIGUOUS, EPI_STORE, sh.K1),
                            self.cfg_c, stats=st_c)
        rec_c["TFLOPs_padded_rows"] = round(self.rows_c * fl_row / (st_c[0] * 1e-6) / 1e12, 2)
        rec_c.update(rows=self.rows_c, valid_rows=valid_c)
        rec_m = gemm_record(st_m[0], wb, valid_m * fl_row, valid_m / max(touched, 1),
                            kernel_name(self.cfg_m, ROUTE_MASKED, EPI_STORE, sh.K1), self.cfg_m, stats=st_m)
        rec_m["TFLOPs_all_rows"] = round(sh.E_loc * sh.max_m * fl_row / (st_m[0] * 1e-6) / 1e12, 2)
        rec_m.update(max_m=int(sh.max_m), valid_rows=valid_m, dropped_rows=int(self.dropped),
                     expected_m=self.expected_m)
        return {"contiguous": rec_c, "masked": rec_m, "zero_row_experts": int((self.mm == 0).sum())}


def measure_grouped(timer, gs: GroupedStep, ramp_ms: float, reps: int, inner: int = 4) -> dict:
    g = timer.graph_of(gs.step, 1)
    ramp = timer.ramp(g, ramp_ms)
    del g
    st_c = timer.per_call(gs.contiguous, inner, reps)
    st_m = timer.per_call(gs.masked, inner, reps)
    rec = gs.records(st_c, st_m)
    rec["clock_ramp_ms"] = round(ramp, 1)
    return rec


# ------------------------------------------------------------------ CPU baseline

def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([d.get("num_threads", 1) for d in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return int(os.cpu_count() or 1)


def _median_seconds(fn, runs: int = 3) -> float:
    t = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        t.append(time.perf_counter() - t0)
    return float(np.median(t))


def cpu_baseline(st: IndexedStep, n_experts: int, n_single: int, tiny: IndexedStep | None) -> dict:
    """The oracle's fp32 path (dequantise, sgemm, combine), untuned, timed on
    the host's cores as the median of 3 runs: on the first n_experts local
    experts of the workload (all rows routed to them) with every BLAS thread,
    on the first n_single with one thread, and on the whole tiny step both
    ways.  GB/s of weight+scale bytes processed."""
    from oracle import moe_oracle as O
    from threadpoolctl import threadpool_limits
    sh = st.sh

    def run(S, step=st):
        s_ = step.sh
        O.indexed_gate_up_fp32(step.x, step.c1[:S], step.s1[:S], step.ids, s_.first, S)
        O.indexed_down_combine_fp32(step.a, step.c2[:S], step.s2[:S], step.ids, step.wts, s_.first, S)

    def gbs(S, sec, step=st):
        s_ = step.sh
        return (weight_bytes(S, s_.N1, s_.K1) + weight_bytes(S, s_.N2, s_.K2)) / sec / 1e9

    threads = _blas_threads()
    t_multi = _median_seconds(lambda: run(n_experts))
    with threadpool_limits(limits=1):
        t_single = _median_seconds(lambda: run(n_single))
    flat = st.ids.reshape(-1)
    rows = int(((flat >= sh.first) & (flat < sh.first + n_experts)).sum())
    out = {"value": round(gbs(n_experts, t_multi), 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "host_cpu_count": os.cpu_count(), "seconds_median_of_3": round(t_multi, 3),
           "sample": f"{sh.name}: gate/up + down+combine for local experts 0..{n_experts - 1} of {sh.E_loc} "
                     f"({rows} routed rows), same inputs as the GPU step, median of 3; GB/s of weight+scale bytes",
           "single_thread": {"value": round(gbs(n_single, t_single), 4), "unit": "GB/s", "cores": 1,
                             "seconds_median_of_3": round(t_single, 3),
                             "sample": f"local experts 0..{n_single - 1}"}}
    if tiny is not None:
        E = tiny.sh.E_loc
        t_tm = _median_seconds(lambda: run(E, tiny))
        with threadpool_limits(limits=1):
            t_t1 = _median_seconds(lambda: run(E, tiny))
        out["tiny"] = {"us_per_step_all_threads": round(t_tm * 1e6, 1), "us_per_step_one_thread": round(t_t1 * 1e6, 1),
                       "GBs_all_threads": round(gbs(E, t_tm, tiny), 4), "GBs_one_thread": round(gbs(E, t_t1, tiny), 4),
                       "sample": "whole tiny step (gate/up + down+combine, all 8 experts), median of 3"}
    return out


def cpu_baseline_mx(st: IndexedStep, n_experts: int) -> dict:
    """The MXFP4 oracle as it stands (quantise the step's activation rows,
    dequantise, float64 matmul, combine) on the first n_experts local
    experts and all rows routed to them, median of 3."""
    from oracle import mx_oracle as X
    sh = st.sh
    S = n_experts

    def run():
        xq = X.mx_quantize(st.x)
        aq = X.mx_quantize(st.a)
        X.mx_indexed_gate_up(*xq, X.unpack_nibbles(st.c1[:S]), st.s1[:S], st.ids, sh.first, S)
        X.mx_indexed_down_combine(*aq, X.unpack_nibbles(st.c2[:S]), st.s2[:S], st.ids, st.wts, sh.first, S)

    t = _median_seconds(run)
    b = mx_weight_bytes(S, sh.N1, sh.K1) + mx_weight_bytes(S, sh.N2, sh.K2)
    return {"value": round(b / t / 1e9, 4), "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "seconds_median_of_3": round(t, 3),
            "sample": f"A4W4: quantise all activation rows, gate/up + down+combine for local experts 0..{S - 1} of "
                      f"{sh.E_loc}, same inputs as the GPU step, median of 3; GB/s of MXFP4 weight+scale bytes"}


# ------------------------------------------------------------------ entry points

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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--ramp-ms", type=float, default=200.0,
                    help="wall time each workload's step is replayed before timing (steady GPU clocks)")
    ap.add_argument("--workload", default="", help="measure only this workload (default: all five configs)")
    ap.add_argument("--block-m", type=int, default=0, help="override the selector's block_m")
    ap.add_argument("--nr", type=int, default=0, help="override the selector's weight tiles per wave")
    ap.add_argument("--waves", type=int, default=0, help="override the selector's waves per workgroup")
    ap.add_argument("--split-k", type=int, default=-1, help="override: 1 one workgroup per tile, 2/4/8/16 K slices, "
                                                             "0 stream-K")
    ap.add_argument("--stages", type=int, default=0, help="override: K chunks of weights in flight per wave")
    ap.add_argument("--combine-cols", type=int, default=0,
                    help="override: output columns per down-projection + combine pass (a multiple of 16)")
    ap.add_argument("--cpu-experts", type=int, default=4, help="experts in the CPU-baseline sample (0: skip)")
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

    dev = torch.device("cuda", 0)
    timer = Timer(torch, dev)
    head_name = args.workload or "ep8_decode"
    sh = W.WORKLOADS[head_name]
    sub_reps = max(8, min(args.steps, 40))
    if sh.name == "grouped_skewed":
        if args.mx or args.fused:
            print("the grouped layouts run the W4A16 gate/up GEMM only (no --mx / --fused)", file=sys.stderr)
            return 2
        gs = GroupedStep(torch, M, W, sh, dev, args)
        rec = measure_grouped(timer, gs, args.ramp_ms, max(8, args.steps // 2))
        for _ in range(args.warmup):
            gs.step()
        g = timer.graph_of(gs.step, 1)
        s_ = timer.stream()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(s_)
        for _ in range(args.steps):
            g.replay()
        t1.record(s_)
        torch.cuda.synchronize()
        ms_step = t0.elapsed_time(t1) / args.steps
        fl = rec["contiguous"]["flops"] + rec["masked"]["flops"]
        out = {"metric": METRIC, "value": round(fl / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
               "timing": "HIP graph replay of the step (one contiguous and one masked call)",
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
               "data": "synthetic", "config": {"workload": sh.name, "T": sh.T, "topk": sh.topk, "E_glob": sh.E_glob,
                                               "E_loc": sh.E_loc, "K1": sh.K1, "N1": sh.N1},
               "grouped": rec,
               "roofline": {k: rec["contiguous"][k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac")}}
        out["roofline"]["traffic"] = None
        print(json.dumps(out), flush=True)
        return 0

    # ---- the headline workload: the whole step, K timed steps
    st = IndexedStep(torch, M, W, sh, dev, args)
    g_step = None if args.eager else timer.graph_of(st.step, 1)
    ramp = timer.ramp(g_step if g_step is not None else timer.graph_of(st.step, 1), args.ramp_ms)
    for _ in range(args.warmup):
        if g_step is not None:
            g_step.replay()
        else:
            st.step()
    torch.cuda.synchronize()
    s_ = timer.stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(s_)
    for _ in range(args.steps):
        if g_step is not None:
            g_step.replay()
        else:
            st.step()
    t1.record(s_)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    # per-call averages: each call replayed back to back inside one graph
    inner = 8
    st_al = timer.per_call(st.align, inner, max(4, args.steps // 2))
    st_gu = timer.per_call(st.gate_up, inner, max(4, args.steps // 2))
    st_dn = timer.per_call(st.down, inner, max(4, args.steps // 2))
    st_q = timer.per_call(st.quant, inner, max(4, args.steps // 2)) if args.mx else None
    flush_buf = torch.zeros(1 << 28, dtype=torch.int32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.int32, device=dev)
    st_cold = {"align": timer.cold(st.align, 20, flush_buf, flush_sink),
               "gate_up": timer.cold(st.gate_up, 20, flush_buf, flush_sink),
               "down_combine": timer.cold(st.down, 20, flush_buf, flush_sink)}
    del flush_buf, flush_sink

    # host cost of choosing a config (first call runs the sampled search,
    # later calls hit the memoised result) and of one launch (binding +
    # argument checks + kernel enqueue), no device time
    def host_us(fn, reps):
        t0_ = time.perf_counter()
        for _ in range(reps):
            fn()
        return (time.perf_counter() - t0_) * 1e6 / reps

    k = sh.topk
    probe_T = st.T + 1                                        # a shape the run has not selected for yet
    t0_ = time.perf_counter()
    M.select(probe_T, k, sh.E_glob, sh.E_loc, sh.N1, sh.K1)
    host_select_first = (time.perf_counter() - t0_) * 1e6
    host_select_memo = host_us(lambda: M.select(probe_T, k, sh.E_glob, sh.E_loc, sh.N1, sh.K1), 200)
    host_launch = host_us(st.gate_up, 50)
    torch.cuda.synchronize()

    rec, s = st.records(st_gu, st_dn, st_al)
    value = (s["wb1"] + s["wb2"]) / (ms_step * 1e-3) / 1e9
    gu = rec["gate_up"]
    roofline = {"kernel": gu["kernel"], "bound": gu["bound"], "achieved": gu["achieved"], "peak": gu["peak"],
                "unit": gu["unit"], "frac": gu["frac"],
                "traffic": None if args.mx else measured_traffic(sh.name, cfg_tag(st.cfg1)),
                "algorithmic": "weight+scale bytes of the touched experts" if gu["bound"] == "hbm"
                               else "flops on routed (valid) rows",
                "algorithmic_bytes": gu["weight_bytes"], "total_bytes": gu["total_bytes"],
                "achieved_on_total_bytes_GBs": gu["total_GBs"], "rows_per_expert": gu["rows_per_expert"],
                "ridge_rows_per_expert": gu["ridge_rows_per_expert"]}
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp_ms": round(ramp, 1),
        "ms_per_step": round(ms_step, 4),
        "timing": "HIP graph replay of the step" if g_step is not None else "eager launches",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if args.mx else "bf16",
        "data": "synthetic",
        "config": {"workload": sh.name, "variant": "a4w4-mxfp4" if args.mx else "w4a16",
                   "fused_silu": bool(args.fused), "T": st.T, "topk": k, "E_glob": sh.E_glob, "E_loc": sh.E_loc,
                   "K1": sh.K1, "N1": sh.N1, "K2": sh.K2, "N2": sh.N2, "block_m": st.routing.block_m,
                   "gate_up_config": cfg_tag(st.cfg1), "down_config": cfg_tag(st.cfg2),
                   "routed_rows": s["routed_rows"], "experts_touched": s["experts_touched"],
                   "num_tokens_padded": s["num_tokens_padded"]},
        "per_call_us": {"align": round(st_al[0], 2), "gate_up": round(st_gu[0], 2), "down_combine": round(st_dn[0], 2)},
        "per_call_stats_us": {name: {"median": round(v[1], 2), "min": round(v[2], 2), "p90": round(v[3], 2)}
                              for name, v in (("align", st_al), ("gate_up", st_gu), ("down_combine", st_dn))},
        "per_call_cold_us": {name: {"median": round(v[0], 2), "min": round(v[1], 2), "p90": round(v[2], 2)}
                             for name, v in st_cold.items()},
        "host_us": {"select_first_call": round(host_select_first, 1), "select_memoised": round(host_select_memo, 2),
                    "gate_up_launch": round(host_launch, 1)},
        "gemm": rec,
        "roofline": roofline,
    }
    if st_q is not None:
        qname = "mxfp4_quant_x" if args.fused else "mxfp4_quant_x_and_a"
        out["per_call_us"][qname] = round(st_q[0], 2)

    # ---- every synthetic configuration (default run)
    if not args.workload and not args.mx and not args.fused:
        configs = {}
        del g_step
        t_cfg = time.perf_counter()
        tiny = IndexedStep(torch, M, W, W.WORKLOADS["tiny"], dev, args)
        configs["0_tiny"] = measure_indexed(timer, tiny, args.ramp_ms, sub_reps)
        configs["1_ep8_decode"] = {"same_as": "headline", **{k_: out["gemm"][k_] for k_ in ("gate_up", "down_combine")},
                                   "align_us": out["per_call_us"]["align"]}
        cpu_args = (st, tiny)
        pre = IndexedStep(torch, M, W, W.WORKLOADS["ep8_prefill"], dev, args)
        configs["2_ep8_prefill"] = measure_indexed(timer, pre, args.ramp_ms, sub_reps)
        del pre
        torch.cuda.empty_cache()
        sh3 = W.WORKLOADS["tp8_t1"]
        w3 = (W.weight_codes(sh3.seed, "w1_codes", sh3.E_loc, sh3.N1, sh3.K1),
              W.weight_scales(sh3.seed, "w1_scales", sh3.E_loc, sh3.N1, sh3.K1),
              W.weight_codes(sh3.seed, "w2_codes", sh3.E_loc, sh3.N2, sh3.K2),
              W.weight_scales(sh3.seed, "w2_scales", sh3.E_loc, sh3.N2, sh3.K2))
        sweep = {}
        for T in W.TP8_TOKENS:
            tp = IndexedStep(torch, M, W, W.WORKLOADS[f"tp8_t{T}"], dev, args, weights=w3)
            sweep[f"T{T}"] = measure_indexed(timer, tp, args.ramp_ms, sub_reps)
            del tp
            torch.cuda.empty_cache()
        configs["3_tp8"] = sweep
        del w3
        gs = GroupedStep(torch, M, W, W.WORKLOADS["grouped_skewed"], dev, args)
        configs["4_grouped_skewed"] = measure_grouped(timer, gs, args.ramp_ms, sub_reps)
        del gs
        torch.cuda.empty_cache()
        out["configs"] = configs
        out["configs_seconds"] = round(time.perf_counter() - t_cfg, 1)
    else:
        cpu_args = (st, None)

    if args.cpu_experts > 0:
        log("timing the CPU oracle baseline ...")
        if args.mx:
            out["cpu_baseline"] = cpu_baseline_mx(st, args.cpu_experts)
        else:
            out["cpu_baseline"] = cpu_baseline(cpu_args[0], args.cpu_experts, max(1, args.cpu_experts // 2),
                                               cpu_args[1])
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
