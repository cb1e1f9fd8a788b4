"""Benchmark of the packed W4A4 block-scaled linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama_prefill]

A step is one pass of the hot path over one batch: for each of the four
Llama-3.1-8B linears (QKV, O, gate+up, down) the activations are rescaled
and quantized (w4a4_quantize_act) and multiplied with the packed weight
(w4a4_linear, row-scale epilogue included).  Weights are quantized and
packed once, before timing (the paper packs them offline).  Inputs are
seeded synthetic tensors already resident in HBM.  The step's launches are
captured once as a HIP graph and replayed for the step time; the same
launches run eagerly with HIP events around each one for the per-kernel
durations.

Printed: one JSON line with the workload's throughput (TFLOP/s, whole step),
the GEMM kernel's roofline position (algorithmic flops per launch over its
HIP-event-timed average duration, against the MI355X dense MXFP4 peak, and
beside it the rate of the FP4 MFMAs alone on register operands, the ceiling
the chip holds under that load),
decode weight-streaming bandwidth and linear-layer tokens/s with the
activation quantization included (MXFP4 Llama linears at M = 1, 4, 16;
MXINT4 Qwen, NVFP4, MXFP8, MXINT8, INT4 G=64 and INT8 G=128 Llama linears
at M = 1;
32 layer copies cycled so that the 256 MB last-level cache cannot hold the
weights), the other formats' prefill configurations (NVFP4 Llama at
M = 4096, MXINT4 Qwen at M = 512 and 4096, MXFP8, MXINT8, INT4 G=64 and
INT8 G=128 Llama at M = 2048), each against the peak of the MFMA it runs on, the offline
dual-scale solver on fp32 weights of the Llama linears' shapes, the q, k, v
projections with their own column scales (one multi-output quantize and one
grouped GEMM against three separate pairs), and the CPU oracle timed on a
bounded sample of the same workload (activation quantization and linear
apart, with the host's core count and CPU model).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import w4a4_block_scaled_amd as w4  # noqa: E402
from w4a4_block_scaled_amd import inputs  # noqa: E402

PEAK = {  # MI355X published dense peaks
    "mxfp4": (10.1e15, "TFLOP/s", "mfma"),   # FP4 / FP6 MFMA
    "mxint4": (5.0e15, "TFLOP/s", "mfma"),   # runs on the FP8 scaled MFMA
    "nvfp4": (2.5e15, "TFLOP/s", "mfma"),    # runs on the fp16 MFMA
    "int4g64": (2.5e15, "TFLOP/s", "mfma"),  # exact fp16 expansion of code x BF16 scale, fp16 MFMA
    "mxfp8": (2.5e15, "TFLOP/s", "mfma"),    # exact bf16 expansion on the bf16 MFMA
    "mxint8": (5.0e15, "TOP/s", "mfma"),     # FP8 scaled MFMA, four per int8 product
    "int8g128": (5.0e15, "TOP/s", "mfma"),   # int8 MFMA, BF16 block scales on the VALU
}
HBM_PEAK = 8.0e12
DTYPE = {"mxfp4": "fp4", "nvfp4": "fp4xe4m3->fp16", "mxint4": "int4->fp8",
         "int4g64": "int4xbf16->fp16", "mxfp8": "fp8->bf16", "mxint8": "int8->2xfp8",
         "int8g128": "int8"}
CODE_BYTES = {"mxfp8": 1.0, "mxint8": 1.0, "int8g128": 1.0}   # bytes per code (0.5 for the 4-bit formats)
SCALE_BYTES = {"int4g64": 2, "int8g128": 2}   # bytes per block scale (1 for E8M0 / UE4M3)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Layer:
    """Device tensors of one linear: inputs, packed weight, outputs."""

    def __init__(self, case, dev):
        self.case = case
        self.N, self.K, self.M, self.fmt = case.N, case.K, case.M, case.fmt
        if case.w_codes is not None:
            wc = torch.from_numpy(case.w_codes).to(dev)
            ws = torch.from_numpy(case.w_scales).to(dev)
            if case.fmt in ("int4g64", "int8g128"):        # BF16 bit patterns
                ws = torch.from_numpy(case.w_scales.view(np.int16)).to(dev).view(torch.bfloat16)
            tw = torch.tensor([case.t_w], dtype=torch.float32, device=dev)
        else:
            wc, ws, tw = w4.quantize_act(case.w_prescaled.to(dev), None, case.fmt)
        self.blob = w4.pack_weight(wc, ws, tw, torch.from_numpy(case.r).to(dev), case.fmt)
        del wc, ws
        self.x = case.x.to(dev)
        self.c = torch.from_numpy(case.c).to(dev)
        G = w4.block_size(case.fmt)
        self.codes = torch.empty((self.M, w4.code_cols(case.fmt, self.K)), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((self.M, self.K // G), dtype=w4.scale_dtype(case.fmt), device=dev)
        self.t = torch.ones(1, dtype=torch.float32, device=dev)
        self.ws = torch.empty(max(16, w4.lib().w4a4_quantize_workspace_bytes(
            w4.FORMATS[case.fmt], self.M, self.K)), dtype=torch.uint8, device=dev)
        self.y = torch.empty((self.M, self.N), dtype=torch.bfloat16, device=dev)

    def quantize(self):
        w4.quantize_act(self.x, self.c, self.fmt, out=(self.codes, self.scales, self.t),
                        workspace=self.ws)

    def gemm(self, blob=None):
        w4.linear(self.codes, self.scales, self.t, self.blob if blob is None else blob, self.fmt,
                  self.N, self.K, out=self.y)

    @property
    def flops(self):
        return 2.0 * self.M * self.N * self.K

    @property
    def quant_bytes(self):
        """quantize_act algorithmic bytes: X in, c in, codes and scales out."""
        G = w4.block_size(self.fmt) / SCALE_BYTES.get(self.fmt, 1)
        cb = CODE_BYTES.get(self.fmt, 0.5)
        return 2 * self.M * self.K + 4 * self.K + cb * self.M * self.K + self.M * self.K / G

    @property
    def gemm_bytes(self):
        return gemm_bytes(self.fmt, self.M, self.N, self.K)


def gemm_bytes(fmt, M, N, K):
    """GEMM algorithmic bytes: weight codes, scales and r, activation codes and
    scales, BF16 output."""
    G = w4.block_size(fmt) / SCALE_BYTES.get(fmt, 1)
    cb = CODE_BYTES.get(fmt, 0.5)
    return cb * N * K + N * K / G + 4 * N + cb * M * K + M * K / G + 2 * M * N


def time_steps(layers, steps, warmup):
    """ms per step, launched eagerly from the host (quantize_act + linear for
    every linear)."""
    for _ in range(warmup):
        for L in layers:
            L.quantize()
            L.gemm()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        for L in layers:
            L.quantize()
            L.gemm()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_launches(fn, reps=10, bursts=5):
    """Average duration (ms) of one launch of fn: a HIP graph of `reps`
    back-to-back calls is replayed `bursts` times between two HIP events on
    the stream the kernels run on (the graph's own stream ordering leaves no
    host gaps, and an event pair around every launch would add its own)."""
    def many():
        for _ in range(reps):
            fn()
    g = capture(many)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(bursts):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (reps * bursts)


def per_launch(layers, steps):
    """Per-layer average GEMM and quantize_act launch durations (ms)."""
    bursts = max(2, steps // 10)
    gemm_ms = [time_launches(L.gemm, bursts=bursts) for L in layers]
    quant_ms = [time_launches(L.quantize, bursts=bursts) for L in layers]
    return gemm_ms, quant_ms


def capture(fn):
    """A HIP graph of fn()'s launches (run once eagerly on a side stream first)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(layers, steps, warmup):
    """ms per step with the step (quantize_act + linear for every linear)
    captured once as a HIP graph and replayed: no host launch cost, and the
    kernels follow each other as the GPU allows."""
    def step():
        for L in layers:
            L.quantize()
            L.gemm()
    g = capture(step)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_projection_rate(dev, M=2048, K=4096, Ns=(4096, 1024, 1024), reps=50):
    """Per-projection c on a fused input: the Llama q, k, v projections of one
    hidden state (MXFP4), each with its own column scale.  Against three
    separate (quantize_act, linear) pairs: one w4a4_quantize_act_multi
    (X read once) and one w4a4_linear_grouped (the three problems' tiles in
    one launch).  Every variant replayed from a HIP graph of `reps` steps;
    random codes stand in for the weights (the kernels' work does not depend
    on the values)."""
    g = torch.Generator(device="cpu").manual_seed(9)
    x = torch.randn((M, K), generator=g).to(torch.bfloat16).to(dev)
    P = len(Ns)
    cs = [torch.ldexp(torch.ones(K), torch.randint(-2, 3, (K,), generator=g)).to(dev) for _ in range(P)]
    blobs = []
    for N in Ns:
        wc = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, generator=g).to(dev)
        wsc = torch.randint(118, 124, (N, K // 32), dtype=torch.uint8, generator=g).to(dev)
        blobs.append(w4.pack_weight(wc, wsc, None, torch.ones(N, device=dev), "mxfp4"))
    q = [w4.quantize_act(x, c, "mxfp4") for c in cs]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for N in Ns]

    def timed(fn):
        gr = capture(lambda: [fn() for _ in range(reps)])
        gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    problems = [(q[p][0], q[p][1], None, blobs[p], Ns[p]) for p in range(P)]
    quant_multi = timed(lambda: w4.quantize_act_multi(x, cs, "mxfp4"))
    quant_sep = timed(lambda: [w4.quantize_act(x, c, "mxfp4") for c in cs])
    gemm_grouped = timed(lambda: w4.linear_grouped(problems, "mxfp4", K, outs=ys))
    gemm_sep = timed(lambda: [w4.linear(q[p][0], q[p][1], None, blobs[p], "mxfp4", Ns[p], K, out=ys[p])
                              for p in range(P)])

    def step_fused():
        qs = w4.quantize_act_multi(x, cs, "mxfp4")
        w4.linear_grouped([(qs[p][0], qs[p][1], None, blobs[p], Ns[p]) for p in range(P)], "mxfp4", K, outs=ys)

    def step_sep():
        for p in range(P):
            a, s_, _ = w4.quantize_act(x, cs[p], "mxfp4")
            w4.linear(a, s_, None, blobs[p], "mxfp4", Ns[p], K, out=ys[p])

    fused = timed(step_fused)
    sep = timed(step_sep)
    flops = 2.0 * M * K * sum(Ns)
    return {"M": M, "K": K, "N": list(Ns), "quantize_multi_us": round(quant_multi, 2),
            "quantize_separate_us": round(quant_sep, 2), "gemm_grouped_us": round(gemm_grouped, 2),
            "gemm_separate_us": round(gemm_sep, 2),
            "gemm_grouped_TFLOP/s": round(flops / (gemm_grouped * 1e-6) / 1e12, 1),
            "step_fused_us": round(fused, 2), "step_separate_us": round(sep, 2)}


def solver_rate(dev, iters=15):
    """The offline dual-scale solver (w4a4_dualquant_solve, MXFP4) on fp32
    weights of each Llama linear's shape: synthetic N(0, 0.02) weights with
    1/64 of the columns scaled x20 and lognormal column and row scales.  One
    warm-up solve, then one timed solve per linear (T = 15; the solve stops
    at a fixed point of the scales, so fewer passes may run)."""
    g = torch.Generator(device="cpu").manual_seed(7)
    out = {}
    total = 0.0
    for name, N, K in inputs.LLAMA_LINEARS:
        w = torch.randn((N, K), generator=g) * 0.02
        cols = torch.randperm(K, generator=g)[: K // 64]
        w[:, cols] *= 20
        w *= torch.exp(0.5 * torch.randn((1, K), generator=g)) * torch.exp(0.3 * torch.randn((N, 1), generator=g))
        w = w.to(dev)
        ws = torch.empty(w4.lib().w4a4_dualquant_workspace_bytes(0, N, K), dtype=torch.uint8, device=dev)
        w4.dualquant_solve(w, "mxfp4", iters, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        w4.dualquant_solve(w, "mxfp4", iters, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        total += ms
        out[name] = {"N": N, "K": K, "ms": round(ms, 3),
                     "W_bytes_per_pass_over_ms_GB/s": round(4.0 * N * K / (ms * 1e-3) / 1e9, 1)}
        del w, ws
        torch.cuda.empty_cache()
    return {"format": "mxfp4", "iters": iters, "layer_ms": round(total, 3), "per_linear": out}


def prefill_rates(dev, workload, M, steps, warmup):
    """Prefill at M tokens for the linears of `workload` (quantize_act + linear
    per linear): the graph-timed step, and the GEMM rate from per-launch HIP
    events against the peak of the MFMA the format runs on."""
    fmt = inputs.WORKLOADS[workload][1]
    layers = [Layer(c, dev) for c in inputs.workload_cases(workload, M=M)]
    torch.cuda.synchronize()
    gemm_ms, quant_ms = per_launch(layers, steps)
    ms = time_graph(layers, steps, warmup)
    peak, unit, bound = PEAK[fmt]
    ops = sum(L.flops for L in layers)
    achieved = ops / (sum(gemm_ms) * 1e-3)
    out = {"format": fmt, "M": M, "dtype": DTYPE[fmt],
           "step_ms": round(ms, 4), "tokens_per_s": round(M / (ms * 1e-3), 1),
           unit + "_step": round(ops / (ms * 1e-3) / 1e12, 1),
           "roofline": {"bound": bound, "achieved": round(achieved / 1e12, 1), "peak": peak / 1e12,
                        "unit": unit, "frac": round(achieved / peak, 4),
                        "traffic": traffic_record(f"gemm_{workload}_M{M}", fmt),
                        "kernel": gemm_kernel_label(fmt, M)},
           "per_linear": {L.case.name: {"gemm_us": round(t * 1e3, 2),
                                        unit: round(L.flops / (t * 1e-3) / 1e12, 1),
                                        "frac": round(L.flops / (t * 1e-3) / peak, 4),
                                        "quantize_us": round(qt * 1e3, 2)}
                          for L, t, qt in zip(layers, gemm_ms, quant_ms)}}
    del layers
    torch.cuda.empty_cache()
    return out


def decode_bandwidth(dev, steps, workload="llama_decode", Ms=(1, 4, 16), copies=32):
    """Decode at small M (default: MXFP4 Llama shapes at M = 1, 4, 16).

    A "layer" is the workload's four linears; 32 distinct copies of the packed
    weights (3.7 GB for the MXFP4 Llama linears, like the 32 layers of the
    model) are cycled so that no copy is still cached in the 256 MB
    last-level cache.  Two HIP graphs of the 32 layers are replayed: the
    GEMMs alone (the weight-streaming rate: algorithmic GEMM bytes over their
    time, against 8 TB/s) and quantize_act + GEMM per linear (tokens/s =
    M / time per layer of the four linears with their quantizations; linear
    layers only, not a whole transformer block).
    """
    out = {}
    fmt = inputs.WORKLOADS[workload][1]
    base = [Layer(c, dev) for c in inputs.workload_cases(workload, M=max(Ms))]
    blobs = [[L.blob.clone() for L in base] for _ in range(copies)]
    for M in Ms:
        cases = inputs.workload_cases(workload, M=M, build_weights=False)
        act = [(c.x.to(dev), torch.from_numpy(c.c).to(dev)) for c in cases]
        # quantized activations for this M (one buffer set per linear)
        q = [w4.quantize_act(x, c, fmt) for x, c in act]
        qws = [torch.empty(max(16, w4.lib().w4a4_quantize_workspace_bytes(w4.FORMATS[fmt], M, L.K)),
                           dtype=torch.uint8, device=dev) for L in base]
        ys = [torch.empty((M, L.N), dtype=torch.bfloat16, device=dev) for L in base]
        nbytes = sum(gemm_bytes(fmt, M, L.N, L.K) for L in base)

        def run_model(with_quant):
            for k in range(copies):
                for j, L in enumerate(base):
                    if with_quant:
                        w4.quantize_act(act[j][0], act[j][1], fmt, out=q[j], workspace=qws[j])
                    w4.linear(q[j][0], q[j][1], q[j][2], blobs[k][j], fmt, L.N, L.K, out=ys[j])

        res = {}
        for with_quant in (False, True):
            g = capture(lambda: run_model(with_quant))
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(1, (steps + copies - 1) // copies)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            res[with_quant] = e0.elapsed_time(e1) * 1e3 / (reps * copies)
            del g
        us, us_q = res[False], res[True]
        out[str(M)] = {"us_per_4_linears": round(us, 2), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                       "frac_of_8TBps": round(nbytes / (us * 1e-6) / HBM_PEAK, 3),
                       "us_per_4_linears_with_quantize": round(us_q, 2),
                       "tokens_per_s_linears": round(M / (us_q * 1e-6), 1)}
    del blobs
    torch.cuda.empty_cache()
    return out


def decode_ceiling(dev, steps, copies=32,
                   workloads=(("llama_decode", "llama_mxfp4"), ("qwen_mxint4", "qwen_mxint4"),
                              ("llama_nvfp4", "llama_nvfp4"))):
    """The ceiling the decode GEMMs are compared with: at the byte count of
    each decode linear (M = 1), the rate of one launch that only reads that
    many bytes once (w4a4_probe_stream_read: 16-byte non-temporal loads, four
    in flight per lane), measured like decode_bandwidth (a HIP graph over 32
    distinct buffers, so none is served from the 256 MB last-level cache),
    beside the decode GEMM of the same linear alone, measured the same way;
    and the cost of one launch (an empty kernel)."""
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(1, (steps + copies - 1) // copies)

    def timed(fn):
        g = capture(fn)
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / (reps * copies)

    out = {}
    for workload, key in workloads:
        fmt = inputs.WORKLOADS[workload][1]
        res = {"read_probe": {}, "decode_gemm_M1": {}}
        tr = tg = total = 0.0
        for case in inputs.workload_cases(workload, M=1):
            L = Layer(case, dev)
            L.quantize()
            nbytes = gemm_bytes(fmt, 1, L.N, L.K)
            size = int(nbytes) // 16 * 16
            bufs = [torch.empty(size, dtype=torch.uint8, device=dev) for _ in range(copies)]
            us_r = timed(lambda: [w4.probe_stream_read(b, sink) for b in bufs])
            del bufs
            blobs = [L.blob.clone() for _ in range(copies)]
            us_g = timed(lambda: [L.gemm(b) for b in blobs])
            del blobs
            rate_r, rate_g = size / (us_r * 1e-6), nbytes / (us_g * 1e-6)
            res["read_probe"][case.name] = {"MB": round(size / 1e6, 2), "us": round(us_r, 2),
                                            "GB/s": round(rate_r / 1e9, 1),
                                            "frac_of_8TBps": round(rate_r / HBM_PEAK, 3)}
            res["decode_gemm_M1"][case.name] = {"us": round(us_g, 2), "GB/s": round(rate_g / 1e9, 1),
                                                "of_read_probe": round(rate_g / rate_r, 3)}
            tr, tg, total = tr + us_r, tg + us_g, total + nbytes
            del L
            torch.cuda.empty_cache()
        res["four_linears"] = {"read_probe_us": round(tr, 2), "read_probe_frac_of_8TBps": round(total / (tr * 1e-6) / HBM_PEAK, 3),
                               "decode_gemm_us": round(tg, 2), "gemm_of_read_probe": round(tr / tg, 3)}
        out[key] = res
    out["empty_kernel_us_per_launch"] = round(timed(lambda: [w4.probe_empty(dev) for _ in range(copies)]), 2)
    return out


def mfma_ceiling(dev, iters=400, reps=10, bursts=5):
    """The FP4 matrix-core rate without the GEMM around it
    (w4a4_probe_mfma_fp4: each wave holds a persistent-GEMM wave's 128 x 128
    fp32 tile and runs `iters` rounds of its 16 scaled 32 x 32 x 64 FP4 MFMAs
    on register operands): with random codes on all 256 CUs (the operand
    bits of a real GEMM), with zero codes (less power drawn), and with random
    codes on half the CUs (the power of the idle half goes to the clock of
    the busy one).  TFLOP/s from HIP-graph bursts of back-to-back launches."""
    g = torch.Generator(device="cpu").manual_seed(20261204)
    rnd = torch.randint(0, 256, (16384,), dtype=torch.uint8, generator=g).to(dev)
    zero = torch.zeros(16384, dtype=torch.uint8, device=dev)
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    out = {}
    for key, ops, wgs in (("random_256_workgroups", rnd, 256), ("zeros_256_workgroups", zero, 256),
                          ("random_128_workgroups", rnd, 128)):
        ms = time_launches(lambda: w4.probe_mfma_fp4(ops, iters, wgs, sink), reps=reps, bursts=bursts)
        flops = 2 * 128 * 128 * 64 * iters * 4 * wgs
        rate = flops / (ms * 1e-3)
        out[key] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(rate / 1e12, 1),
                    "frac_of_peak": round(rate / PEAK["mxfp4"][0], 4),
                    "per_CU_TFLOP/s": round(rate / wgs / 1e12, 2)}
    return out


def host_cpu():
    """(cores this process may run on, CPU model string)."""
    try:
        ncpu = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        ncpu = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return ncpu, model


def cpu_baseline(workload, M, rows=512, cols=4096):
    """The oracle as it stands, on a bounded sample: `rows` activation rows and
    `cols` weight rows of each linear.  Timed separately: the activation
    quantization (rescale, block scales, codes) and the linear (the weights'
    quantization plus the fp64 product with one BF16 rounding).  Reported in
    the workload's unit (TFLOP/s of the sampled GEMMs over both parts)."""
    import oracle
    from oracle.quant import quantize_rows, rescale, nv_tensor_scale, pack_codes
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    ncpu, model = host_cpu()
    flops, t_quant, t_lin = 0.0, 0.0, 0.0
    for case in inputs.workload_cases(workload, M=M):
        rr = np.arange(min(rows, case.M))
        cc = np.arange(min(cols, case.N))
        x = case.x.float().numpy()[rr]
        t0 = time.perf_counter()
        xt = rescale(x, case.c)
        ta = nv_tensor_scale(xt) if case.fmt == "nvfp4" else None
        ac, as_, _ = quantize_rows(xt, case.fmt, t=ta)
        ac = pack_codes(ac, case.fmt)
        t1 = time.perf_counter()
        if case.w_codes is not None:
            wc, ws, tw = case.w_codes[cc], case.w_scales[cc], case.t_w
        else:
            w = case.w_prescaled[cc].float().numpy()
            tw = nv_tensor_scale(w) if case.fmt == "nvfp4" else 1.0
            wq, ws, _ = quantize_rows(w, case.fmt, t=tw if case.fmt == "nvfp4" else None)
            wc = pack_codes(wq, case.fmt)
        oracle.linear_bf16(ac, as_, ta, wc, ws, tw, case.r[cc], case.fmt)
        t2 = time.perf_counter()
        t_quant += t1 - t0
        t_lin += t2 - t1
        flops += 2.0 * len(rr) * len(cc) * case.K
    secs = t_quant + t_lin
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle", "nproc": ncpu, "cpu_model": model,
            "quantize_act_s": round(t_quant, 3), "linear_s": round(t_lin, 3),
            "sample": f"{rows} activation rows x {cols} weight rows of each of the 4 linears "
                      f"(activation quantization {t_quant:.1f} s, weight quantization + fp64 linear "
                      f"{t_lin:.1f} s; the fp64 product on {blas_threads} BLAS threads, "
                      f"the quantization on one)"}


def gemm_kernel_label(fmt, M):
    """The GEMM kernels behind the roofline figure (all launches of a step)."""
    if fmt == "mxfp4":
        if M <= 16:
            return "gemm_fp4_decode16_kernel"
        if M <= 32:
            return "gemm_fp4_decode_kernel"
        return ("gemm_fp4_persistent_kernel (256x256 tiles; 256x192 tiles where those fill one "
                "round; n halves of 96..128-tile shapes), gemm_fp4_splitk_kernel (64..128 tiles, "
                "K >= 8192) and gemm_fp4_kernel (the others)")
    if fmt == "mxint4":
        if M <= 16:
            return ("gemm_mxint4_dot_kernel (VALU int4 dot products)" if M == 1 else
                    "gemm_decode_kernel<mxint4>")
        return ("gemm_mx_lean_kernel<mxint4> (256x256 tiles, where their rounds over the CUs are not "
                "coarser) and gemm_mx_kernel<mxint4> (256x128 tiles)")
    if fmt == "int4g64":
        if M <= 16:
            return "gemm_int4g64_dot_kernel (VALU int4 dot products)" if M <= 3 else "gemm_int4g64_decode_kernel"
        return "gemm_int4g64_f16_kernel (256x256 tiles for qkv and gate+up, 256x128 for o and down)"
    if fmt == "int8g128":
        if M <= 3:
            return ("gemm_int8g128_dot_kernel (VALU int8 dot products; the decode kernel where the rows "
                    "exceed 64 KiB of LDS)")
        if M <= 16:
            return "gemm_int8g128_decode_kernel (int8 MFMA, 16 features per workgroup)"
        if M <= 64:
            return "gemm_int8g128_tile_kernel (64x128 tiles, 32x128 for M <= 32)"
        return "gemm_int8g128_lds_kernel (128x128 tiles staged through a 4-deep LDS ring)"
    if fmt in ("mxfp8", "mxint8"):
        if M <= 3:
            return (f"gemm_mx8_dot_kernel<{fmt}> (VALU dot products; gemm_mx8_decode_kernel where the "
                    "rows exceed 64 KiB of LDS)")
        return (f"gemm_mx8_decode_kernel<{fmt}>" if M <= 16 else
                f"gemm_mx8_tile_kernel<{fmt}, 256, 128, 2, 2, 3>")
    if M == 1:
        return "gemm_nv_dot_kernel (VALU fp16 dot products)"
    return "gemm_nv_decode_kernel" if M <= 16 else "gemm_tile_kernel<nvfp4>"


def traffic_record(kernel, fmt="mxfp4"):
    """Measured HBM bytes per GEMM launch (FETCH_SIZE + WRITE_SIZE, each scaled
    by its reading for a 1 GiB copy), averaged over the workload's launches,
    from the committed rocprofv3 counter summary -- None unless the counters
    were taken on the current GEMM source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    name = {"int4g64": "int4g64.hip", "int8g128": "int8g128.hip"}.get(fmt, "gemm.hip")
    src = open(os.path.join(ROOT, "w4a4_block_scaled_amd", "csrc", name), "rb").read()
    if kernel not in rec:
        return None
    want = rec[kernel].get("source_sha256", rec.get("gemm_source_sha256"))
    if want != hashlib.sha256(src).hexdigest():
        return None
    return round(rec[kernel]["traffic_bytes_per_launch"])


def traffic_probe(layers, dev):
    """One device-to-device copy of exactly 1 GiB (the counter calibration:
    its FETCH_SIZE / WRITE_SIZE should read 1 GiB each), then one pass of the
    workload's kernels, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for L in layers:
        L.quantize()
        L.gemm()
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama_prefill", choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--M", type=int, default=None)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-solver", action="store_true")
    ap.add_argument("--no-formats", action="store_true",
                    help="skip the other formats' prefill and decode figures")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a 1 GiB calibration copy and one pass of the kernels, print nothing")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only the FP4 MFMA ceiling leg (scaled FP4 MFMAs on register operands)")
    ap.add_argument("--ceiling-probe", action="store_true",
                    help="only the decode ceiling leg (read probe, single-linear decode GEMMs, launch cost)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(the hot path would shard by tokens or by output features)",
              file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if a.ceiling_probe:
        print(json.dumps({"decode_ceiling": decode_ceiling(dev, a.steps)}), flush=True)
        return
    if a.mfma_probe:
        print(json.dumps({"mfma_ceiling": mfma_ceiling(dev)}), flush=True)
        return
    seed, fmt, Ms, lins = inputs.WORKLOADS[a.workload]
    M = a.M or Ms[-1]
    log(f"[bench] building {a.workload} M={M} ({fmt})")
    layers = [Layer(c, dev) for c in inputs.workload_cases(a.workload, M=M)]
    torch.cuda.synchronize()
    if a.traffic_probe:
        traffic_probe(layers, dev)
        return
    log("[bench] timing")
    # the step time from graph replays (and launched eagerly), then the
    # per-launch durations from graphs of back-to-back launches
    ms_eager = time_steps(layers, a.steps, a.warmup)
    ms = time_graph(layers, a.steps, a.warmup)
    gemm_ms, quant_ms = per_launch(layers, a.steps)
    flops = sum(L.flops for L in layers)
    value = flops / (ms * 1e-3) / 1e12
    peak, unit, bound = PEAK[fmt]
    achieved = sum(L.flops for L in layers) / (sum(gemm_ms) * 1e-3)   # per-launch average
    roof = {"bound": bound, "achieved": round(achieved / 1e12, 1), "peak": peak / 1e12,
            "unit": unit, "frac": round(achieved / peak, 4),
            "traffic": traffic_record(f"gemm_{a.workload}_M{M}", fmt),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes_per_launch": round(sum(L.gemm_bytes for L in layers) / len(layers)),
            "kernel": gemm_kernel_label(fmt, M),
            "per_linear": {L.case.name: {"us": round(t * 1e3, 2),
                                         "TFLOP/s": round(L.flops / (t * 1e-3) / 1e12, 1),
                                         "frac": round(L.flops / (t * 1e-3) / peak, 4)}
                           for L, t in zip(layers, gemm_ms)}}
    out = {"metric": "W4A4 linear TFLOPS & % MXFP4 MFMA peak (prefill); HBM GB/s (decode)",
           "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": round(ms, 4),
           "ms_per_step_eager": round(ms_eager, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": DTYPE[fmt], "data": "synthetic",
           "config": {"workload": a.workload, "format": fmt, "M": M,
                      "linears": [[L.case.name, L.N, L.K] for L in layers],
                      "step": "quantize_act + linear for each linear; weights packed once"},
           "tokens_per_s": round(M / (ms * 1e-3), 1),
           "quantize_act": {L.case.name: {"us": round(t * 1e3, 2),
                                          "GB/s": round(L.quant_bytes / (t * 1e-3) / 1e9, 1)}
                            for L, t in zip(layers, quant_ms)},
           "roofline": roof}
    del layers
    torch.cuda.empty_cache()
    if fmt == "mxfp4":
        log("[bench] FP4 MFMA ceiling: the MFMAs alone on register operands")
        out["mfma_ceiling"] = mfma_ceiling(dev)
        rc = out["mfma_ceiling"]["random_256_workgroups"]["TFLOP/s"]
        out["mfma_ceiling"]["gemm_achieved_of_random_256"] = round(roof["achieved"] / rc, 3)
        # beside the nominal peak: the same GEMM rate against what the FP4
        # MFMAs alone sustain on random operands on this chip (power-limited)
        roof["measured_mfma_ceiling"] = rc
        roof["frac_of_measured_mfma_ceiling"] = round(roof["achieved"] / rc, 4)
    if not a.no_decode:
        log("[bench] decode: MXFP4 Llama linears at M = 1, 4, 16")
        out["decode_hbm"] = decode_bandwidth(dev, a.steps)
        log("[bench] decode: MXINT4 Qwen, NVFP4 Llama at M = 1")
        out["decode_hbm_qwen_mxint4"] = decode_bandwidth(dev, a.steps, "qwen_mxint4", (1,))
        out["decode_hbm_llama_nvfp4"] = decode_bandwidth(dev, a.steps, "llama_nvfp4", (1,))
        log("[bench] decode ceiling: read probe and single-linear decode GEMMs")
        out["decode_ceiling"] = decode_ceiling(dev, a.steps)
    if not a.no_formats:
        # the other formats' prefill configurations, each against the peak of
        # the MFMA it runs on
        steps = max(5, a.steps // 4)
        out["prefill_formats"] = {}
        for wl, Mp in (("llama_nvfp4", 4096), ("qwen_mxint4", 512), ("qwen_mxint4", 4096),
                       ("llama_mxfp8", 2048), ("llama_mxint8", 2048), ("llama_int4g64", 2048),
                       ("llama_int8g128", 2048)):
            log(f"[bench] prefill {wl} M={Mp}")
            out["prefill_formats"][f"{wl}_M{Mp}"] = prefill_rates(dev, wl, Mp, steps, min(a.warmup, 5))
        if not a.no_decode:
            for wl in ("llama_mxfp8", "llama_mxint8", "llama_int4g64", "llama_int8g128"):
                log(f"[bench] decode {wl} M=1")
                out[f"decode_hbm_{wl}"] = decode_bandwidth(dev, a.steps, wl, (1,))
    if not a.no_solver:
        log("[bench] dual-scale solver")
        out["dualquant_solver"] = solver_rate(dev)
        log("[bench] per-projection c: q, k, v with their own column scales")
        out["per_projection"] = per_projection_rate(dev)
    if not a.no_cpu:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(a.workload, M)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
