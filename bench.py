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
HIP-event-timed average duration, against the MI355X dense MXFP4 peak),
decode weight-streaming bandwidth (MXFP4 Llama linears at M = 1, 4, 16,
MXINT4 Qwen linears and NVFP4 Llama linears at M = 1, cycling 32 layer
copies so that the 256 MB last-level cache cannot hold the weights), the
offline dual-scale solver on fp32 weights of the Llama linears' shapes, the
q, k, v projections with their own column scales (one multi-output quantize
and one grouped GEMM against three separate pairs), and the CPU oracle timed
on a
bounded sample of the same workload.
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
    "int4g64": (5.0e15, "TOP/s", "mfma"),    # int8 MFMA (5.0 POP/s dense)
}
HBM_PEAK = 8.0e12
DTYPE = {"mxfp4": "fp4", "nvfp4": "fp4xe4m3->fp16", "mxint4": "int4->fp8",
         "int4g64": "int4->int8 (bf16 block scales)"}
SCALE_BYTES = {"int4g64": 2}   # bytes per block scale (1 for E8M0 / UE4M3)


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
            if case.fmt == "int4g64":                       # BF16 bit patterns
                ws = torch.from_numpy(case.w_scales.view(np.int16)).to(dev).view(torch.bfloat16)
            tw = torch.tensor([case.t_w], dtype=torch.float32, device=dev)
        else:
            wc, ws, tw = w4.quantize_act(case.w_prescaled.to(dev), None, case.fmt)
        self.blob = w4.pack_weight(wc, ws, tw, torch.from_numpy(case.r).to(dev), case.fmt)
        del wc, ws
        self.x = case.x.to(dev)
        self.c = torch.from_numpy(case.c).to(dev)
        G = w4.block_size(case.fmt)
        self.codes = torch.empty((self.M, self.K // 2), dtype=torch.uint8, device=dev)
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
        return 2 * self.M * self.K + 4 * self.K + self.M * self.K / 2 + self.M * self.K / G

    @property
    def gemm_bytes(self):
        G = w4.block_size(self.fmt) / SCALE_BYTES.get(self.fmt, 1)
        return (self.N * self.K / 2 + self.N * self.K / G + 4 * self.N + self.M * self.K / 2 +
                self.M * self.K / G + 2 * self.M * self.N)


def time_steps(layers, steps, warmup, with_events=True):
    """Run warmup + timed steps; returns (ms per step, per-layer GEMM ms list,
    per-layer quantize_act ms list), the per-layer figures from HIP events
    recorded on the stream the kernels run on."""
    for _ in range(warmup):
        for L in layers:
            L.quantize()
            L.gemm()
    torch.cuda.synchronize()
    ev = [[tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in layers]
          for _ in range(steps)] if with_events else None
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s in range(steps):
        for i, L in enumerate(layers):
            if with_events:
                ev[s][i][0].record()
            L.quantize()
            if with_events:
                ev[s][i][1].record()
            L.gemm()
            if with_events:
                ev[s][i][2].record()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    gemm_ms = quant_ms = None
    if with_events:
        gemm_ms = [float(np.mean([ev[s][i][1].elapsed_time(ev[s][i][2]) for s in range(steps)]))
                   for i in range(len(layers))]
        quant_ms = [float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)]))
                    for i in range(len(layers))]
    return ms, gemm_ms, quant_ms


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
    warm-up solve, then one timed solve per linear.  Every pass reads W once
    (fp32), 2T + 2 passes per solve; the rate is those reads over the time
    (the passes are HBM-bound), against 8 TB/s."""
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
        rate = (2 * iters + 2) * 4.0 * N * K / (ms * 1e-3) / 1e9
        out[name] = {"N": N, "K": K, "ms": round(ms, 3), "W_read_GB/s": round(rate, 1),
                     "frac_of_8TBps": round(rate / 8000.0, 3)}
        del w, ws
        torch.cuda.empty_cache()
    return {"format": "mxfp4", "iters": iters, "layer_ms": round(total, 3), "per_linear": out}


def int4g64_rates(dev, steps, warmup, M=2048):
    """INT4 G=64 with BF16 block scales (the pages' packed deployment format)
    on the Llama linears: prefill at M tokens (quantize_act + linear per
    linear, graph-timed step; GEMM rates from per-launch events, against the
    int8 MFMA peak) and the decode weight-streaming rate at M = 1."""
    layers = [Layer(c, dev) for c in inputs.workload_cases("llama_int4g64", M=M)]
    torch.cuda.synchronize()
    _, gemm_ms, quant_ms = time_steps(layers, steps, warmup)
    ms = time_graph(layers, steps, warmup)
    peak = PEAK["int4g64"][0]
    ops = sum(L.flops for L in layers)
    out = {"prefill_M%d" % M: {
        "step_ms": round(ms, 4), "TOP/s_step": round(ops / (ms * 1e-3) / 1e12, 1),
        "TOP/s_gemm": round(ops / (sum(gemm_ms) * 1e-3) / 1e12, 1),
        "frac_of_int8_peak": round(ops / (sum(gemm_ms) * 1e-3) / peak, 4),
        "traffic": traffic_record(f"gemm_llama_int4g64_M{M}", "int4g64"),
        "kernel": gemm_kernel_label("int4g64", M),
        "per_linear": {L.case.name: {"gemm_us": round(t * 1e3, 2),
                                     "TOP/s": round(L.flops / (t * 1e-3) / 1e12, 1),
                                     "quantize_us": round(qt * 1e3, 2)}
                       for L, t, qt in zip(layers, gemm_ms, quant_ms)}}}
    del layers
    torch.cuda.empty_cache()
    out["decode_hbm"] = decode_bandwidth(dev, steps, "llama_int4g64", (1,))
    return out


def decode_bandwidth(dev, steps, workload="llama_decode", Ms=(1, 4, 16), copies=32):
    """Weight-streaming rate of the GEMM at small M (default: MXFP4 Llama
    shapes at M = 1, 4, 16).

    Each step runs the four linears of one "layer"; 32 distinct copies of the
    packed weights (3.7 GB for Llama, like the 32 layers of the model) are
    cycled so that no copy is still cached.  The 32 layers are captured as
    one HIP graph and replayed, so the figure is the GPU's, not the host's
    launch rate.
    """
    out = {}
    fmt = inputs.WORKLOADS[workload][1]
    base = [Layer(c, dev) for c in inputs.workload_cases(workload, M=max(Ms))]
    blobs = [[L.blob.clone() for L in base] for _ in range(copies)]
    for M in Ms:
        cases = inputs.workload_cases(workload, M=M, build_weights=False)
        act = [(c.x.to(dev), torch.from_numpy(c.c).to(dev)) for c in cases]
        # quantized activations for this M
        q = [w4.quantize_act(x, c, fmt) for x, c in act]
        ys = [torch.empty((M, L.N), dtype=torch.bfloat16, device=dev) for L in base]
        G = w4.block_size(fmt) / SCALE_BYTES.get(fmt, 1)
        nbytes = sum(L.N * L.K / 2 + L.N * L.K / G + 4 * L.N + M * L.K / 2 + M * L.K / G +
                     2 * M * L.N for L in base)

        def run_layer(k):
            for j, L in enumerate(base):
                w4.linear(q[j][0], q[j][1], q[j][2], blobs[k % copies][j], fmt, L.N, L.K, out=ys[j])

        def run_model():
            for k in range(copies):
                run_layer(k)

        g = capture(run_model)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, (steps + copies - 1) // copies)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
        del g
        out[str(M)] = {"us_per_4_linears": round(us, 2), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                       "frac_of_8TBps": round(nbytes / (us * 1e-6) / HBM_PEAK, 3)}
    del blobs
    return out


def cpu_baseline(workload, M, rows=512, cols=4096):
    """The oracle as it stands, on a bounded sample: `rows` activation rows and
    `cols` weight rows of each linear (quantization of both plus the fp64
    linear).  Reported in the workload's unit (TFLOP/s of the sampled GEMM)."""
    import oracle
    from oracle.quant import quantize_rows, rescale, nv_tensor_scale, pack_nibbles
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    flops, secs = 0.0, 0.0
    for case in inputs.workload_cases(workload, M=M):
        rr = np.arange(min(rows, case.M))
        cc = np.arange(min(cols, case.N))
        x = case.x.float().numpy()[rr]
        t0 = time.perf_counter()
        xt = rescale(x, case.c)
        ta = nv_tensor_scale(xt) if case.fmt == "nvfp4" else None
        ac, as_, _ = quantize_rows(xt, case.fmt, t=ta)
        if case.w_codes is not None:
            wc, ws, tw = case.w_codes[cc], case.w_scales[cc], case.t_w
        else:
            w = case.w_prescaled[cc].float().numpy()
            tw = nv_tensor_scale(w) if case.fmt == "nvfp4" else 1.0
            wq, ws, _ = quantize_rows(w, case.fmt, t=tw if case.fmt == "nvfp4" else None)
            wc = pack_nibbles(wq)
        oracle.linear_bf16(pack_nibbles(ac), as_, ta, wc, ws, tw, case.r[cc], case.fmt)
        secs += time.perf_counter() - t0
        flops += 2.0 * len(rr) * len(cc) * case.K
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} activation rows x {cols} weight rows of each of the 4 linears "
                      f"(quantize both + fp64 linear), {secs:.1f} s"}


def gemm_kernel_label(fmt, M):
    """The GEMM kernels behind the roofline figure (all launches of a step)."""
    if fmt == "mxfp4":
        if M <= 16:
            return "gemm_fp4_decode16_kernel"
        if M <= 32:
            return "gemm_fp4_decode_kernel"
        return ("gemm_fp4_persistent_kernel (linears of 192+ tiles of 256x256), "
                "gemm_fp4_splitk_kernel (64..128 tiles, K >= 8192) and gemm_fp4_kernel (the others)")
    if fmt == "mxint4":
        if M <= 16:
            return "gemm_decode_kernel<mxint4>"
        return ("gemm_mx_lean_kernel<mxint4> (256x256 tiles, where their rounds over the CUs are not "
                "coarser) and gemm_mx_kernel<mxint4> (256x128 tiles)")
    if fmt == "int4g64":
        return "gemm_int4g64_decode_kernel" if M <= 16 else "gemm_int4g64_tile_kernel<4, 4>"
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
    name = "int4g64.hip" if fmt == "int4g64" else "gemm.hip"
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
    ap.add_argument("--no-int4g64", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a 1 GiB calibration copy and one pass of the kernels, print nothing")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(the hot path would shard by tokens or by output features)",
              file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    seed, fmt, Ms, lins = inputs.WORKLOADS[a.workload]
    M = a.M or Ms[-1]
    log(f"[bench] building {a.workload} M={M} ({fmt})")
    layers = [Layer(c, dev) for c in inputs.workload_cases(a.workload, M=M)]
    torch.cuda.synchronize()
    if a.traffic_probe:
        traffic_probe(layers, dev)
        return
    log("[bench] timing")
    # per-launch durations from HIP events around each launch (eager), then
    # the step time from graph replays
    ms_eager, gemm_ms, quant_ms = time_steps(layers, a.steps, a.warmup)
    ms = time_graph(layers, a.steps, a.warmup)
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
    if not a.no_decode:
        log("[bench] decode bandwidth")
        out["decode_hbm"] = decode_bandwidth(dev, a.steps)
        torch.cuda.empty_cache()
        out["decode_hbm_qwen_mxint4"] = decode_bandwidth(dev, a.steps, "qwen_mxint4", (1,))
        torch.cuda.empty_cache()
        out["decode_hbm_llama_nvfp4"] = decode_bandwidth(dev, a.steps, "llama_nvfp4", (1,))
    if not a.no_solver:
        log("[bench] dual-scale solver")
        out["dualquant_solver"] = solver_rate(dev)
        log("[bench] per-projection c: q, k, v with their own column scales")
        out["per_projection"] = per_projection_rate(dev)
    if not a.no_int4g64 and a.workload != "llama_int4g64":
        log("[bench] INT4 G=64 with BF16 scales (Llama, prefill and decode)")
        out["int4g64"] = int4g64_rates(dev, a.steps, a.warmup)
    if not a.no_cpu:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(a.workload, M)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
