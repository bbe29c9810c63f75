#!/usr/bin/env python3
"""NVFP4 prefill linear throughput on one MI355X, activation quantization included.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2|3|5]

One step = one pass of the prefill hot path over one 8B-shaped decoder layer
(default: M=4096 tokens through q,k,v,o,gate,up,down): each of the layer's
four activation tensors is quantized to NVFP4 on the fly (amax pass +
encode), then every NVFP4 x NVFP4 GEMM that consumes it runs (bf16 output).
Projections that read the same activation share a launch where that fills
the GPU better (k with v, gate with up: mq_gemm_nvfp4_prefill_grouped);
``--launches separate`` runs one launch per projection instead.
Weights are quantized once before timing (offline, as the method keeps them
in the low-precision format).  With --config 3 (M=32768) every GEMM instead
quantizes its bf16 input in its own prologue: by default each workgroup
quantizes the 256-row panel of A its tiles read, once, into A's NVFP4
buffers and multiplies from them (``--fused-form tile``: every A tile is
re-quantized inside the GEMM's pipeline for each column tile).  Inputs are
seeded synthetic bf16 tensors, resident in HBM before the timed region.

Prints one JSON line with the whole-step TFLOP/s, the roofline of the
dominant kernel (the GEMM), torch's BF16 GEMM at the same shapes for
comparison, and the CPU oracle's throughput on a bounded sample.

Two timed passes of K steps each: the first, with no events in it, gives
`value` and `ms_per_step`; the second repeats the same K steps with HIP
events around every GEMM launch (on the launching stream) and gives the
GEMM kernel's average launch duration for the roofline and the per-launch
split.  Event records are kept out of the first pass because each costs the
step a few microseconds (about 30 us over a default step's ten events).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 prefill GEMM TFLOP/s incl. act-quant at 8B shapes; % MFMA peak"
PEAK_F16_MFMA_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200, help="timed steps (a default step takes about 1.4 ms)")
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=2, choices=(2, 3, 5))
    p.add_argument("--launches", choices=("grouped", "separate"), default="grouped",
                   help="grouped: k+v and gate+up as one launch each; separate: one launch per projection")
    p.add_argument("--fused-form", choices=("panel", "tile"), default="panel",
                   help="config 3's fused quantization: panel = each workgroup quantizes its 256-row A panel "
                        "once into A's NVFP4 buffers, then multiplies from them; tile = every A tile is "
                        "re-quantized in the GEMM's pipeline for each column tile")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-bf16", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the per-kernel rates measured after the timed region (quantizer and decode GEMV)")
    p.add_argument("--cpu-rows", type=int, default=4096, help="activation rows in the CPU sample (at most M)")
    p.add_argument("--cpu-wrows", type=int, default=4096, help="weight rows per projection in the CPU sample")
    p.add_argument("--layer", action="store_true",
                   help="only the decoder-layer prefill context measurement (NVFP4 vs BF16 linears)")
    p.add_argument("--single-linear", action="store_true",
                   help="only the one-linear configuration (M=128, K=N=512): per-call latency of each form")
    p.add_argument("--decode-only", action="store_true",
                   help="only measure the BF16 decode GEMV at the decode shapes (one JSON line, not the step metric)")
    p.add_argument("--peak", action="store_true",
                   help="only measure the fp16 MFMA rate the chip sustains (MFMA only, and with 4 and 6 VALU "
                        "instructions per MFMA as the GEMM's dequantization issues) and the clock it holds")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain elementwise copy of 1 GiB (reads 1 GiB, writes 1 GiB) three "
                        "times, as the reference for scaling HBM byte counters")
    return p.parse_args()


def copy_calibration():
    import torch
    n = (1 << 30) // 2
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": 1 << 30, "bytes_written": 1 << 30, "launches": 3,
                                           "kernel": "torch.neg (elementwise, bf16)"}}), flush=True)


def mfma_peak(reps=5, iters=20000, warm=10):
    """The fp16 MFMA rate of the GEMM's register-resident inner loop (4x4
    fragments of v_mfma_f32_32x32x16_f16 per wave, one wave per SIMD on
    every CU, no memory traffic) with 0, 4 and 6 VALU instructions per MFMA:
    median TFLOP/s over `reps` event-timed launches, and the clock the SIMDs
    ran at, from each block's shader-clock and constant-rate counters
    (s_memtime / s_memrealtime) over its run; `warm` untimed launches of each
    variant come first (the clock ramps up over the first ~0.1 s of load).  The datasheet peak assumes
    2.4 GHz; `peak_at_clock` is what 256 CUs x 4 SIMDs x 1024 flop/cycle give
    at the measured clock, and `mfma_busy` the achieved share of it."""
    import statistics
    import torch
    import fp4_block_scaled_elem_amd as mq
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros((blocks, 4), dtype=torch.int64, device="cuda")
    khz = mq.wall_clock_khz()
    flops = blocks * 4 * iters * 32 * 32768
    res = {"datasheet_tflops": PEAK_F16_MFMA_TFLOPS, "cus": blocks, "wall_clock_khz": khz}
    for v in (0, 4, 6):
        for _ in range(warm):
            mq.mq_check_mfma_rate(v, iters, blocks, sink, clocks)
        ts, mhz = [], []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            mq.mq_check_mfma_rate(v, iters, blocks, sink, clocks)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
            c = clocks.cpu().numpy().astype("float64")
            mhz.append(float(((c[:, 2] - c[:, 0]) / (c[:, 3] - c[:, 1])).mean() * khz / 1e3))
        t = statistics.median(ts)
        f = statistics.median(mhz)
        at_clock = blocks * 4 * 1024 * f * 1e6 / 1e12
        res[f"valu_per_mfma_{v}"] = {"tflops": round(flops / t / 1e12, 1), "ms": round(t * 1e3, 3),
                                     "clock_mhz": round(f, 1), "peak_at_clock_tflops": round(at_clock, 1),
                                     "mfma_busy": round(flops / t / 1e12 / at_clock, 4)}
    return res


def dev_bf16(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def setup(cfg_id):
    import torch
    import fp4_block_scaled_elem_amd as mq
    import workloads
    cfg = workloads.CONFIGS[cfg_id]
    M = cfg.M[0]
    acts_host = {a: workloads.activation(cfg_id, a) for a in workloads.ACTS}
    acts = {a: dev_bf16(b) for a, b in acts_host.items()}
    qw, wdev = {}, {}
    for p in cfg.projs:
        wb = workloads.weight(cfg_id, p)
        wdev[p] = dev_bf16(wb)
        qw[p] = mq.quantize(wdev[p])          # offline weight quantization
    qa = {a: mq.NVFP4.empty(*acts[a].shape) for a in workloads.ACTS}
    fa = {p: mq.NVFP4(None, None, torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda"))
          for p in cfg.projs}
    out = {p: torch.empty((M, cfg.layer.proj_nk(p)[0]), dtype=torch.bfloat16, device="cuda")
           for p in cfg.projs}
    torch.cuda.synchronize()
    return cfg, acts_host, acts, wdev, qw, qa, fa, out


def setup_device(cfg_id, seed=0):
    """Like setup(), but every input is drawn on the GPU with torch's seeded
    generator (same shapes and distributions as the configuration's recipe:
    normal or unit-variance Student-t activations with the stated share of
    outlier columns, normal weights; not the bit patterns workloads.py
    draws).  For the timing-only legs of the default run, where drawing the
    long-context and 70B-slice tensors on the host would take minutes."""
    import torch
    import fp4_block_scaled_elem_amd as mq
    import workloads
    cfg = workloads.CONFIGS[cfg_id]
    M = cfg.M[0]
    gen = torch.Generator(device="cuda").manual_seed(10_000 * cfg_id + seed)

    def draw(rows, cols, dist):
        if dist.kind == "normal":
            x = torch.randn((rows, cols), generator=gen, device="cuda")
        else:  # Student-t: normal / sqrt(chi2_df / df), scaled to unit variance
            z = torch.randn((rows, cols), generator=gen, device="cuda")
            chi2 = torch._standard_gamma(torch.full((rows, cols), dist.df / 2.0, device="cuda"), generator=gen) * 2.0
            x = z / torch.sqrt(chi2 / dist.df) * ((dist.df - 2.0) / dist.df) ** 0.5
            del z, chi2
        x *= dist.std
        if dist.outlier_frac > 0:
            n = int(round(dist.outlier_frac * cols))
            idx = torch.randperm(cols, generator=gen, device="cuda")[:n]
            x[:, idx] *= dist.outlier_factor
        return x.to(torch.bfloat16)

    acts = {a: draw(M, cfg.layer.act_k(a), cfg.act) for a in workloads.ACTS}
    qw, wdev = {}, {}
    for p in cfg.projs:
        n, k = cfg.layer.proj_nk(p)
        wdev[p] = draw(n, k, cfg.weight)
        qw[p] = mq.quantize(wdev[p])
    qa = {a: mq.NVFP4.empty(*acts[a].shape) for a in workloads.ACTS}
    fa = {p: mq.NVFP4(None, None, torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda"))
          for p in cfg.projs}
    out = {p: torch.empty((M, cfg.layer.proj_nk(p)[0]), dtype=torch.bfloat16, device="cuda")
           for p in cfg.projs}
    torch.cuda.synchronize()
    return cfg, None, acts, wdev, qw, qa, fa, out


def config_step_rate(cfg_id, steps, warmup, fused_form="panel"):
    """Whole-step TFLOP/s of another prefill configuration (the long-context
    M=32768 step with quantization fused into every GEMM, or the 70B-shaped
    slice at M=16384), on device-drawn inputs, timed like the headline: W
    untimed steps, then K steps between two synchronisations."""
    import torch
    import workloads
    cfg, _, acts, wdev, qw, qa, fa, out = setup_device(cfg_id)
    if cfg.fused_act_quant and fused_form == "panel":
        fa = {p: qa[workloads.PROJ_INPUT[p]] for p in cfg.projs}
    plan = launch_plan(cfg, "grouped")
    for _ in range(warmup):
        run_step(cfg, plan, acts, qw, qa, fa, out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run_step(cfg, plan, acts, qw, qa, fa, out)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    flops = cfg.flops()
    res = {"workload": cfg.name, "M": cfg.M[0], "inputs": "drawn on the GPU (torch generator)",
           "act_quant": f"fused-{fused_form}" if cfg.fused_act_quant else "separate",
           "tflops": round(flops / dt / 1e12, 1), "ms_per_step": round(dt * 1e3, 4),
           "pct_mfma_peak": round(100.0 * flops / dt / 1e12 / PEAK_F16_MFMA_TFLOPS, 2),
           "steps": steps, "warmup": warmup}
    del acts, wdev, qw, qa, fa, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def single_linear_latency(reps=50):
    """The one-linear configuration (M=128, K=512, N=512, seeded inputs of
    workloads.py), per call, in microseconds: quantize the activations (one
    launch: on an input this small every workgroup of the quantizer takes
    the maximum itself) and run the NVFP4 GEMM, and the same linear with
    the quantization fused into the GEMM (one launch, bit-identical output)
    -- calls made back to back from Python (eager) and the same calls
    captured in a HIP graph and replayed (the kernels' own time).  67 MFLOP
    is far too little work for a throughput figure; this configuration
    measures launch latency.  On 128 rows the GEMM is the small-problem
    kernel (K split over each workgroup's waves, 256 workgroups)."""
    import torch
    import fp4_block_scaled_elem_amd as mq
    import workloads
    x = dev_bf16(workloads.activation(1))
    qw = mq.quantize(dev_bf16(workloads.weight(1)))
    qa = mq.NVFP4.empty(128, 512)
    c = torch.empty((128, 512), dtype=torch.bfloat16, device="cuda")

    def call(_):
        mq.mq_quantize_nvfp4(x, qa)
        mq.mq_gemm_nvfp4_prefill(qa, None, qw, c)

    med, mn = _median_us(call, reps=reps)
    g = _graph_us(call, c)
    # the same linear with the quantization inside the GEMM: on an input this
    # small the GEMM's workgroups also take the maximum, so it is one launch
    rec = mq.NVFP4(None, None, torch.zeros(mq.REC_BYTES // 4, dtype=torch.int32, device="cuda"))
    cf = torch.empty_like(c)
    fused = lambda _: mq.mq_gemm_nvfp4_prefill(rec, x, qw, cf, mq.MQ_A_FUSED_BF16)
    fmed, fmn = _median_us(fused, reps=reps)
    fg = _graph_us(fused, cf)
    # the GEMM alone on the already quantized activation
    cg = torch.empty_like(c)
    gemm_only = lambda _: mq.mq_gemm_nvfp4_prefill(qa, None, qw, cg)
    gg = _graph_us(gemm_only, cg)
    torch.cuda.synchronize()
    if not torch.equal(c.view(torch.int16), cf.view(torch.int16)):
        raise RuntimeError("fused single-launch linear differs from quantize + GEMM")
    if not torch.equal(c.view(torch.int16), cg.view(torch.int16)):
        raise RuntimeError("GEMM on the quantized activation differs from quantize + GEMM")
    flops = 2 * 128 * 512 * 512
    return {"workload": workloads.CONFIGS[1].name,
            "gemm_only": {"launches": 1, "us_graph": round(gg, 2), "tflops_graph": round(flops / gg / 1e6, 2)},
            "quantize_then_gemm": {"launches": 2, "us_median_eager": round(med, 2), "us_min_eager": round(mn, 2),
                                   "us_graph": round(g, 2), "tflops_graph": round(flops / g / 1e6, 2)},
            "fused_one_launch": {"launches": 1, "us_median_eager": round(fmed, 2), "us_min_eager": round(fmn, 2),
                                 "us_graph": round(fg, 2), "tflops_graph": round(flops / fg / 1e6, 2)}}


# projections launched together (they read the same activation)
GROUPED = (("q",), ("k", "v"), ("o",), ("gate", "up"), ("down",))


def launch_plan(cfg, mode):
    """[(activation, (projections of one launch))] in execution order."""
    import workloads
    groups = GROUPED if mode == "grouped" else tuple((p,) for p in cfg.projs)
    plan = []
    for a in workloads.ACTS:
        for g in groups:
            g = tuple(p for p in g if p in cfg.projs and workloads.PROJ_INPUT[p] == a)
            if g:
                plan.append((a, g))
    assert sorted(p for _, g in plan for p in g) == sorted(cfg.projs)
    return plan


def run_step(cfg, plan, acts, qw, qa, fa, out, events=None):
    import fp4_block_scaled_elem_amd as mq
    import workloads
    for a in workloads.ACTS:
        if not cfg.fused_act_quant:
            mq.mq_quantize_nvfp4(acts[a], qa[a])
        for act, g in plan:
            if act != a:
                continue
            if events is not None:
                events["g"].append(_ev())
            if cfg.fused_act_quant:
                A, x, flags = fa[g[0]], acts[a], mq.MQ_A_FUSED_BF16
            else:
                A, x, flags = qa[a], None, 0
            if len(g) == 1:
                mq.mq_gemm_nvfp4_prefill(A, x, qw[g[0]], out[g[0]], flags)
            else:
                mq.mq_gemm_nvfp4_prefill_grouped(A, x, [qw[p] for p in g], [out[p] for p in g], flags)
            if events is not None:
                events["g"].append(_ev())


def _ev():
    import torch
    e = torch.cuda.Event(enable_timing=True)
    e.record()  # on the current stream, which the binding launches on
    return e


def _pairs_ms(evs):
    return sum(evs[i].elapsed_time(evs[i + 1]) for i in range(0, len(evs), 2))


def _median_us(fn, reps=50, warm=20, batch=10):
    """Median and min over `reps` HIP-event timings of the per-call duration
    of `batch` back-to-back calls (fn(i) with i counting calls, so inputs can
    rotate); a lone call would be dominated by launch latency."""
    import statistics
    import torch
    i = 0
    for _ in range(warm):
        fn(i)
        i += 1
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(batch):
            fn(i)
            i += 1
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / batch)
    return statistics.median(ts), min(ts)


def _graph_us(fn, out, calls=20, reps=20):
    """Median per-call microseconds of `calls` calls (fn(i)) captured in one
    HIP graph and replayed `reps` times: the kernels' own back-to-back time,
    without the host's per-call launch cost that bounds small calls made one
    by one.  Every replay's output must equal the eager result of the last
    call (the captured calls record no memsets; the check makes sure)."""
    import statistics
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    fn(calls - 1)
    torch.cuda.synchronize()
    ref = out.clone()
    ts = []
    for _ in range(reps):
        out.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / calls)
        if not torch.equal(out.view(torch.int16), ref.view(torch.int16)):
            raise RuntimeError("graph replay differs from the eager call")
    del g
    return statistics.median(ts)


def per_launch(cfg, plan, acts, qw, qa, fa, out, events, steps):
    """TFLOP/s of each launch of the step, from the events of the kernel-timing pass."""
    import workloads
    res = {}
    n = len(plan)
    for idx, (a, g) in enumerate(plan):
        ms = sum(events["g"][2 * (s * n + idx)].elapsed_time(events["g"][2 * (s * n + idx) + 1])
                 for s in range(steps)) / steps
        flops = sum(2 * cfg.M[0] * cfg.layer.proj_nk(p)[0] * cfg.layer.proj_nk(p)[1] for p in g)
        res["+".join(g)] = {"us": round(ms * 1e3, 2), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
    return res


def act_quant_rates(acts):
    """The standalone quantizer per activation tensor: achieved GB/s for the
    single-read algorithmic bytes (2 + 0.5625 per element) and for the bytes
    the two passes move (the amax pass reads the input again).  Inputs and
    outputs rotate over copies so the working set exceeds the 256 MB
    Infinity Cache."""
    import fp4_block_scaled_elem_amd as mq
    res = {}
    for a, x0 in acts.items():
        n = x0.numel()
        ncopy = max(2, -(-600 * 2 ** 20 // (n * 2)))
        xs = [x0.clone() for _ in range(ncopy)]
        qs = [mq.NVFP4.empty(*x0.shape) for _ in range(ncopy)]
        med, mn = _median_us(lambda r: mq.mq_quantize_nvfp4(xs[r % ncopy], qs[r % ncopy]))
        del xs, qs
        res[a] = {"shape": list(x0.shape), "us_median": round(med, 2), "us_min": round(mn, 2),
                  "GBps_1pass": round(n * 2.5625 / med / 1e3, 1), "GBps_2pass": round(n * 4.5625 / med / 1e3, 1),
                  "pct_hbm_2pass": round(100 * n * 4.5625 / med / 1e3 / PEAK_HBM_GBS, 1)}
    return res


def decode_gemv_rates(reps=50):
    """The BF16 decode GEMV at the decode configuration's shapes (M in
    {1, 4, 16, 32} x the 8B layer's (N, K) pairs), weights rotated over copies
    so that the working set exceeds the 256 MB Infinity Cache; achieved GB/s
    over 2NK + 2MK + 2MN bytes, and torch's BF16 linear at the same shapes."""
    import torch
    import torch.nn.functional as F
    import fp4_block_scaled_elem_amd as mq
    import workloads
    lay = workloads.LLAMA8B
    res = {}
    for p in ("q", "k", "gate", "down"):
        N, K = lay.proj_nk(p)
        ncopy = max(2, -(-600 * 2 ** 20 // (2 * N * K)))
        gen = torch.Generator(device="cuda").manual_seed(1000 + N + K)
        ws = [(torch.randn((N, K), generator=gen, device="cuda") * 0.02).to(torch.bfloat16) for _ in range(ncopy)]
        for M in (1, 4, 16, 32):
            x = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            med, mn = _median_us(lambda r: mq.mq_gemv_bf16_decode(x, ws[r % ncopy], y), reps=reps)
            gus = _graph_us(lambda r: mq.mq_gemv_bf16_decode(x, ws[r % ncopy], y), y)
            tmed, _ = _median_us(lambda r: F.linear(x, ws[r % ncopy]), reps=reps)
            b = 2 * N * K + 2 * M * K + 2 * M * N
            res[f"{p}_M{M}"] = {"N": N, "K": K, "M": M, "us_median": round(med, 2), "us_min": round(mn, 2),
                                "GBps": round(b / med / 1e3, 1), "pct_hbm": round(100 * b / med / 1e3 / PEAK_HBM_GBS, 1),
                                "us_graph": round(gus, 2), "GBps_graph": round(b / gus / 1e3, 1),
                                "torch_us": round(tmed, 2)}
        del ws
    return res


def decode_layer_rates():
    """One 8B-shaped decoder layer's decode linears on BF16 weights (q, k, v,
    o, gate, up, down: 432 MB, more than the 256 MB Infinity Cache, so every
    step streams them from HBM), M in {1, 4, 16, 32}: seven launches of
    mq_gemv_bf16_decode vs four (q+k+v and gate+up through
    mq_gemv_bf16_decode_grouped: they read the same input).  Both timed as
    graph replays (the kernels' own time); GB/s over the weights' bytes."""
    import torch
    import fp4_block_scaled_elem_amd as mq
    import workloads
    lay = workloads.LLAMA8B
    gen = torch.Generator(device="cuda").manual_seed(3000)
    projs = ("q", "k", "v", "o", "gate", "up", "down")
    w = {p: (torch.randn(lay.proj_nk(p), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
         for p in projs}
    wbytes = sum(2 * t.numel() for t in w.values())
    res = {}
    for M in (1, 4, 16, 32):
        x = {a: torch.randn((M, lay.act_k(a)), generator=gen, device="cuda").to(torch.bfloat16)
             for a in ("x_qkv", "x_o", "x_gu", "x_down")}
        inp = {"q": "x_qkv", "k": "x_qkv", "v": "x_qkv", "o": "x_o", "gate": "x_gu", "up": "x_gu",
               "down": "x_down"}
        y = {p: torch.empty((M, lay.proj_nk(p)[0]), dtype=torch.bfloat16, device="cuda") for p in projs}

        def singles(_):
            for p in projs:
                mq.mq_gemv_bf16_decode(x[inp[p]], w[p], y[p])

        def grouped(_):
            mq.mq_gemv_bf16_decode_grouped(x["x_qkv"], [w["q"], w["k"], w["v"]], [y["q"], y["k"], y["v"]])
            mq.mq_gemv_bf16_decode(x["x_o"], w["o"], y["o"])
            mq.mq_gemv_bf16_decode_grouped(x["x_gu"], [w["gate"], w["up"]], [y["gate"], y["up"]])
            mq.mq_gemv_bf16_decode(x["x_down"], w["down"], y["down"])

        t7 = _graph_us(singles, y["v"], calls=5)
        t4 = _graph_us(grouped, y["v"], calls=5)
        res[f"M{M}"] = {"us_7_launches": round(t7, 2), "us_4_launches": round(t4, 2),
                        "GBps_4_launches": round(wbytes / t4 / 1e3, 1), "speedup": round(t7 / t4, 3)}
        del x, y
    del w
    return res


def decode_nvfp4_rates(bf16_rates=None, reps=50):
    """The uniform-NVFP4 decode GEMV (X and W both NVFP4) at the decode
    configuration's shapes, M in {1, 16, 32}; weights rotated over copies
    past the 256 MB Infinity Cache.  GB/s over the algorithmic bytes
    0.5625 (N K + M K) + 2 M N, and the time relative to the BF16 decode GEMV
    at the same shape (bf16_rates: decode_gemv_rates' result).  X is
    quantized once outside the timed calls (its M x K elements are small)."""
    import torch
    import fp4_block_scaled_elem_amd as mq
    import workloads
    lay = workloads.LLAMA8B
    res = {}
    for p in ("q", "k", "gate", "down"):
        N, K = lay.proj_nk(p)
        wbytes = N * K * 9 // 16
        ncopy = max(2, -(-600 * 2 ** 20 // wbytes))
        gen = torch.Generator(device="cuda").manual_seed(2000 + N + K)
        ws = []
        for _ in range(ncopy):
            ws.append(mq.quantize((torch.randn((N, K), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)))
        for M in (1, 16, 32):
            xq = mq.quantize(torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16))
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            med, mn = _median_us(lambda r: mq.mq_gemv_nvfp4_decode(xq, ws[r % ncopy], y), reps=reps)
            gus = _graph_us(lambda r: mq.mq_gemv_nvfp4_decode(xq, ws[r % ncopy], y), y)
            b = (N * K + M * K) * 9 // 16 + 2 * M * N
            e = {"N": N, "K": K, "M": M, "us_median": round(med, 2), "us_min": round(mn, 2),
                 "GBps": round(b / med / 1e3, 1), "pct_hbm": round(100 * b / med / 1e3 / PEAK_HBM_GBS, 1),
                 "us_graph": round(gus, 2), "GBps_graph": round(b / gus / 1e3, 1)}
            ref = (bf16_rates or {}).get(f"{p}_M{M}")
            if ref:
                e["bf16_gemv_us"] = ref["us_median"]
                e["speedup_vs_bf16"] = round(ref["us_median"] / med, 2)
                e["speedup_vs_bf16_graph"] = round(ref["us_graph"] / gus, 2)
            res[f"{p}_M{M}"] = e
        del ws
    return res


def producer_fused_rates(reps=50):
    """Activation quantization with the amax pass folded into the op that
    writes the activation: RMSNorm at the q/k/v and gate/up inputs' shape
    (4096 x 4096) and the SwiGLU gate at the down input's (4096 x 14336).
    For each: the producer with its partial maxima (GB/s over its bytes: 2
    read + 2 written per element for RMSNorm, 4 + 2 for SwiGLU), then the
    quantization of its output by the two-pass quantizer and by the encode
    pass alone from the producer's partials (bit-identical results); for
    RMSNorm also the op fused with the quantization, whose bf16 output never
    goes to HBM (the same codes).  Inputs rotate over copies past the
    Infinity Cache."""
    import torch
    import fp4_block_scaled_elem_amd as mq
    res = {}
    gen = torch.Generator(device="cuda").manual_seed(3000)
    for name, rows, cols in (("rmsnorm_4096x4096", 4096, 4096), ("swiglu_4096x14336", 4096, 14336)):
        swiglu = name.startswith("swiglu")
        per = (2 if swiglu else 1) * rows * cols * 2
        ncopy = max(2, -(-600 * 2 ** 20 // per))
        ins = [torch.randn((rows, cols), generator=gen, device="cuda").to(torch.bfloat16)
               for _ in range(ncopy * (2 if swiglu else 1))]
        g = torch.randn((cols,), generator=gen, device="cuda").to(torch.bfloat16)
        y = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
        q = mq.NVFP4.empty(rows, cols)
        if swiglu:
            prod = lambda r: mq.mq_swiglu_amax(ins[2 * (r % ncopy)], ins[2 * (r % ncopy) + 1], y, q)
        else:
            prod = lambda r: mq.mq_rmsnorm_amax(ins[r % ncopy], g, y, q)
        tp, _ = _median_us(prod, reps=reps)
        t2, _ = _median_us(lambda r: mq.mq_quantize_nvfp4(y, q), reps=reps)
        prod(0)
        t1, _ = _median_us(lambda r: mq.mq_quantize_nvfp4(y, q, mq.MQ_SCALE_PARTIALS), reps=reps)
        nbytes = rows * cols * (6 if swiglu else 4)
        res[name] = {"producer_us": round(tp, 2), "producer_GBps": round(nbytes / tp / 1e3, 1),
                     "quant_two_pass_us": round(t2, 2), "quant_from_partials_us": round(t1, 2),
                     "saved_us": round(t2 - t1, 2)}
        if not swiglu:
            # the RMSNorm fused with quantization (its bf16 output never
            # stored): 2 + 2 + 0.5625 bytes per element over its two passes
            qf = mq.NVFP4.empty(rows, cols)
            tf, _ = _median_us(lambda r: mq.mq_rmsnorm_quantize_nvfp4(ins[r % ncopy], g, qf), reps=reps)
            fbytes = rows * cols * 4.5625
            res[name].update({"fused_to_nvfp4_us": round(tf, 2), "fused_to_nvfp4_GBps": round(fbytes / tf / 1e3, 1),
                              "producer_then_quant_us": round(tp + t1, 2)})
        del ins
    return res


def phase_linear_rates(reps=50):
    """The phase-aware linear (mq_linear_forward) on the 8B q projection's
    weight (4096 x 4096, both formats resident): a decode step at M = 1 and
    32 routes to the BF16 GEMV, a 4096-token prefill to quantize + NVFP4
    GEMM; each timed next to the direct calls it routes to (the dispatch is
    host logic).  Weights rotate over copies past the Infinity Cache for the
    decode rows; the prefill is compute-bound."""
    import torch
    import fp4_block_scaled_elem_amd as mq
    import workloads
    N, K = workloads.LLAMA8B.proj_nk("q")
    gen = torch.Generator(device="cuda").manual_seed(77)
    ncopy = max(2, -(-600 * 2 ** 20 // (2 * N * K)))
    lins = [mq.Linear((torch.randn((N, K), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)).prepare()
            for _ in range(ncopy)]
    res = {}
    for M in (1, 32, 4096):
        x = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        a = mq.NVFP4.empty(M, K)
        path = lins[0].path(M)
        if path == mq.MQ_PATH_DECODE_BF16:
            direct = lambda r: mq.mq_gemv_bf16_decode(x, lins[r % ncopy].w_bf16, y)
        else:
            def direct(r):
                mq.mq_quantize_nvfp4(x, a)
                mq.mq_gemm_nvfp4_prefill(a, None, lins[r % ncopy].w_nvfp4, y)
        med, _ = _median_us(lambda r: lins[r % ncopy].forward(x, out=y, a_work=a), reps=reps)
        dmed, _ = _median_us(direct, reps=reps)
        entry = {"path": "decode_bf16" if path == mq.MQ_PATH_DECODE_BF16 else "prefill_nvfp4",
                 "us_median": round(med, 2), "direct_us_median": round(dmed, 2)}
        if path == mq.MQ_PATH_DECODE_BF16:
            entry["GBps"] = round((2 * N * K + 2 * M * K + 2 * M * N) / med / 1e3, 1)
        else:
            entry["tflops"] = round(2 * M * N * K / med / 1e6, 1)
        res[f"M{M}"] = entry
    del lins
    return res


def layer_prefill(M=4096, reps=20, warm=5):
    """Context: one 8B-shaped decoder layer's prefill over M tokens (one
    causal sequence; 32 query heads and 8 key/value heads of 128, no rotary
    embedding), run twice -- with the method's prefill linears (producer-fused
    quantization: the RMSNorms straight to NVFP4, the SwiGLU gate emitting
    its maxima; NVFP4 GEMMs) and with torch's BF16 linears (hipBLASLt),
    everything else the same torch BF16 ops (attention: torch's
    scaled_dot_product_attention restricted to its flash / memory-efficient
    kernels).  Median layer time of each over `reps` event-timed runs, their
    ratio, the attention's share, and the relative Frobenius difference of
    the two layers' outputs.  Weights random (N(0, 0.02)), input N(0, 1)."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import fp4_block_scaled_elem_amd as mq
    import workloads
    lay = workloads.LLAMA8B
    D, DKV, FF, H, HKV, HD = lay.d_model, lay.d_kv, lay.d_ffn, 32, 8, 128
    gen = torch.Generator(device="cuda").manual_seed(4000)
    rnd = lambda *s, sc=0.02: (torch.randn(s, generator=gen, device="cuda") * sc).to(torch.bfloat16)
    w = {"q": rnd(D, D), "k": rnd(DKV, D), "v": rnd(DKV, D), "o": rnd(D, D), "gate": rnd(FF, D),
         "up": rnd(FF, D), "down": rnd(D, FF)}
    w4 = {p: mq.quantize(t) for p, t in w.items()}
    g1, g2 = rnd(D, sc=1.0), rnd(D, sc=1.0)
    h = rnd(M, D, sc=1.0)
    eps = 1e-5
    buf = {n: torch.empty((M, c), dtype=torch.bfloat16, device="cuda")
           for n, c in (("x1", D), ("q", D), ("k", DKV), ("v", DKV), ("o", D), ("x2", D), ("gate", FF),
                        ("up", FF), ("x3", FF), ("d", D))}
    qa = {n: mq.NVFP4.empty(M, c) for n, c in (("qkv", D), ("o", D), ("gu", D), ("down", FF))}

    def attention(q, k, v):
        qh = q.view(1, M, H, HD).transpose(1, 2).contiguous()
        kh = k.view(1, M, HKV, HD).transpose(1, 2).repeat_interleave(H // HKV, dim=1).contiguous()
        vh = v.view(1, M, HKV, HD).transpose(1, 2).repeat_interleave(H // HKV, dim=1).contiguous()
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            a = F.scaled_dot_product_attention(qh, kh, vh, is_causal=True)
        return a.transpose(1, 2).reshape(M, D).contiguous()

    def nvfp4_layer():
        b = buf
        mq.mq_rmsnorm_quantize_nvfp4(h, g1, qa["qkv"], eps)  # x1 only feeds the linears: never stored
        mq.mq_gemm_nvfp4_prefill(qa["qkv"], None, w4["q"], b["q"])
        mq.mq_gemm_nvfp4_prefill_grouped(qa["qkv"], None, [w4["k"], w4["v"]], [b["k"], b["v"]])
        xo = attention(b["q"], b["k"], b["v"])
        mq.mq_quantize_nvfp4(xo, qa["o"])
        mq.mq_gemm_nvfp4_prefill(qa["o"], None, w4["o"], b["o"])
        h2 = h + b["o"]
        mq.mq_rmsnorm_quantize_nvfp4(h2, g2, qa["gu"], eps)
        mq.mq_gemm_nvfp4_prefill_grouped(qa["gu"], None, [w4["gate"], w4["up"]], [b["gate"], b["up"]])
        mq.mq_swiglu_amax(b["gate"], b["up"], b["x3"], qa["down"])
        mq.mq_quantize_nvfp4(b["x3"], qa["down"], mq.MQ_SCALE_PARTIALS)
        mq.mq_gemm_nvfp4_prefill(qa["down"], None, w4["down"], b["d"])
        return h2 + b["d"]

    def bf16_layer():
        x1 = F.rms_norm(h, (D,), g1, eps)
        xo = attention(F.linear(x1, w["q"]), F.linear(x1, w["k"]), F.linear(x1, w["v"]))
        h2 = h + F.linear(xo, w["o"])
        x2 = F.rms_norm(h2, (D,), g2, eps)
        x3 = F.silu(F.linear(x2, w["gate"])) * F.linear(x2, w["up"])
        return h2 + F.linear(x3, w["down"])

    def attn_only():
        return attention(buf["q"], buf["k"], buf["v"])

    def timed(fn):
        import statistics
        for _ in range(warm):
            fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    t4, t16, ta = timed(nvfp4_layer), timed(bf16_layer), timed(attn_only)
    y4, y16 = nvfp4_layer().float(), bf16_layer().float()
    torch.cuda.synchronize()
    lin_flops = 2 * M * sum(a * b for a, b in (lay.proj_nk(p) for p in ("q", "k", "v", "o", "gate", "up", "down")))
    return {"M": M, "nvfp4_layer_ms": round(t4, 4), "bf16_layer_ms": round(t16, 4),
            "speedup_vs_bf16": round(t16 / t4, 3), "attention_ms": round(ta, 4),
            "linear_tflop": round(lin_flops / 1e12, 3),
            "rel_fro_nvfp4_vs_bf16": round(float(torch.linalg.norm(y4 - y16) / torch.linalg.norm(y16)), 5)}


def bf16_reference(cfg, acts, wdev, iters=10):
    """torch's BF16 GEMM (hipBLASLt) at the same shapes, TFLOP/s."""
    import torch
    import torch.nn.functional as F
    import workloads
    flops = cfg.flops()
    for _ in range(3):
        for p in cfg.projs:
            F.linear(acts[workloads.PROJ_INPUT[p]], wdev[p])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(iters):
        for p in cfg.projs:
            F.linear(acts[workloads.PROJ_INPUT[p]], wdev[p])
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / iters
    return flops / dt / 1e12


def cpu_baseline(cfg_id, acts_host, rows, wrows):
    """The oracle as it stands, on a bounded sample of the same workload:
    the first ``rows`` tokens of each activation (quantized as a tensor of
    their own) times the first ``wrows`` weight rows of every projection
    (weights quantized beforehand, untimed, as on the GPU).  The BLAS
    library that NumPy's float64 matmul calls runs on every host CPU this
    process may use (len(os.sched_getaffinity(0))); NumPy's elementwise
    steps are single-threaded."""
    import numpy as np
    import oracle
    import workloads
    cores = len(os.sched_getaffinity(0))
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas_name = f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:
        blas_name = "unknown"
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
        used = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        limiter, used = None, 1
    cfg = workloads.CONFIGS[cfg_id]
    wq = {}
    for p in cfg.projs:
        wb = workloads.weight(cfg_id, p)
        wq[p] = oracle.quantize_nvfp4(wb[:wrows])
    flops, dt = 0, 0.0
    for a in workloads.ACTS:
        xs = acts_host[a][:rows]
        t0 = time.perf_counter()
        qa = oracle.quantize_nvfp4(xs)
        for p in cfg.projs:
            if workloads.PROJ_INPUT[p] != a:
                continue
            c = oracle.gemm_nvfp4_ref(qa, wq[p])
            flops += 2 * c.shape[0] * c.shape[1] * xs.shape[1]
        dt += time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(used), "kind": "oracle",
            "host_cpus": cores, "blas": blas_name,
            "sample": (f"first {min(rows, cfg.M[0])} tokens of each activation x first {wrows} weight rows of each of "
                       f"{len(cfg.projs)} projections ({flops / 1e9:.1f} GFLOP, {dt:.1f} s; NumPy "
                       f"elementwise steps single-threaded, float64 matmul on {used} {blas_name} threads)")}


GEMM_SRC = os.path.join(ROOT, "fp4_block_scaled_elem_amd", "csrc", "gemm.hip")


def code_digest(path=GEMM_SRC) -> str:
    """sha256[:16] of a source file's code with comments and whitespace
    removed: a comment edit keeps it, any change to the code does not."""
    import hashlib
    import re
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = re.sub(r"\s+", " ", src).strip()
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def gemm_traffic(workload):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    or None when the GEMM's code has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"gemm_traffic_{workload}.json")
    try:
        rec = json.load(open(path))
        h = code_digest()
    except (OSError, ValueError):
        return None
    if rec.get("gemm_code_digest_16") != h:
        return None
    return int(rec["bytes_per_launch"])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is not implemented", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    if args.peak:
        print(json.dumps({"mfma_peak": mfma_peak()}), flush=True)
        return
    if args.layer:
        print(json.dumps({"layer_prefill": layer_prefill()}), flush=True)
        return
    if args.single_linear:
        print(json.dumps({"single_linear_m128": single_linear_latency()}), flush=True)
        return
    if args.decode_only:
        gemv = decode_gemv_rates()
        print(json.dumps({"decode_gemv": gemv, "decode_nvfp4_gemv": decode_nvfp4_rates(gemv),
                          "decode_layer": decode_layer_rates()}), flush=True)
        return
    cfg, acts_host, acts, wdev, qw, qa, fa, out = setup(args.config)
    fused_form = args.fused_form if cfg.fused_act_quant else None
    if fused_form == "panel":
        # the fused launches get A's NVFP4 buffers: the quantize-once form
        fa = {p: qa[workloads.PROJ_INPUT[p]] for p in cfg.projs}
    flops = cfg.flops()
    plan = launch_plan(cfg, args.launches)

    # The MFMA rate measurement runs first: about half a second of full MFMA
    # load, which also brings the chip out of idle clocks before the timed
    # region (a 20-step timed region right after idle reads about 3% below
    # the steady state).  torch's BF16 GEMMs run after the timed region, at
    # the same (warm) state as the NVFP4 step.
    peak = None if args.no_extras else mfma_peak(reps=3)

    for _ in range(args.warmup):
        run_step(cfg, plan, acts, qw, qa, fa, out)
    torch.cuda.synchronize()

    # timed region: exactly K steps between two device synchronisations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(cfg, plan, acts, qw, qa, fa, out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    value = flops / (wall / args.steps) / 1e12

    # kernel timing: the same K steps again with HIP events around every GEMM
    # launch (recorded on the launching stream)
    events = {"g": []}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(cfg, plan, acts, qw, qa, fa, out, events)
    torch.cuda.synchronize()
    ms_step_ev = (time.perf_counter() - t0) / args.steps * 1e3
    gemm_ms = _pairs_ms(events["g"]) / args.steps
    rest_ms = ms_step_ev - gemm_ms
    n_gemm = len(plan)
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12

    launches = per_launch(cfg, plan, acts, qw, qa, fa, out, events, args.steps)
    quant = None if (args.no_extras or cfg.fused_act_quant) else act_quant_rates(acts)
    gemv = None if args.no_extras else decode_gemv_rates()
    gemv_fp4 = None if args.no_extras else decode_nvfp4_rates(gemv)
    dec_layer = None if args.no_extras else decode_layer_rates()
    phase = None if args.no_extras else phase_linear_rates()
    producer = None if (args.no_extras or cfg.fused_act_quant) else producer_fused_rates()
    bf16 = None if args.no_bf16 else bf16_reference(cfg, acts, wdev)
    others = None
    if not args.no_extras and args.config == 2:
        # the other configurations, timed after the headline (device-drawn
        # inputs for the two large ones)
        del acts, wdev, qw, qa, fa, out
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        others = {"single_linear_m128": single_linear_latency(),
                  "longctx_m32768_fused": config_step_rate(3, args.steps, args.warmup),
                  "llama70b_slice_m16384": config_step_rate(5, args.steps, args.warmup),
                  "layer_prefill_m4096": layer_prefill()}
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.config, acts_host, args.cpu_rows, args.cpu_wrows)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "desc": cfg.desc, "M": cfg.M[0],
                   "layer": {"d_model": cfg.layer.d_model, "d_kv": cfg.layer.d_kv, "d_ffn": cfg.layer.d_ffn},
                   "projections": list(cfg.projs), "act_quant": f"fused-{fused_form}" if fused_form else "separate",
                   "launches": ["+".join(g) for _, g in plan],
                   "flop_per_step": flops},
        "pct_mfma_peak": round(100.0 * value / PEAK_F16_MFMA_TFLOPS, 2),
        "roofline": {"bound": "mfma", "kernel": "gemm_panel_kernel" if fused_form == "panel" else "gemm_nvfp4_kernel",
                     "achieved": round(gemm_tflops, 2),
                     "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_F16_MFMA_TFLOPS, 4), "traffic": gemm_traffic(cfg.name),
                     "launches_per_step": n_gemm, "avg_launch_ms": round(gemm_ms / n_gemm, 4),
                     "peak_measured": None if peak is None else {
                         "mfma_only_tflops": peak["valu_per_mfma_0"]["tflops"],
                         "with_dequant_valu_tflops": peak["valu_per_mfma_4"]["tflops"],
                         "clock_mhz": peak["valu_per_mfma_0"]["clock_mhz"],
                         "frac_of_mfma_only": round(gemm_tflops / peak["valu_per_mfma_0"]["tflops"], 4),
                         "frac_of_with_dequant_valu": round(gemm_tflops / peak["valu_per_mfma_4"]["tflops"], 4)}},
        "split_ms": {"gemm": round(gemm_ms, 4), "act_quant_and_gaps": round(rest_ms, 4),
                     "step_with_events": round(ms_step_ev, 4)},
        "per_launch": launches,
        "act_quant": quant,
        "decode_gemv": gemv,
        "decode_nvfp4_gemv": gemv_fp4,
        "decode_layer": dec_layer,
        "phase_linear": phase,
        "producer_fused_act_quant": producer,
        "bf16_torch_tflops": None if bf16 is None else round(bf16, 2),
        "ratio_vs_bf16_torch": None if bf16 is None else round(value / bf16, 3),
        "mfma_peak": peak,
        "other_configs": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
