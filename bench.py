"""Benchmark of the W1.58A8 linear layer on one MI355X.

Headline (`value`): HBM GB/s of the M=1 decode path at the BitNet-2B-4T
projection shapes -- one step = the five projections (qkv 3840x2560,
o_proj 2560x2560, gate_up 13824x2560, down 2560x6912, lm_head 128256x2560) of one
token through bitnet_linear (fused quantise + GEMV), bytes counted as the
algorithmic bytes the method must move (packed weights + weight scales +
activations in + outputs).  Inputs are resident in HBM; the weights rotate
over a pool of >= 1 GiB of distinct copies so the 256 MB last-level cache
cannot hold them.  Steps run as replays of a captured HIP graph.

Beside it: INT8 TOPS of the matrix-core GEMM at M=2048 on the LLaMA-7B shapes
(pre-quantised activations, the GEMM kernel alone, plus the quantise+GEMM
bitnet_linear time), the roofline of the dominant kernel (the lm_head GEMV
launch), and the CPU oracle timed on the host as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Profiling helpers (not part of the timed benchmark):
  python bench.py --pmc-target            eager launches for rocprofv3 --pmc passes: a 256 MiB
                                          device copy (counter calibration), then the lm_head GEMV
  python bench.py --summarize-pmc F W     turn the FETCH_SIZE (F) and WRITE_SIZE (W) rocprofv3 csv
                                          output folders into profiles/gemv_lm_head_m1_traffic.{json,md}
  python bench.py --summarize-trace T     turn a rocprofv3 --kernel-trace --stats csv output folder
                                          into a per-kernel, per-grid table on stdout
  python bench.py --pmc-target-gemm       eager launches for the counter passes over the M=2048 GEMM
  python bench.py --summarize-gemm-pmc A B F W
                                          turn those four passes into profiles/gemm_m2048_counters.md
  python bench.py --gemv-scaling          M=1 bitnet_linear (quantise + GEMV) time against N at K=2560,
                                          and a line fit: fixed cost per launch and marginal stream rate
  python bench.py --pmc-target-small      eager launches for counter passes over the small kernels (M=1 decode
                                          GEMV on qkv / o_proj, small-batch GEMM at M=16 / 64)
  python bench.py --summarize-small-pmc W F R
                                          turn those three passes into profiles/small_kernels_counters.md
  python bench.py --machine               machine ceilings only (int8 MFMA loop, HBM read and copy)
"""
import argparse
import csv
import gzip
import glob
import hashlib
import json
import math
import os
import platform
import subprocess
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import ternary_int8_gemm_amd as tg  # noqa: E402

METRIC = "W1.58A8 GEMV HBM GB/s (M=1) + GEMM INT8 TOPS (M=2048), % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published (5.0 POPS)
POOL_BYTES = 1 << 30           # rotating weight pool, >= 4x the 256 MB last-level cache
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_lm_head_m1_traffic.json")
CALIB_COPY_BYTES = 256 << 20   # plain device copy used to scale the rocprofv3 byte counters
KERNEL_SOURCES = ["ternary_int8_gemm_amd/csrc/gemv.hip", "ternary_int8_gemm_amd/csrc/bitnet_device.h"]


def gemv_bytes(M, N, K):
    """Algorithmic bytes of the fused path: packed W + bf16 scale_wt + bf16 x in + bf16 out."""
    return N * K // 4 + 2 * N + 2 * M * K + 2 * M * N


def gemm_bytes(M, N, K):
    """Algorithmic bytes of the GEMM: packed W + scale_wt + int8 x + scale_act + bf16 out."""
    return N * K // 4 + 2 * N + M * K + 2 * M + 2 * M * N


def dev_bf16(bits, device):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


SPIN_CYCLES = 200_000   # a short spin kernel ahead of each timed region (tens of microseconds)


def time_launches(launch, stream):
    """GPU seconds of the work that `launch()` enqueues on `stream`, from events
    recorded on `stream` around it, after a device-wide synchronisation and
    followed by one.  A short spin kernel goes first, so that the GPU is still
    busy while the host enqueues the work: the start event then marks when the
    work can begin, not the host's launch latency."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
        start.record(stream)
        launch()
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3


def time_graph(graph, replays, stream):
    """Replay `graph` `replays` times on `stream` and time the replays (time_launches)."""
    def launch():
        for _ in range(replays):
            graph.replay()   # launches on the current stream, i.e. `stream`
    return time_launches(launch, stream)


MIN_REPEATS = 50        # timed repeats of a measurement ...
MIN_TIMED_S = 0.1       # ... and at least this much timed GPU time
MAX_REPEATS = 400


def repeat_timing(launch, stream, units, min_repeats=MIN_REPEATS, min_seconds=MIN_TIMED_S, max_repeats=MAX_REPEATS):
    """Time `launch()` (which does `units` units of work) over repeats: at least
    min_repeats of them, or as many as give min_seconds of timed work, whichever
    is more (at most max_repeats).  Returns the seconds per unit of each repeat."""
    out, total = [], 0.0
    while len(out) < max_repeats and (len(out) < min_repeats or total < min_seconds):
        t = time_launches(launch, stream)
        total += t
        out.append(t / units)
    return out


def pstats(per_unit_s, scale=1e6):
    """Median, 10th and 90th percentile (linear interpolation) of per-unit seconds, times `scale`."""
    a = np.asarray(per_unit_s, dtype=np.float64) * scale
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "n": int(a.size)}


RAMP_SECONDS = 0.03


def ramp(graph, stream, seconds=RAMP_SECONDS):
    """Untimed replays of `graph` until `seconds` of GPU time have passed (returns
    the time spent).  The GPU's clocks take several milliseconds of sustained
    work to settle (about 10 ms measured on MI355X after an idle gap), so a
    warm-up of one or two short replays would leave the timed replays inside
    that ramp."""
    spent, n = 0.0, 1
    while spent < seconds:
        spent += time_graph(graph, n, stream)
        n = min(2 * n, 1024)
    return spent


MIN_GRAPH_LAUNCHES = 64  # launches per timed graph: a replay of a short graph adds microseconds of its own


def launches_graph(launch, n, stream, min_launches=MIN_GRAPH_LAUNCHES):
    """A captured graph of L launches, launch(i % n) for i < L, with L the
    smallest multiple of n that is >= min_launches; returns (graph, L).  Each
    replay of a captured graph costs some microseconds of its own on the GPU
    (measured: about 11 us per replay of a graph of four 2 us kernels), so a
    timed graph holds enough launches for that cost to vanish in the average."""
    L = n * max(1, math.ceil(min_launches / n))
    return capture(lambda: [launch(i % n) for i in range(L)], stream), L


def capture(fn, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn()  # warm once outside capture (first-touch of the library, lazy init)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    return g


# ----------------------------------------------------------------------------- decode GEMV

def build_decode(device, log):
    """Weights, pools and outputs for the five M=1 projections."""
    shapes = synth.BITNET_2B_DECODE
    host = {}
    per_set = 0
    for i, (name, N, K) in enumerate(shapes):
        W = synth.ternary_weights(N, K, synth.seed_for(1, 16 * i + synth.T_WEIGHT))
        P = tg.pack_weights(torch.from_numpy(W)).numpy()
        sw = synth.weight_scale_bf16(N, K, synth.seed_for(1, 16 * i + synth.T_SCALE))
        x = synth.activations_bf16(1, K, synth.seed_for(1, 16 * i + synth.T_ACT))
        host[name] = (W, P, sw, x)
        per_set += P.nbytes
        del W
    copies = max(2, -(-POOL_BYTES // per_set))
    log(f"decode: weight set {per_set / 1e6:.1f} MB, {copies} rotating copies ({copies * per_set / 1e9:.2f} GB)")
    dev_sets = []
    for r in range(copies):
        d = {}
        for name, N, K in shapes:
            W, P, sw, x = host[name]
            Pd = torch.from_numpy(P).to(device) if r == 0 else dev_sets[0][name][0].clone()
            d[name] = (Pd, dev_bf16(sw, device), dev_bf16(x, device),
                       torch.empty((1, N), dtype=torch.bfloat16, device=device))
        dev_sets.append(d)
    return shapes, host, dev_sets


WINDOW_GRAPH_MAX_NODES = 60000   # kernel nodes over all the window graphs of the headline


def step_plan(start, n, copies):
    """Graph replays that run exactly n decode steps from step index `start`:
    step i uses weight copy i % copies; None stands for the graph of a whole
    rotation (copies 0 .. copies-1), an integer c for the one-step graph of copy
    c.  Returns (replays, the next step index)."""
    plan, i, left = [], start, n
    while left > 0:
        if i % copies == 0 and left >= copies:
            plan.append(None)
            i, left = i + copies, left - copies
        else:
            plan.append(i % copies)
            i, left = i + 1, left - 1
    return plan, i


def run_decode(shapes, dev_sets, steps, warmup, stream, log):
    """The headline.  One step is the five projections of one token on one copy
    of the weights; consecutive steps use consecutive copies, so no step finds
    its weights in a cache.  After a clock ramp (untimed replays, reported),
    exactly `warmup` steps run untimed, then exactly `steps` steps are timed,
    and that timed window is repeated (each repeat on the next copies, timed on
    its own) to give the median, 10th and 90th percentile; the reported step
    time is the median window's."""
    copies = len(dev_sets)

    def one_step(d):
        for name, N, K in shapes:
            Pd, swd, xd, od = d[name]
            tg.bitnet_linear(xd, Pd, swd, out=od)

    step_graphs = [capture(lambda d=d: one_step(d), stream) for d in dev_sets]
    rotation = capture(lambda: [one_step(d) for d in dev_sets], stream)
    cursor = [0]  # index of the next step's weight copy

    def run_steps(n):
        plan, cursor[0] = step_plan(cursor[0], n, copies)
        for c in plan:
            (rotation if c is None else step_graphs[c]).replay()

    # The timed window is one graph of exactly `steps` steps (one per starting
    # copy it is used at), so that no boundary between graph launches falls
    # inside it; very long windows replay the rotation graphs instead, where
    # such boundaries are one in `copies` steps.
    starts = copies // math.gcd(steps, copies)
    windows = {}
    whole_graph = 5 * steps * starts <= WINDOW_GRAPH_MAX_NODES

    if whole_graph:  # captured before the ramp: the timed windows start at steps warmup + r * steps
        for r in range(starts):
            o = (warmup + r * steps) % copies
            if o not in windows:
                windows[o] = capture(lambda o=o: [one_step(dev_sets[(o + j) % copies]) for j in range(steps)], stream)

    def run_window():
        if whole_graph:
            windows[cursor[0] % copies].replay()
            cursor[0] += steps
        else:
            run_steps(steps)

    t_ramp = ramp(rotation, stream)
    with torch.cuda.stream(stream):
        run_steps(warmup)
    torch.cuda.synchronize()
    window = time_launches(run_window, stream)
    reps = max(11, min(MAX_REPEATS, math.ceil(MIN_TIMED_S / window)))
    per_step = [window / steps] + repeat_timing(run_window, stream, steps, min_repeats=reps - 1, min_seconds=0.0)
    st = pstats(per_step, 1e3)
    step_bytes = sum(gemv_bytes(1, N, K) for _, N, K in shapes)
    ms = st["median"]
    result = {"steps": steps, "warmup": warmup, "ms_per_step": ms, "gbs": step_bytes / (ms * 1e-3) / 1e9,
              "step_bytes": step_bytes,
              "timing": {"repeats_of_steps": st["n"],
                         "window": ("one captured graph of the timed steps" if whole_graph else
                                    "replays of whole-rotation graphs and one-step graphs"),
                         "ms_per_step_median": round(st["median"], 6),
                         "ms_per_step_p10": round(st["p10"], 6), "ms_per_step_p90": round(st["p90"], 6),
                         "ms_per_step_first_repeat": round(per_step[0] * 1e3, 6),
                         "clock_ramp_ms": round(t_ramp * 1e3, 2), "weight_copies": copies}}

    # Per-projection launch durations: a graph of back-to-back launches of one
    # shape over the rotating copies, timed with events around its replays.
    per_shape = {}
    for name, N, K in shapes:
        def launch(i, name=name):
            Pd, swd, xd, od = dev_sets[i][name]
            tg.bitnet_linear(xd, Pd, swd, out=od)
        gs, L = launches_graph(launch, copies, stream)
        ramp(gs, stream)
        r = 2
        st = pstats(repeat_timing(lambda gs=gs: [gs.replay() for _ in range(r)], stream, r * L))
        us = st["median"]
        per_shape[name] = {"N": N, "K": K, "us": us, "us_p10": st["p10"], "us_p90": st["p90"], "repeats": st["n"],
                           "gbs": gemv_bytes(1, N, K) / (us * 1e-6) / 1e9, "bytes": gemv_bytes(1, N, K)}
        log(f"  {name:8s} N={N:6d} K={K:5d}: {us:8.2f} us (p10 {st['p10']:.2f}, p90 {st['p90']:.2f})  "
            f"{per_shape[name]['gbs']:8.1f} GB/s")
    result["per_shape"] = per_shape
    return result


# ----------------------------------------------------------------------------- prefill GEMM

def run_gemm(device, stream, M, log, rotate=4):
    out = {}
    for i, (name, N, K) in enumerate(synth.LLAMA7B_SHAPES):
        W = synth.ternary_weights(N, K, synth.seed_for(3, 16 * i + synth.T_WEIGHT))
        P = tg.pack_weights(torch.from_numpy(W))
        del W
        sw = dev_bf16(synth.weight_scale_bf16(N, K, synth.seed_for(3, 16 * i + synth.T_SCALE)), device)
        x = dev_bf16(synth.activations_bf16(M, K, synth.seed_for(3, 16 * i + synth.T_ACT), outlier_frac=0.01), device)
        Ps = [P.to(device)] + [None] * (rotate - 1)
        for r in range(1, rotate):
            Ps[r] = Ps[0].clone()
        q, sa = tg.quantize_activation(x)
        o = torch.empty((M, N), dtype=torch.bfloat16, device=device)
        ws = torch.empty((tg.linear_workspace_bytes(M, K),), dtype=torch.uint8, device=device)

        def gemm_only(i):
            tg.bitnet_gemm(q, Ps[i], sa, sw, out=o)

        def linear_full(i):
            tg.bitnet_linear(x, Ps[i], sw, out=o, workspace=ws)

        def quant_only(i):
            tg.quantize_activation(x, out=q, scale=sa)

        res = {"N": N, "K": K}
        for tag, fn, least in (("gemm", gemm_only, 16), ("linear", linear_full, 16), ("quant", quant_only, 64)):
            g, L = launches_graph(fn, rotate, stream, least)
            ramp(g, stream)
            st = pstats(repeat_timing(g.replay, stream, L, min_repeats=30))
            res[tag + "_us"] = st["median"]
            res[tag + "_us_p10"], res[tag + "_us_p90"], res[tag + "_repeats"] = st["p10"], st["p90"], st["n"]
        ops = 2.0 * M * N * K
        res["tops"] = ops / (res["gemm_us"] * 1e-6) / 1e12
        res["linear_tops"] = ops / (res["linear_us"] * 1e-6) / 1e12
        res["frac_int8_peak"] = res["tops"] / INT8_PEAK_TOPS
        out[name] = res
        log(f"  M={M} {name:8s} N={N:6d} K={K:5d}: gemm {res['gemm_us']:8.1f} us (p10 {res['gemm_us_p10']:.1f}, "
            f"p90 {res['gemm_us_p90']:.1f}) {res['tops']:7.1f} TOPS ({100 * res['frac_int8_peak']:.1f}% of peak); "
            f"quant {res['quant_us']:.1f} us; linear {res['linear_us']:.1f} us")
        del Ps, q, sa, o, ws, x
        torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- small-batch GEMM

SMALL_M = (8, 16, 32, 64, 128, 256)


def roofline_frac(ops, nbytes, seconds):
    """Fraction of min(INT8 peak, arithmetic intensity x HBM peak) achieved."""
    bound_tops = min(INT8_PEAK_TOPS, ops / nbytes * HBM_PEAK_GBS / 1e3)
    return ops / seconds / 1e12 / bound_tops


def run_small_batch(device, stream, log):
    """bitnet_gemm at M = 8..256 on the LLaMA-7B layer shapes (pre-quantised
    activations), weights rotating over >= 1 GiB of copies."""
    out = {}
    for i, (name, N, K) in enumerate(synth.LLAMA7B_SHAPES[:3]):
        W = synth.ternary_weights(N, K, synth.seed_for(2, 16 * i + synth.T_WEIGHT))
        P = tg.pack_weights(torch.from_numpy(W)).to(device)
        del W
        copies = max(2, -(-POOL_BYTES // P.numel()))
        Ps = [P] + [P.clone() for _ in range(copies - 1)]
        sw = dev_bf16(synth.row_scales_bf16(N, synth.seed_for(2, 16 * i + synth.T_ROWSCALE)), device)
        for M in SMALL_M:
            x = dev_bf16(synth.activations_bf16(M, K, synth.seed_for(2, 16 * i + synth.T_ACT) + M), device)
            q, sa = tg.quantize_activation(x)
            o = torch.empty((M, N), dtype=torch.bfloat16, device=device)

            g, L = launches_graph(lambda i: tg.bitnet_gemm(q, Ps[i], sa, sw, out=o), copies, stream)
            ramp(g, stream)
            st = pstats(repeat_timing(g.replay, stream, L, min_repeats=15))
            t = st["median"] * 1e-6
            ops, nbytes = 2.0 * M * N * K, gemm_bytes(M, N, K)
            r = {"us": round(t * 1e6, 2), "us_p10": round(st["p10"], 2), "us_p90": round(st["p90"], 2),
                 "gbs": round(nbytes / t / 1e9, 1), "tops": round(ops / t / 1e12, 1),
                 "frac_roofline": round(roofline_frac(ops, nbytes, t), 4)}
            out[f"{name}_M{M}"] = r
            log(f"  {name:8s} M={M:4d}: {r['us']:8.2f} us {r['gbs']:8.1f} GB/s {r['tops']:8.1f} TOPS "
                f"({100 * r['frac_roofline']:.1f}% of roofline)")
        del Ps
        torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- full decode step

def run_decode_full(device, stream, log, layers=30):
    """One token through every BitLinear of a 30-layer BitNet-2B-4T (4 fused
    projections per layer) plus the LM head: 121 calls on 121 distinct weight
    buffers (603 MB).  The layers hold copies of one synthetic layer's packed
    weights (distinct memory, same values).  M = 1 (fused GEMV) and M = 16
    (quantise + GEMM), each step captured as one graph; then the same with the
    RMSNorm that precedes every BitLinear fused in (bitnet_linear_rms: the
    decode GEMV's prologue at M = 1, RMSNorm-quantise + GEMM at M = 16)."""
    shapes = synth.BITNET_2B_DECODE
    layer_shapes = [s for s in shapes if s[0] != "lm_head"]
    head = [s for s in shapes if s[0] == "lm_head"]
    base = {}
    for i, (name, N, K) in enumerate(shapes):
        W = synth.ternary_weights(N, K, synth.seed_for(1, 16 * i + synth.T_WEIGHT))
        base[name] = (tg.pack_weights(torch.from_numpy(W)).to(device),
                      dev_bf16(synth.weight_scale_bf16(N, K, synth.seed_for(1, 16 * i + synth.T_SCALE)), device))
        del W
    calls = []
    for _ in range(layers):
        for name, N, K in layer_shapes:
            calls.append((name, N, K, base[name][0].clone(), base[name][1]))
    for name, N, K in head:
        calls.append((name, N, K, base[name][0], base[name][1]))
    total_w = sum(c[3].numel() for c in calls)
    res = {"calls": len(calls), "weight_bytes": total_w}
    for M, rms in ((1, False), (16, False), (1, True), (16, True)):
        xs, outs = [], []
        for j, (name, N, K, _, _) in enumerate(calls):
            xs.append(dev_bf16(synth.activations_bf16(M, K, synth.seed_for(5, j) + M), device))
            outs.append(torch.empty((M, N), dtype=torch.bfloat16, device=device))
        ws = torch.empty((max(tg.linear_rms_workspace_bytes(M, c[2]) for c in calls) + 256,), dtype=torch.uint8,
                         device=device)

        def step():
            for (name, N, K, Pd, swd), xd, od in zip(calls, xs, outs):
                if rms:
                    tg.bitnet_linear_rms(xd, Pd, swd, out=od, workspace=ws)
                else:
                    tg.bitnet_linear(xd, Pd, swd, out=od, workspace=ws)

        g = capture(step, stream)
        ramp(g, stream)
        st = pstats(repeat_timing(g.replay, stream, 1, min_repeats=50))
        t = st["median"] * 1e-6
        if M == 1:
            nbytes = sum(gemv_bytes(M, N, K) for _, N, K, _, _ in calls)
        else:  # quantise (2MK in, MK + 2M out) + GEMM
            nbytes = sum(gemm_bytes(M, N, K) + 3 * M * K + 2 * M for _, N, K, _, _ in calls)
        key = f"M{M}_rmsnorm" if rms else f"M{M}"
        res[key] = {"us_per_step": round(t * 1e6, 2), "us_p10": round(st["p10"], 2), "us_p90": round(st["p90"], 2),
                    "tokens_per_s": round(M / t, 1),
                    "gbs": round(nbytes / t / 1e9, 1), "frac_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                    "step_bytes": nbytes}
        log(f"  full decode step M={M:2d}{' +RMSNorm' if rms else '         '}: {t * 1e6:8.1f} us/step, {M / t:9.1f} tok/s, "
            f"{nbytes / t / 1e9:7.1f} GB/s ({100 * nbytes / t / 1e9 / HBM_PEAK_GBS:.1f}% of HBM peak)")
        del xs, outs, ws
    del calls, base
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- f32 input and bias

def run_options(device, stream, log):
    """bitnet_linear_ex at the decode shapes (M = 1) and at M = 2048 on the
    LLaMA-7B qkvo shape: f32 activations (quantise + GEMM) and bf16
    activations with a bias, beside the plain bf16 call."""
    out = {}
    cases = [(name, N, K, 1) for name, N, K in synth.BITNET_2B_DECODE] + [("llama_qkvo", 4096, 4096, 2048)]
    for i, (name, N, K, M) in enumerate(cases):
        W = synth.ternary_weights(N, K, synth.seed_for(6, 16 * i + synth.T_WEIGHT))
        P = tg.pack_weights(torch.from_numpy(W)).to(device)
        del W
        copies = max(2, -(-POOL_BYTES // P.numel()))
        Ps = [P] + [P.clone() for _ in range(copies - 1)]
        sw = dev_bf16(synth.weight_scale_bf16(N, K, synth.seed_for(6, 16 * i + synth.T_SCALE)), device)
        bias = dev_bf16(synth.row_scales_bf16(N, synth.seed_for(6, 16 * i + synth.T_ROWSCALE)), device)
        xb = dev_bf16(synth.activations_bf16(M, K, synth.seed_for(6, 16 * i + synth.T_ACT)), device)
        xf = xb.float()
        o = torch.empty((M, N), dtype=torch.bfloat16, device=device)
        ws = torch.empty((tg.linear_ex_workspace_bytes(M, K, torch.float32) + 256,), dtype=torch.uint8, device=device)
        r = {"M": M, "N": N, "K": K}
        for tag, x, b in (("bf16", xb, None), ("bf16_bias", xb, bias), ("f32", xf, None)):
            g, L = launches_graph(lambda i, x=x, b=b: tg.bitnet_linear(x, Ps[i], sw, out=o, workspace=ws, bias=b),
                                  copies, stream)
            ramp(g, stream)
            r[tag + "_us"] = round(pstats(repeat_timing(g.replay, stream, L, min_repeats=15))["median"], 2)
        out[f"{name}_M{M}"] = r
        log(f"  {name:10s} M={M:5d} N={N:6d} K={K:5d}: bf16 {r['bf16_us']:8.2f} us, +bias {r['bf16_bias_us']:8.2f} us, "
            f"f32 input {r['f32_us']:8.2f} us")
        del Ps, xb, xf, o, ws
        torch.cuda.empty_cache()
    return out


FUSED_M = (1, 2, 4, 5, 8, 12, 15)


def run_fused_small_m(device, stream, log):
    """bitnet_gemv_fused (quantise + product in one launch, without a workspace)
    against the split path (bitnet_quantize_act, then bitnet_gemm) at
    M = 1 ... 15 on the BitNet-2B-4T decode shapes, and bitnet_linear, which
    takes whichever of the two its dispatch rule picks; weights rotate through
    a 1 GiB pool.  Times are medians of graph-timed launches in microseconds."""
    out = {}
    for i, (name, N, K) in enumerate(synth.BITNET_2B_DECODE):
        W = synth.ternary_weights(N, K, synth.seed_for(8, 16 * i + synth.T_WEIGHT))
        P = tg.pack_weights(torch.from_numpy(W)).to(device)
        del W
        copies = max(2, -(-POOL_BYTES // P.numel()))
        Ps = [P] + [P.clone() for _ in range(copies - 1)]
        sw = dev_bf16(synth.weight_scale_bf16(N, K, synth.seed_for(8, 16 * i + synth.T_SCALE)), device)
        rows = {}
        for M in FUSED_M:
            x = dev_bf16(synth.activations_bf16(M, K, synth.seed_for(8, 16 * i + synth.T_ACT) + M), device)
            o = torch.empty((M, N), dtype=torch.bfloat16, device=device)
            q = torch.empty((M, K), dtype=torch.int8, device=device)
            sa = torch.empty((M,), dtype=torch.bfloat16, device=device)
            ws = torch.empty((max(tg.linear_workspace_bytes(M, K), 256),), dtype=torch.uint8, device=device)
            r = {}
            for tag, fn in (("fused_us", lambda j: tg.bitnet_gemv_fused(x, Ps[j], sw, out=o)),
                            ("split_us", lambda j: (tg.quantize_activation(x, out=q, scale=sa),
                                                    tg.bitnet_gemm(q, Ps[j], sa, sw, out=o))),
                            ("linear_us", lambda j: tg.bitnet_linear(x, Ps[j], sw, out=o, workspace=ws))):
                g, L = launches_graph(fn, copies, stream)
                ramp(g, stream)
                r[tag] = round(pstats(repeat_timing(g.replay, stream, L, min_repeats=10))["median"], 2)
                del g
            r["fused_over_split"] = round(r["fused_us"] / r["split_us"], 3)
            rows[M] = r
            del x, o, q, sa, ws
        out[name] = {"N": N, "K": K, "by_M": rows}
        log(f"  {name:8s} N={N:6d} K={K:5d}: " + " | ".join(
            f"M={M} {r['fused_us']:.2f}/{r['split_us']:.2f}/{r['linear_us']:.2f}" for M, r in rows.items()))
        del Ps, P
        torch.cuda.empty_cache()
    return out


def w8a16_bytes(M, N, K):
    """Algorithmic bytes of the INT8 weight-only matmul: int8 W + fp32 scale + bf16 x + fp32 y."""
    return N * K + 4 * N + 2 * M * K + 4 * M * N


def run_w8a16(device, stream, log):
    """bitnet_w8a16_gemv (int8 weights, bf16 activations) at the BitNet-2B-4T and
    LLaMA-7B decode shapes, M = 1 and 16, weights rotated through a 1 GiB pool."""
    out = {}
    cases = [("bitnet_" + n, N, K) for n, N, K in synth.BITNET_2B_DECODE] + \
            [("llama_" + n, N, K) for n, N, K in synth.LLAMA7B_SHAPES]
    for i, (name, N, K) in enumerate(cases):
        q = torch.from_numpy(synth.random_int8((N, K), synth.seed_for(7, 16 * i + synth.T_WEIGHT))).to(device)
        copies = max(2, -(-POOL_BYTES // q.numel()))
        qs = [q] + [q.clone() for _ in range(copies - 1)]
        sc = torch.full((N,), 1.0 / 127.0, dtype=torch.float32, device=device)
        r = {"N": N, "K": K}
        for M in (1, 16):
            x = dev_bf16(synth.activations_bf16(M, K, synth.seed_for(7, 16 * i + synth.T_ACT) + M), device)
            y = torch.empty((M, N), dtype=torch.float32, device=device)

            g, L = launches_graph(lambda i, x=x, y=y: tg.w8a16_gemv(x, qs[i], sc, out=y), copies, stream, 16)
            ramp(g, stream)
            t = pstats(repeat_timing(g.replay, stream, L, min_repeats=15))["median"] * 1e-6
            r[f"M{M}_us"] = round(t * 1e6, 2)
            r[f"M{M}_gbs"] = round(w8a16_bytes(M, N, K) / t / 1e9, 1)
        out[name] = r
        log(f"  {name:16s} N={N:6d} K={K:5d}: M=1 {r['M1_us']:8.2f} us {r['M1_gbs']:7.1f} GB/s, "
            f"M=16 {r['M16_us']:8.2f} us {r['M16_gbs']:7.1f} GB/s")
        del qs, q
        torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- CPU oracle

def host_facts():
    """What the CPU baseline ran on: logical CPUs (nproc), the CPUs this process
    may use, and the CPU model."""
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def run_cpu_baseline(host, shapes, budget_s, log):
    """The oracle on the host cores over a bounded sample of the headline
    workload (whole M=1 decode steps of the five projections): first on one
    thread (about a third of the budget, at least one step), then on every
    thread OpenMP gives it (the rest).  The value is the multi-threaded rate."""
    import oracle  # the oracle is only ever used here, for the CPU baseline leg
    packed = {name: oracle.pack(host[name][0]) for name, _, _ in shapes}
    step_bytes = sum(gemv_bytes(1, N, K) for _, N, K in shapes)
    threads_all = oracle.num_threads()

    def timed_steps(threads, seconds):
        oracle.set_num_threads(threads)
        t0 = time.perf_counter()
        n = 0
        while True:
            for name, N, K in shapes:
                _, _, sw, x = host[name]
                oracle.linear(x, packed[name], sw)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds or n >= 1000:
                return n, el

    n1, el1 = timed_steps(1, budget_s / 3)
    nm, elm = timed_steps(threads_all, budget_s - el1)
    oracle.set_num_threads(threads_all)
    gbs1, gbsm = step_bytes * n1 / el1 / 1e9, step_bytes * nm / elm / 1e9
    facts = host_facts()
    log(f"cpu oracle: 1 thread {n1} steps in {el1:.1f} s -> {gbs1:.3f} GB/s; {threads_all} threads {nm} steps in "
        f"{elm:.1f} s -> {gbsm:.3f} GB/s ({facts['cpu_model']}, nproc {facts['nproc']})")
    return {"value": gbsm, "unit": "GB/s", "cores": threads_all, "kind": "oracle",
            "sample": f"{nm} full M=1 decode steps (all five BitNet-2B-4T projections) on {threads_all} threads, "
                      f"{elm:.1f} s; before that {n1} steps on one thread, {el1:.1f} s",
            "ms_per_step": elm / nm * 1e3,
            "single_thread": {"value": gbs1, "unit": "GB/s", "ms_per_step": el1 / n1 * 1e3, "steps": n1},
            **facts}


def gpu_clock_info():
    """Clocks as the SMI tool reports them right now (a child process; null when
    neither amd-smi nor rocm-smi answers)."""
    for cmd in (["amd-smi", "metric", "--clock", "--json"], ["rocm-smi", "--showclocks", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
        except (OSError, subprocess.SubprocessError):
            continue
        if r.returncode != 0 or not r.stdout.strip():
            continue
        try:
            return {"tool": cmd[0], "report": json.loads(r.stdout)}
        except ValueError:
            return {"tool": cmd[0], "text": r.stdout.strip()[:2000]}
    return None


# ----------------------------------------------------------------------------- machine ceilings

PROBE_LIB = os.path.join(ROOT, "ternary_int8_gemm_amd", "libbitnet_probe.so")


def load_probe():
    """libbitnet_probe.so (built beside the layer's library): read, copy and
    int8-MFMA loops that measure this box's practical ceilings."""
    import ctypes
    lib = ctypes.CDLL(PROBE_LIB)
    p, i64, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.probe_read.argtypes = [p, i64, p, i, p]
    lib.probe_copy.argtypes = [p, p, i64, i, p]
    lib.probe_mfma_i8.argtypes = [p, i, p, i, p]
    lib.probe_gemm_loop.argtypes = [p, i, p, i, p]
    for fn in (lib.probe_read, lib.probe_copy, lib.probe_mfma_i8, lib.probe_gemm_loop):
        fn.restype = i
    return lib


def run_vendor_int8_gemm(device, stream, log, M=2048, N=4096, K=4096):
    """torch._int_mm (hipBLASLt's int8 x int8 -> int32 GEMM) at the qkvo prefill
    shape, on the workload's quantised activations and the ternary weights
    unpacked to int8 [K][N] (column-major, as a weight matrix is stored):
    a reference point for what a dense int8 library GEMM reaches on this GPU
    and data.  Launched eagerly (library calls stay out of captured graphs)."""
    try:
        x = dev_bf16(synth.activations_bf16(M, K, synth.seed_for(3, synth.T_ACT), outlier_frac=0.01), device)
        q, _ = tg.quantize_activation(x)
        W = torch.from_numpy(synth.ternary_weights(N, K, synth.seed_for(3, synth.T_WEIGHT))).to(device)
        Wt = W.t()  # [K][N] view of the row-major [N][K] weights
        with torch.cuda.stream(stream):
            torch._int_mm(q, Wt)
        torch.cuda.synchronize()

        def launch():
            for _ in range(16):
                torch._int_mm(q, Wt)
        for _ in range(3):
            time_launches(launch, stream)
        st = pstats(repeat_timing(launch, stream, 16, min_repeats=10))
        tops = 2.0 * M * N * K / (st["median"] * 1e-6) / 1e12
        res = {"shape": [M, N, K], "us": round(st["median"], 2), "tops": round(tops, 1),
               "frac_of_published": round(tops / INT8_PEAK_TOPS, 4)}
        log(f"  vendor int8 GEMM (torch._int_mm) {M}x{N}x{K}: {res['us']:.2f} us, {res['tops']:.1f} TOPS "
            f"({100 * res['frac_of_published']:.1f}% of 5.0 POPS)")
        return res
    except (RuntimeError, NotImplementedError) as e:
        log(f"  vendor int8 GEMM unavailable: {e}")
        return {"shape": [M, N, K], "error": str(e)[:200]}


def run_machine(device, stream, log):
    """Practical ceilings of this GPU, measured with the probe kernels:
    the int8 MFMA rate of back-to-back v_mfma_i32_32x32x32_i8 (2 waves per SIMD),
    with the shader clock it ran at; the same for the GEMM's inner loop alone
    (LDS fragments, weight expansion, MFMAs; 128 x 64 wave tiles, 2 waves per
    SIMD) on operand data distributed like the prefill workload's, which
    changes every MFMA and draws more power; the vendor int8 GEMM
    (torch._int_mm, hipBLASLt) at the M = 2048 qkvo shape with unpacked int8
    weights; the HBM read rate over 1 GiB and over 82 MB pieces of a 1 GiB pool
    (the LM head's weight size); the copy rate over 512 MiB.  Each is the median
    of repeated, ramped timings."""
    import ctypes
    lib = load_probe()
    sp = ctypes.c_void_p(stream.cuda_stream)
    res = {}

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with status {rc}")

    blocks, iters = 512, 20000
    out = torch.empty((blocks * 256,), dtype=torch.int32, device=device)
    clk = torch.zeros((2,), dtype=torch.int64, device=device)

    def mfma():
        check(lib.probe_mfma_i8(ctypes.c_void_p(out.data_ptr()), iters, ctypes.c_void_p(clk.data_ptr()), blocks, sp),
              "probe_mfma_i8")
    g = capture(mfma, stream)
    ramp(g, stream)
    st = pstats(repeat_timing(g.replay, stream, 1, min_repeats=20), 1.0)
    ops = blocks * 4 * 4 * iters * 65536.0
    ticks, real = (int(v) for v in clk.cpu())
    res["mfma_i8"] = {"tops": round(ops / st["median"] / 1e12, 1), "tops_p10_time": round(ops / st["p90"] / 1e12, 1),
                      "tops_p90_time": round(ops / st["p10"] / 1e12, 1),
                      "frac_of_published": round(ops / st["median"] / 1e12 / INT8_PEAK_TOPS, 4),
                      "sclk_mhz": round(ticks / real * 100.0, 1) if real > 0 else None,
                      "kernel_ms": round(st["median"] * 1e3, 3), "waves_per_simd": 2}
    log(f"  int8 MFMA loop: {res['mfma_i8']['tops']:.1f} TOPS ({100 * res['mfma_i8']['frac_of_published']:.1f}% of "
        f"5.0 POPS), shader clock {res['mfma_i8']['sclk_mhz']} MHz")
    del g

    gl_iters = 2000

    def gemm_loop():
        check(lib.probe_gemm_loop(ctypes.c_void_p(out.data_ptr()), gl_iters, ctypes.c_void_p(clk.data_ptr()), blocks,
                                  sp), "probe_gemm_loop")
    g = capture(gemm_loop, stream)
    ramp(g, stream)
    st = pstats(repeat_timing(g.replay, stream, 1, min_repeats=20), 1.0)
    ops = blocks * 4 * gl_iters * 32 * 65536.0
    ticks, real = (int(v) for v in clk.cpu())
    res["gemm_loop_i8"] = {"tops": round(ops / st["median"] / 1e12, 1),
                           "frac_of_published": round(ops / st["median"] / 1e12 / INT8_PEAK_TOPS, 4),
                           "sclk_mhz": round(ticks / real * 100.0, 1) if real > 0 else None,
                           "kernel_ms": round(st["median"] * 1e3, 3), "waves_per_simd": 2,
                           "operands": "activation codes bell-shaped in -22..23 (sd about 8), ternary weight codes "
                                       "P(0)=0.4, changing every MFMA"}
    log(f"  GEMM inner loop on workload-like data: {res['gemm_loop_i8']['tops']:.1f} TOPS "
        f"({100 * res['gemm_loop_i8']['frac_of_published']:.1f}% of 5.0 POPS), shader clock "
        f"{res['gemm_loop_i8']['sclk_mhz']} MHz")
    del g, out
    res["vendor_int8_gemm"] = run_vendor_int8_gemm(device, stream, log)

    pool = torch.empty((1 << 30,), dtype=torch.uint8, device=device)
    pool.fill_(3)
    sink = torch.empty((2048 * 256,), dtype=torch.int32, device=device)

    def read(lo, n):
        check(lib.probe_read(ctypes.c_void_p(pool.data_ptr() + lo), n, ctypes.c_void_p(sink.data_ptr()), 2048, sp),
              "probe_read")
    g = capture(lambda: [read(0, 1 << 30) for _ in range(8)], stream)
    ramp(g, stream)
    st = pstats(repeat_timing(g.replay, stream, 8, min_repeats=20), 1.0)
    res["read_1GiB"] = {"tbs": round((1 << 30) / st["median"] / 1e12, 3), "us": round(st["median"] * 1e6, 1)}
    piece = 82_080_768  # the LM head's packed weights, 128256 x 640 bytes
    npieces = (1 << 30) // piece
    g = capture(lambda: [read(i * piece, piece) for _ in range(4) for i in range(npieces)], stream)
    ramp(g, stream)
    st = pstats(repeat_timing(g.replay, stream, 4 * npieces, min_repeats=20), 1.0)
    res["read_82MB"] = {"tbs": round(piece / st["median"] / 1e12, 3), "us": round(st["median"] * 1e6, 2),
                        "us_p10": round(st["p10"] * 1e6, 2), "us_p90": round(st["p90"] * 1e6, 2),
                        "workgroups": 2048}

    def read256(lo, n):
        check(lib.probe_read(ctypes.c_void_p(pool.data_ptr() + lo), n, ctypes.c_void_p(sink.data_ptr()), 256, sp),
              "probe_read")
    g = capture(lambda: [read256(i * piece, piece) for _ in range(4) for i in range(npieces)], stream)
    ramp(g, stream)
    st = pstats(repeat_timing(g.replay, stream, 4 * npieces, min_repeats=20), 1.0)
    res["read_82MB_256wg"] = {"tbs": round(piece / st["median"] / 1e12, 3), "us": round(st["median"] * 1e6, 2),
                              "workgroups": 256}
    half = 1 << 29

    def copy():
        check(lib.probe_copy(ctypes.c_void_p(pool.data_ptr() + half), ctypes.c_void_p(pool.data_ptr()), half, 2048, sp),
              "probe_copy")
    g = capture(lambda: [copy() for _ in range(8)], stream)
    ramp(g, stream)
    st = pstats(repeat_timing(g.replay, stream, 8, min_repeats=20), 1.0)
    res["copy_512MiB"] = {"tbs_read_plus_write": round(2 * half / st["median"] / 1e12, 3),
                          "us": round(st["median"] * 1e6, 1)}
    log(f"  HBM read 1 GiB {res['read_1GiB']['tbs']:.2f} TB/s; 82 MB pieces {res['read_82MB']['tbs']:.2f} TB/s "
        f"({res['read_82MB']['us']:.2f} us; {res['read_82MB_256wg']['us']:.2f} us with 256 workgroups); "
        f"copy 512 MiB {res['copy_512MiB']['tbs_read_plus_write']:.2f} TB/s")
    del g, pool, sink
    torch.cuda.empty_cache()
    return res


def load_traffic(lm_head_launch_bytes):
    """HBM traffic of the dominant kernel from the committed rocprofv3 counter runs,
    or None if absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


# ----------------------------------------------------------------------------- profiling helpers

def lm_head_inputs(device, copies):
    """The lm_head projection of the decode step (same seeds as the timed run), with `copies` weight copies."""
    i, (name, N, K) = next((i, s) for i, s in enumerate(synth.BITNET_2B_DECODE) if s[0] == "lm_head")
    W = synth.ternary_weights(N, K, synth.seed_for(1, 16 * i + synth.T_WEIGHT))
    P = tg.pack_weights(torch.from_numpy(W)).to(device)
    del W
    Ps = [P] + [P.clone() for _ in range(copies - 1)]
    sw = dev_bf16(synth.weight_scale_bf16(N, K, synth.seed_for(1, 16 * i + synth.T_SCALE)), device)
    x = dev_bf16(synth.activations_bf16(1, K, synth.seed_for(1, 16 * i + synth.T_ACT)), device)
    return N, K, Ps, sw, x


GEMV_SCALING_N = (4008, 8016, 16032, 32064, 64128, 128256, 256512, 513024)
GEMV_SCALING_FIT_MIN_N = 32064


def scaling_fit(rows):
    """Least-squares line time_us = fixed + MB / rate over the (N, MB, seconds)
    rows with N >= GEMV_SCALING_FIT_MIN_N; returns (fixed_us, rate_TBs)."""
    fit = [(mb, t * 1e6) for N, mb, t in rows if N >= GEMV_SCALING_FIT_MIN_N]
    A = np.array([[1.0, mb] for mb, _ in fit])
    c = np.linalg.lstsq(A, np.array([t for _, t in fit]), rcond=None)[0]
    return float(c[0]), float(1.0 / c[1])


def run_gemv_scaling(device, stream):
    """bitnet_linear at M=1, K=2560 for the N in GEMV_SCALING_N: the lm_head weight
    rows repeated to N rows, enough copies to cycle through about 1 GiB (none stays
    in the caches), one graph of back-to-back launches per N, the best of three
    ramped timings.  A least-squares line over N >= GEMV_SCALING_FIT_MIN_N
    (scaling_fit) splits the time into a fixed cost per launch and the marginal
    streaming rate."""
    # the floor of a dependent launch in a graph: one-element kernels back to back
    one = torch.zeros(1, device=device)

    def tiny():
        for _ in range(200):
            one.add_(1.0)
    g = capture(tiny, stream)
    floor = float("inf")
    for _ in range(3):
        ramp(g, stream)
        floor = min(floor, time_graph(g, 5, stream) / (5 * 200))
    print(f"launch floor: {floor * 1e6:.2f} us per one-element kernel in a graph", flush=True)
    del g

    N0, K, Ps0, sw0, x = lm_head_inputs(device, 1)
    P0 = Ps0[0]
    rows = []
    for N in GEMV_SCALING_N:
        P = torch.cat([P0] * (-(-N // N0)))[:N].contiguous()
        Ps = [P] + [P.clone() for _ in range(max(2, (1 << 30) // P.numel()) - 1)]
        sw = torch.cat([sw0] * (-(-N // N0)))[:N].contiguous()
        out = torch.empty((1, N), dtype=torch.bfloat16, device=device)

        def launches():
            for Q in Ps:
                tg.bitnet_linear(x, Q, sw, out=out)
        g = capture(launches, stream)
        best = float("inf")
        for _ in range(3):
            ramp(g, stream)
            best = min(best, time_graph(g, 5, stream) / (5 * len(Ps)))
        mb = N * K / 4 / 1e6
        rows.append((N, mb, best))
        print(f"N={N:7d}  weights {mb:8.2f} MB  {best * 1e6:8.2f} us  {mb / best / 1e6:5.2f} TB/s  "
              f"({len(Ps)} copies)", flush=True)
        del Ps, P, g
        torch.cuda.empty_cache()
    fixed_us, rate = scaling_fit(rows)
    print(json.dumps({"gemv_scaling": [{"N": N, "MB": round(mb, 2), "us": round(t * 1e6, 2)} for N, mb, t in rows],
                      "fit_fixed_us": round(fixed_us, 2), "fit_marginal_TBs": round(rate, 2),
                      "launch_floor_us": round(floor * 1e6, 2)}))


def run_pmc_target(device, reps=3):
    """Eager launches for hardware-counter passes (counter collection serialises
    dispatches, so no graph): a plain device-to-device copy of CALIB_COPY_BYTES,
    then the lm_head GEMV over four weight copies (328 MB, more than the 256 MB
    last-level cache)."""
    a = torch.full((CALIB_COPY_BYTES,), 7, dtype=torch.uint8, device=device)
    b = torch.empty_like(a)
    N, K, Ps, sw, x = lm_head_inputs(device, 4)
    out = torch.empty((1, N), dtype=torch.bfloat16, device=device)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        for P in Ps:
            tg.bitnet_linear(x, P, sw, out=out)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_target": "done", "copy_bytes": CALIB_COPY_BYTES, "gemv_launches": reps * len(Ps),
                      "N": N, "K": K}), flush=True)


def _csv_rows(folder, suffix):
    """Rows of every *suffix (or gzip-compressed *suffix.gz) file under folder."""
    rows = []
    paths = glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True) + \
        glob.glob(os.path.join(folder, "**", "*" + suffix + ".gz"), recursive=True)
    for path in sorted(paths):
        opener = gzip.open if path.endswith(".gz") else open
        with opener(path, "rt", newline="") as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no *{suffix} under {folder}")
    return rows


def _col(row, *names):
    low = {k.lower(): k for k in row}
    for n in names:
        if n.lower() in low:
            return row[low[n.lower()]]
    raise KeyError(f"none of {names} in {sorted(row)}")


def _grid(row):
    try:
        return int(_col(row, "Grid_Size", "Grid_Size_X"))
    except KeyError:
        return -1


TRACE_ARGS = "--steps 22 --warmup 5 --no-cpu-baseline --no-extra --no-machine"


def summarize_trace(folder, bench_args=TRACE_ARGS):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of this script
    (with bench_args): the --stats table as rocprofv3 wrote it, then the trace
    split by launch grid (one template instance serves several shapes)."""
    extra = "" if bench_args == TRACE_ARGS else f' --trace-args="{bench_args}"'
    out = [f"# rocprofv3 kernel trace of `bench.py {bench_args}`", "",
           "Command (from the repository root, after `cd /tmp && export TMPDIR=/tmp`):", "",
           f"    rocprofv3 --kernel-trace --stats --output-format csv -d {folder} -o bench -- "
           f"python3 bench.py {bench_args}",
           f"    gzip {folder}/*kernel_trace.csv   # the per-dispatch trace, compressed for transfer",
           f"    python bench.py --summarize-trace {folder}{extra}", "",
           "## --stats (kernel_stats.csv)", "",
           "| kernel | calls | total ms | avg us | min us | max us | % |", "|---|---:|---:|---:|---:|---:|---:|"]
    for r in _csv_rows(folder, "kernel_stats.csv"):
        out.append(f"| `{_col(r, 'Name')[:100]}` | {_col(r, 'Calls')} | {float(_col(r, 'TotalDurationNs')) / 1e6:.3f} | "
                   f"{float(_col(r, 'AverageNs')) / 1e3:.3f} | {float(_col(r, 'MinNs')) / 1e3:.3f} | "
                   f"{float(_col(r, 'MaxNs')) / 1e3:.3f} | {float(_col(r, 'Percentage')):.2f} |")
    stats = {}
    for r in _csv_rows(folder, "kernel_trace.csv"):
        name = _col(r, "Kernel_Name")
        dur = int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))
        stats.setdefault((name, _grid(r)), []).append(dur)
    out += ["", "## Per launch grid (kernel_trace.csv)", "",
            "| kernel | grid (threads) | calls | avg us | min us | max us |", "|---|---|---:|---:|---:|---:|"]
    for (name, grid), d in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| `{name[:100]}` | {grid} | {len(d)} | {sum(d) / len(d) / 1e3:.3f} | "
                   f"{min(d) / 1e3:.3f} | {max(d) / 1e3:.3f} |")
    print("\n".join(out))


def summarize_pmc(fetch_dir, write_dir):
    """HBM bytes per lm_head GEMV launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the plain copy of
    CALIB_COPY_BYTES."""
    def per_dispatch(folder, counter):
        rows = []
        for r in _csv_rows(folder, "counter_collection.csv"):
            if _col(r, "Counter_Name") == counter:
                rows.append((_col(r, "Kernel_Name"), _grid(r), float(_col(r, "Counter_Value"))))
        return rows

    res = {}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = per_dispatch(folder, counter)
        # The calibration copy is the largest device copy of the run (the weight
        # clones are smaller copies with the same kernel and grid).
        copies = [v for n, g, v in rows if "copyBuffer" in n]
        gemv = [(g, v) for n, g, v in rows if "gemv_stream_kernel" in n]
        if not copies or not gemv:
            raise SystemExit(f"{counter}: copy or GEMV dispatches missing in {folder}")
        big = [v for v in copies if v >= 0.9 * max(copies)]
        copy_kib = sum(big) / len(big)
        factor = CALIB_COPY_BYTES / (copy_kib * 1024.0)
        grid = max(g for g, _ in gemv)
        vals = [v for g, v in gemv if g == grid]
        gemv_kib = sum(vals) / len(vals)
        res[counter] = {"copy_kib": copy_kib, "copy_dispatches": len(big), "factor": factor, "gemv_kib": gemv_kib,
                        "gemv_dispatches": len(vals), "grid": grid, "gemv_bytes": gemv_kib * 1024.0 * factor}
    N, K = next((N, K) for n, N, K in synth.BITNET_2B_DECODE if n == "lm_head")
    algo = gemv_bytes(1, N, K)
    total = res["FETCH_SIZE"]["gemv_bytes"] + res["WRITE_SIZE"]["gemv_bytes"]
    out = {"kernel": "gemv_stream_kernel (lm_head 128256x2560, M=1)", "kernel_source_sha256_16": kernel_source_hash(),
           "bytes_per_launch": round(total), "algorithmic_bytes_per_launch": algo,
           "traffic_over_algorithmic": round(total / algo, 4), "counters": res,
           "commands": [
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o run -- python3 bench.py --pmc-target",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o run -- python3 bench.py --pmc-target",
               "python bench.py --summarize-pmc gpurun_out/pmc_fetch gpurun_out/pmc_write"]}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    md = [f"# HBM traffic of the lm_head GEMV launch (M=1, N={N}, K={K})", "",
          "Commands (each counter in its own pass, run from the repository root after `cd /tmp && export TMPDIR=/tmp`):", ""]
    md += ["    " + c for c in out["commands"]]
    md += ["", "| counter | copy of 256 MiB reads (KiB) | scale factor | GEMV launch (KiB) | GEMV bytes (scaled) |",
           "|---|---:|---:|---:|---:|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        r = res[c]
        md.append(f"| {c} | {r['copy_kib']:.1f} | {r['factor']:.4f} | {r['gemv_kib']:.1f} | {r['gemv_bytes']:.0f} |")
    md += ["", f"Traffic per launch: {total:.0f} B; algorithmic bytes per launch: {algo} B "
           f"(packed weights N*K/4 + bf16 weight scales + bf16 x + bf16 out); ratio {total / algo:.4f}.",
           f"Kernel source hash (gemv.hip + bitnet_device.h): {out['kernel_source_sha256_16']}."]
    with open(TRAFFIC_FILE[:-5] + ".md", "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(out))


GEMM_PMC_FILE = os.path.join(ROOT, "profiles", "gemm_m2048_counters.md")
GEMM_PMC_PASSES = {  # pass name -> counters (each pass a run of its own)
    "a": "SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_VALU_MFMA_COEXEC_CYCLES",
    "b": "SQ_WAIT_INST_ANY SQ_WAVE_CYCLES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS SQ_BUSY_CYCLES",
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
}
# LLaMA-7B shapes the counter passes cover, in launch order: qkvo takes one round
# of eight-wave 128 x 256 blocks, gate_up 1.34 rounds of two four-wave blocks per CU
GEMM_PMC_SHAPES = ("qkvo", "gate_up")
GEMM_PMC_M = 2048
GEMM_PMC_WARM, GEMM_PMC_REPS = 300, 20


def run_pmc_target_gemm(device):
    """Eager launches for counter passes over the prefill GEMM: a plain copy of
    CALIB_COPY_BYTES (byte-counter calibration), then, for each shape of
    GEMM_PMC_SHAPES in turn, GEMM_PMC_WARM + GEMM_PMC_REPS launches of
    bitnet_gemm at M = GEMM_PMC_M (pre-quantised activations); the summary keeps
    the last GEMM_PMC_REPS of each shape, when the clocks have settled."""
    a = torch.full((CALIB_COPY_BYTES,), 7, dtype=torch.uint8, device=device)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    M = GEMM_PMC_M
    for shape in GEMM_PMC_SHAPES:
        i, (name, N, K) = next((i, sh) for i, sh in enumerate(synth.LLAMA7B_SHAPES) if sh[0] == shape)
        P = tg.pack_weights(torch.from_numpy(synth.ternary_weights(N, K, synth.seed_for(3, 16 * i + synth.T_WEIGHT))))
        P = P.to(device)
        sw = dev_bf16(synth.weight_scale_bf16(N, K, synth.seed_for(3, 16 * i + synth.T_SCALE)), device)
        x = dev_bf16(synth.activations_bf16(M, K, synth.seed_for(3, 16 * i + synth.T_ACT), outlier_frac=0.01), device)
        q, sa = tg.quantize_activation(x)
        o = torch.empty((M, N), dtype=torch.bfloat16, device=device)
        torch.cuda.synchronize()
        for _ in range(GEMM_PMC_WARM + GEMM_PMC_REPS):
            tg.bitnet_gemm(q, P, sa, sw, out=o)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_target_gemm": name, "M": M, "N": N, "K": K,
                          "launches": GEMM_PMC_WARM + GEMM_PMC_REPS}), flush=True)
        del P, sw, x, q, sa, o


def _gemm_block(kernel_name):
    """(block rows, block columns, waves) from a gemm_mfma_kernel<BM, BN, WM, WN, ...> name."""
    m = re.search(r"gemm_mfma_kernel<\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+)", kernel_name)
    if not m:
        return None
    bm, bn, wm, wn = (int(g) for g in m.groups())
    return bm, bn, wm * wn


def summarize_gemm_pmc(dirs):
    """Markdown summary of the four counter passes of run_pmc_target_gemm (the
    directories in GEMM_PMC_PASSES order): per shape, per-launch averages over the
    last GEMM_PMC_REPS of its GEMM dispatches (the dispatches of a pass, in
    order, fall into len(GEMM_PMC_SHAPES) equal runs)."""
    ns = len(GEMM_PMC_SHAPES)
    vals = [{} for _ in range(ns)]
    durs = [[] for _ in range(ns)]
    knames = [set() for _ in range(ns)]
    calib = {}
    for (pname, counters), folder in zip(GEMM_PMC_PASSES.items(), dirs):
        rows = _csv_rows(folder, "counter_collection.csv")
        gemm_ids = sorted({int(_col(r, "Dispatch_Id")) for r in rows if "gemm_mfma_kernel" in _col(r, "Kernel_Name")})
        if len(gemm_ids) % ns != 0 or len(gemm_ids) // ns < GEMM_PMC_REPS:
            raise SystemExit(f"pass {pname}: {len(gemm_ids)} GEMM dispatches in {folder}, "
                             f"expected {ns} runs of at least {GEMM_PMC_REPS}")
        per = len(gemm_ids) // ns
        which = {}
        for s in range(ns):
            for did in gemm_ids[(s + 1) * per - GEMM_PMC_REPS:(s + 1) * per]:
                which[did] = s
        seen_dur = set()
        for r in rows:
            did = int(_col(r, "Dispatch_Id"))
            cname = _col(r, "Counter_Name")
            v = float(_col(r, "Counter_Value"))
            if did in which:
                s = which[did]
                vals[s].setdefault(cname, []).append(v)
                m = re.search(r"gemm_mfma_kernel<[^>]*>", _col(r, "Kernel_Name"))
                knames[s].add(m.group(0) if m else _col(r, "Kernel_Name"))
                if pname == "a" and did not in seen_dur:
                    seen_dur.add(did)
                    durs[s].append(float(_col(r, "End_Timestamp")) - float(_col(r, "Start_Timestamp")))
            elif "copyBuffer" in _col(r, "Kernel_Name") and cname in ("FETCH_SIZE", "WRITE_SIZE"):
                calib.setdefault(cname, []).append(v)
    factor = {c: CALIB_COPY_BYTES / (1024.0 * max(v)) for c, v in calib.items()}
    M = GEMM_PMC_M
    simds, clk = 256 * 4, 2.4e9
    cmds = [f"timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_gemm_{p} -o run -- "
            "python3 bench.py --pmc-target-gemm" for p, c in GEMM_PMC_PASSES.items()]
    cmds.append("python bench.py --summarize-gemm-pmc " + " ".join(f"gpurun_out/pmc_gemm_{p}" for p in GEMM_PMC_PASSES))
    shapes = [next(sh for sh in synth.LLAMA7B_SHAPES if sh[0] == s) for s in GEMM_PMC_SHAPES]
    md = [f"# Counters of the prefill GEMM (bitnet_gemm, LLaMA-7B shapes, M={M})", "",
          "Commands (each pass a run of its own, from the repository root after `cd /tmp && export TMPDIR=/tmp`):", ""]
    md += ["    " + c for c in cmds]
    md += ["", f"Per-launch averages over the last {GEMM_PMC_REPS} of {GEMM_PMC_WARM + GEMM_PMC_REPS} eager launches "
           "of each shape.", "",
           "| quantity | " + " | ".join(f"{n} ({N}×{K})" for n, N, K in shapes) + " |",
           "|---|" + "---:|" * ns]
    cols = {k: [] for k in ("kernel", "grid", "dur", "mfma", "busy", "frac", "valu", "coexec", "lds", "conf", "wait",
                            "waitlds", "hbm")}
    for s, (name, N, K) in enumerate(shapes):
        avg = {k: sum(v) / len(v) for k, v in vals[s].items()}
        dur_ns = sum(durs[s]) / len(durs[s])
        busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"]
        kn = ", ".join(f"`{k}`" for k in sorted(knames[s]))
        blk = _gemm_block(next(iter(sorted(knames[s]))))
        fetch_b = avg["FETCH_SIZE"] * 1024.0 * factor["FETCH_SIZE"]
        write_b = avg["WRITE_SIZE"] * 1024.0 * factor["WRITE_SIZE"]
        algo = gemm_bytes(M, N, K)
        cols["kernel"].append(kn)
        cols["grid"].append(f"{-(-M // blk[0]) * -(-N // blk[1])} of {blk[2]} waves" if blk else "?")
        cols["dur"].append(f"{dur_ns / 1e3:.2f} µs")
        cols["mfma"].append(f"{avg['SQ_INSTS_MFMA']:.0f} (2MNK / 65536 = {2 * M * N * K // 65536})")
        cols["busy"].append(f"{busy:.4g} ({busy / avg['SQ_INSTS_MFMA']:.1f} per MFMA)")
        cols["frac"].append(f"{busy / (dur_ns * 1e-9 * clk * simds):.3f}")
        cols["valu"].append(f"{avg['SQ_INSTS_VALU'] / avg['SQ_INSTS_MFMA']:.2f}")
        cols["coexec"].append(f"{avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / busy:.3f}")
        cols["lds"].append(f"{avg['SQ_INSTS_LDS'] / avg['SQ_INSTS_MFMA']:.2f}")
        cols["conf"].append(f"{avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_INSTS_LDS']:.2f}")
        cols["wait"].append(f"{avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.3f}")
        cols["waitlds"].append(f"{avg['SQ_WAIT_INST_LDS'] / avg['SQ_WAVE_CYCLES']:.3f}")
        cols["hbm"].append(f"{fetch_b + write_b:.4g} ({(fetch_b + write_b) / algo:.2f} × the {algo} algorithmic bytes)")
    labels = [("kernel", "kernel"), ("grid", "workgroups"), ("dur", "dispatch duration (profiled)"),
              ("mfma", "SQ_INSTS_MFMA"), ("busy", "SQ_VALU_MFMA_BUSY_CYCLES"),
              ("frac", f"MFMA busy / (duration × 2.4 GHz × {simds} SIMDs)"), ("valu", "VALU instructions per MFMA"),
              ("coexec", "MFMA cycles with VALU co-issued (COEXEC / MFMA busy)"),
              ("lds", "LDS instructions per MFMA"), ("conf", "LDS bank-conflict cycles per LDS instruction"),
              ("wait", "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES"), ("waitlds", "SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES"),
              ("hbm", f"HBM bytes (FETCH_SIZE × {factor['FETCH_SIZE']:.3f} + WRITE_SIZE × "
                      f"{factor['WRITE_SIZE']:.3f})")]
    md += [f"| {label} | " + " | ".join(cols[k]) + " |" for k, label in labels]
    md += ["", "The byte counters are scaled by what they read for a plain device copy of 256 MiB in the same run.",
           "The MFMA peak used for the fraction is the dense int8 rate at 2.4 GHz: 1024 SIMDs × 32768 MACs per",
           "32 cycles = 5.0 POPS."]
    with open(GEMM_PMC_FILE, "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


SMALL_PMC_FILE = os.path.join(ROOT, "profiles", "small_kernels_counters.md")
SMALL_PMC_PASSES = {  # pass name -> counters (each pass a run of its own)
    "waits": "SQ_WAIT_INST_ANY SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAVES GRBM_GUI_ACTIVE",
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
}
SMALL_PMC_WARM, SMALL_PMC_REPS = 100, 20


def small_pmc_cases():
    """(tag, kind, M, N, K, seed index) of the small-kernel counter passes: the M=1
    decode GEMV on the BitNet-2B-4T qkv and o_proj projections, and the
    small-batch GEMM (pre-quantised activations) at M=16 and 64 on the LLaMA-7B
    qkvo and gate_up shapes."""
    cases = [("gemv qkv M=1", "gemv", 1, 3840, 2560, 0), ("gemv o_proj M=1", "gemv", 1, 2560, 2560, 1)]
    for j, (name, N, K) in enumerate(synth.LLAMA7B_SHAPES[:2]):
        for M in (16, 64):
            cases.append((f"gemm {name} M={M}", "gemm", M, N, K, j))
    return cases


def run_pmc_target_small(device):
    """Eager launches for counter passes over the small kernels: the calibration
    copy, then for each case of small_pmc_cases SMALL_PMC_WARM + SMALL_PMC_REPS
    launches over 16 weight copies (the summary keeps the last SMALL_PMC_REPS)."""
    a = torch.full((CALIB_COPY_BYTES,), 7, dtype=torch.uint8, device=device)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    for tag, kind, M, N, K, j in small_pmc_cases():
        W = synth.ternary_weights(N, K, synth.seed_for(8, 16 * j + synth.T_WEIGHT))
        P = tg.pack_weights(torch.from_numpy(W)).to(device)
        del W
        Ps = [P] + [P.clone() for _ in range(15)]
        sw = dev_bf16(synth.weight_scale_bf16(N, K, synth.seed_for(8, 16 * j + synth.T_SCALE)), device)
        x = dev_bf16(synth.activations_bf16(M, K, synth.seed_for(8, 16 * j + synth.T_ACT)), device)
        o = torch.empty((M, N), dtype=torch.bfloat16, device=device)
        q, sa = tg.quantize_activation(x)
        torch.cuda.synchronize()
        for i in range(SMALL_PMC_WARM + SMALL_PMC_REPS):
            if kind == "gemv":
                tg.bitnet_linear(x, Ps[i % 16], sw, out=o)
            else:
                tg.bitnet_gemm(q, Ps[i % 16], sa, sw, out=o)
        torch.cuda.synchronize()
        del Ps, P
    print(json.dumps({"pmc_target_small": "done", "cases": [c[0] for c in small_pmc_cases()]}), flush=True)


def summarize_small_pmc(dirs):
    """Markdown summary of the counter passes of run_pmc_target_small (directories
    in SMALL_PMC_PASSES order): per case, per-dispatch averages over its last
    SMALL_PMC_REPS dispatches; byte counters scaled by the calibration copy."""
    per = {}   # case index -> counter -> values
    dur = {}
    calib = {}
    for (pname, counters), folder in zip(SMALL_PMC_PASSES.items(), dirs):
        rows = _csv_rows(folder, "counter_collection.csv")
        disp = {}
        for r in rows:
            name = _col(r, "Kernel_Name")
            did = int(_col(r, "Dispatch_Id"))
            cname = _col(r, "Counter_Name")
            v = float(_col(r, "Counter_Value"))
            if "copyBuffer" in name:
                if cname in ("FETCH_SIZE", "WRITE_SIZE"):
                    calib.setdefault(cname, []).append(v)
                continue
            if "gemv_stream_kernel" in name or "gemm_" in name:
                d = disp.setdefault(did, {"name": name, "vals": {}, "dur": float(_col(r, "End_Timestamp")) -
                                          float(_col(r, "Start_Timestamp"))})
                d["vals"][cname] = d["vals"].get(cname, 0.0) + v
        ids = sorted(disp)
        n_case = len(small_pmc_cases())
        per_case = SMALL_PMC_WARM + SMALL_PMC_REPS
        if len(ids) < n_case * per_case:
            raise SystemExit(f"pass {pname}: {len(ids)} layer dispatches in {folder}, expected {n_case * per_case}")
        ids = ids[-n_case * per_case:]
        for c in range(n_case):
            keep = ids[c * per_case + SMALL_PMC_WARM:(c + 1) * per_case]
            for did in keep:
                for cname, v in disp[did]["vals"].items():
                    per.setdefault(c, {}).setdefault(cname, []).append(v)
                if pname == "waits":
                    dur.setdefault(c, []).append(disp[did]["dur"])
                per[c].setdefault("_name", []).append(disp[did]["name"])
    factor = {cn: CALIB_COPY_BYTES / (1024.0 * max(v)) for cn, v in calib.items()}
    cmds = [f"timeout -s KILL 90 rocprofv3 --pmc {cs} --output-format csv -d gpurun_out/pmc_small_{p} -o run -- "
            "python3 bench.py --pmc-target-small" for p, cs in SMALL_PMC_PASSES.items()]
    cmds.append("python bench.py --summarize-small-pmc " + " ".join(f"gpurun_out/pmc_small_{p}" for p in SMALL_PMC_PASSES))
    md = ["# Counters of the small kernels (decode GEMV at M=1, small-batch GEMM at M=16 and 64)", "",
          "Commands (each pass a run of its own, from the repository root after `cd /tmp && export TMPDIR=/tmp`):", ""]
    md += ["    " + c for c in cmds]
    md += ["", f"Per-dispatch averages over the last {SMALL_PMC_REPS} of {SMALL_PMC_WARM + SMALL_PMC_REPS} eager launches "
           "of each case (16 weight copies in rotation). HBM bytes are FETCH_SIZE and WRITE_SIZE scaled by what they "
           f"read for a plain copy of {CALIB_COPY_BYTES >> 20} MiB in the same run "
           f"(factors {factor.get('FETCH_SIZE', float('nan')):.3f} and {factor.get('WRITE_SIZE', float('nan')):.3f}). "
           "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES is the fraction of the waves' lifetime spent waiting to issue "
           "(on memory, LDS or barriers).", "",
           "| case | kernel | dispatch µs (profiled) | HBM bytes | algorithmic bytes | ratio | HBM GB/s | wait / wave cycles | waves |",
           "|---|---|---:|---:|---:|---:|---:|---:|---:|"]
    for c, (tag, kind, M, N, K, j) in enumerate(small_pmc_cases()):
        a = {k: sum(v) / len(v) for k, v in per[c].items() if k != "_name"}
        name = per[c]["_name"][-1]
        m = re.search(r"(gemv_stream_kernel|gemm_\w+?kernel)<[^>]*>", name)
        kname = m.group(0) if m else name[:60]
        hbm = a.get("FETCH_SIZE", 0.0) * 1024 * factor.get("FETCH_SIZE", 1.0) + \
            a.get("WRITE_SIZE", 0.0) * 1024 * factor.get("WRITE_SIZE", 1.0)
        algo = gemv_bytes(M, N, K) if kind == "gemv" else gemm_bytes(M, N, K)
        d_us = sum(dur[c]) / len(dur[c]) / 1e3
        md.append(f"| {tag} | `{kname}` | {d_us:.2f} | {hbm:.4g} | {algo} | {hbm / algo:.3f} | "
                  f"{hbm / (d_us * 1e-6) / 1e9:.0f} | {a['SQ_WAIT_INST_ANY'] / a['SQ_WAVE_CYCLES']:.3f} | "
                  f"{a.get('SQ_WAVES', 0):.0f} |")
    with open(SMALL_PMC_FILE, "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2200)
    ap.add_argument("--warmup", type=int, default=220)
    ap.add_argument("--gemm-m", type=int, nargs="+", default=[2048, 4096])
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the small-batch GEMM and full decode-step lines")
    ap.add_argument("--no-machine", action="store_true", help="skip the machine-ceiling probes")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--machine", action="store_true", help="only the machine-ceiling probes (MFMA loop, read, copy)")
    ap.add_argument("--pmc-target", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR")
    ap.add_argument("--trace-args", default=TRACE_ARGS, help="the bench.py arguments of the traced run")
    ap.add_argument("--pmc-target-gemm", action="store_true")
    ap.add_argument("--summarize-gemm-pmc", nargs=4, metavar=("A_DIR", "B_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--gemv-scaling", action="store_true")
    ap.add_argument("--pmc-target-small", action="store_true")
    ap.add_argument("--summarize-small-pmc", nargs=3, metavar=("WAITS_DIR", "FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.trace_args)
        return
    if args.summarize_gemm_pmc:
        summarize_gemm_pmc(args.summarize_gemm_pmc)
        return
    if args.summarize_small_pmc:
        summarize_small_pmc(args.summarize_small_pmc)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    def log(msg):
        if not args.quiet:
            print(msg, file=sys.stderr, flush=True)

    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    tg.load_library()
    if args.pmc_target:
        run_pmc_target(device)
        return
    if args.pmc_target_gemm:
        run_pmc_target_gemm(device)
        return
    if args.pmc_target_small:
        run_pmc_target_small(device)
        return
    stream = torch.cuda.Stream(device)
    if args.gemv_scaling:
        run_gemv_scaling(device, stream)
        return
    if args.machine:
        print(json.dumps({"machine_ceilings": run_machine(device, stream, log)}), flush=True)
        return

    clock_before = gpu_clock_info()
    shapes, host, dev_sets = build_decode(device, log)
    log(f"decode GEMV M=1 (BitNet-2B-4T shapes), {args.steps} timed steps after {args.warmup} warm-up steps:")
    dec = run_decode(shapes, dev_sets, args.steps, args.warmup, stream, log)
    tm = dec["timing"]
    log(f"decode step: {dec['ms_per_step'] * 1e3:.2f} us/step (median of {tm['repeats_of_steps']} windows of "
        f"{args.steps} steps; p10 {tm['ms_per_step_p10'] * 1e3:.2f}, p90 {tm['ms_per_step_p90'] * 1e3:.2f}), "
        f"{dec['gbs']:.1f} GB/s ({100 * dec['gbs'] / HBM_PEAK_GBS:.1f}% of HBM peak)")
    del dev_sets
    torch.cuda.empty_cache()
    clock_after = gpu_clock_info()

    gemms = {}
    if not args.no_gemm:
        for M in args.gemm_m:
            log(f"prefill GEMM M={M} (LLaMA-7B shapes):")
            gemms[M] = run_gemm(device, stream, M, log)

    small = full = options = w8 = machine = fused_m = None
    if not args.no_extra:
        log("small-batch GEMM M=8..256 (LLaMA-7B layer shapes, pre-quantised):")
        small = run_small_batch(device, stream, log)
        log("full BitNet-2B-4T decode step (30 layers x 4 + lm_head = 121 calls):")
        full = run_decode_full(device, stream, log)
        log("bitnet_linear options (f32 activations, bias):")
        options = run_options(device, stream, log)
        log("fused quantise + product (bitnet_gemv_fused) / quantise then GEMM / bitnet_linear, us, M = 1..15:")
        fused_m = run_fused_small_m(device, stream, log)
        log("INT8 weight-only matmul (W8A16), decode shapes:")
        w8 = run_w8a16(device, stream, log)
    if not args.no_machine:
        log("machine ceilings (probe kernels):")
        machine = run_machine(device, stream, log)

    lm = dec["per_shape"]["lm_head"]
    traffic = load_traffic(lm["bytes"])
    roofline = {"bound": "hbm", "achieved": round(lm["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(lm["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "gemv_stream_kernel (lm_head 128256x2560, M=1)",
                "bytes_per_launch": lm["bytes"], "avg_launch_us": round(lm["us"], 3),
                "launch_us_p10": round(lm["us_p10"], 3), "launch_us_p90": round(lm["us_p90"], 3),
                "launch_time": f"median over {lm['repeats']} repeats of back-to-back graph launches, HIP events on the "
                               "launch stream"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(host, shapes, args.cpu_budget, log)

    line = {
        "metric": METRIC,
        "value": round(dec["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": dec["steps"],
        "warmup": dec["warmup"],
        "ms_per_step": round(dec["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "BitNet-2B-4T decode projections at M=1 through bitnet_linear (fused quantise + GEMV): "
                        "qkv 3840x2560, o_proj 2560x2560, gate_up 13824x2560, down 2560x6912, lm_head 128256x2560",
            "M": 1, "step_bytes": dec["step_bytes"],
            "per_shape_gbs": {k: round(v["gbs"], 1) for k, v in dec["per_shape"].items()},
            "per_shape_us": {k: round(v["us"], 3) for k, v in dec["per_shape"].items()},
            "per_shape_us_p10_p90": {k: [round(v["us_p10"], 3), round(v["us_p90"], 3)]
                                     for k, v in dec["per_shape"].items()},
            "frac_hbm_peak": round(dec["gbs"] / HBM_PEAK_GBS, 4),
            "timing": dec["timing"],
            "gpu_clocks_smi": {"before": clock_before, "after_headline": clock_after},
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    for M, gemm in gemms.items():
        tot_ops = sum(2.0 * M * v["N"] * v["K"] for v in gemm.values())
        tot_t = sum(v["gemm_us"] for v in gemm.values()) * 1e-6
        line["gemm" if M == 2048 else f"gemm_m{M}"] = {
            "metric": f"GEMM INT8 TOPS (M={M}), LLaMA-7B shapes, pre-quantised activations",
            "value": round(tot_ops / tot_t / 1e12, 1), "unit": "TOPS",
            "frac_int8_peak": round(tot_ops / tot_t / 1e12 / INT8_PEAK_TOPS, 4),
            "per_shape": {k: {"tops": round(v["tops"], 1), "gemm_us": round(v["gemm_us"], 2),
                              "gemm_us_p10": round(v["gemm_us_p10"], 2), "gemm_us_p90": round(v["gemm_us_p90"], 2),
                              "frac_int8_peak": round(v["frac_int8_peak"], 4),
                              "quant_us": round(v["quant_us"], 2), "linear_us": round(v["linear_us"], 2)}
                          for k, v in gemm.items()},
        }
    if small is not None:
        line["small_batch_gemm"] = small
        line["decode_full_step"] = full
        line["linear_options"] = options
        line["fused_small_m"] = fused_m
        line["w8a16_gemv"] = w8
    if machine is not None:
        line["machine_ceilings"] = machine
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
