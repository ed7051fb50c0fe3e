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
                                          turn those four passes into profiles/gemm_m2048_qkvo_counters.md
  python bench.py --gemv-scaling          M=1 bitnet_linear (quantise + GEMV) time against N at K=2560,
                                          and a line fit: fixed cost per launch and marginal stream rate
"""
import argparse
import csv
import gzip
import glob
import hashlib
import json
import os
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


def time_graph(graph, replays, stream):
    """Replay `graph` on `stream` and time the replays with events on that stream."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(replays):
            graph.replay()   # launches on the current stream, i.e. `stream`
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3  # seconds


RAMP_SECONDS = 0.03


def ramp(graph, stream, seconds=RAMP_SECONDS):
    """Untimed replays of `graph` until `seconds` of GPU time have passed.  The
    GPU's clocks take several milliseconds of sustained work to settle (about
    10 ms measured on MI355X after an idle gap), so a warm-up of one or two short
    replays would leave the timed replays inside that ramp."""
    spent, n = 0.0, 1
    while spent < seconds:
        spent += time_graph(graph, n, stream)
        n = min(2 * n, 1024)


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


def run_decode(shapes, dev_sets, steps, warmup, stream, log):
    copies = len(dev_sets)

    def one_rotation():
        for d in dev_sets:
            for name, N, K in shapes:
                Pd, swd, xd, od = d[name]
                tg.bitnet_linear(xd, Pd, swd, out=od)

    g = capture(one_rotation, stream)
    reps = max(1, -(-steps // copies))
    wreps = max(1, -(-warmup // copies))
    time_graph(g, wreps, stream)
    secs = time_graph(g, reps, stream)
    n_steps = reps * copies
    step_bytes = sum(gemv_bytes(1, N, K) for _, N, K in shapes)
    result = {"steps": n_steps, "warmup": wreps * copies, "seconds": secs, "ms_per_step": secs / n_steps * 1e3,
              "gbs": step_bytes * n_steps / secs / 1e9, "step_bytes": step_bytes}

    # Per-projection launch durations: a graph of back-to-back launches of one
    # shape over the rotating copies, timed with events around its replays.
    per_shape = {}
    for name, N, K in shapes:
        def launches(name=name):
            for d in dev_sets:
                Pd, swd, xd, od = d[name]
                tg.bitnet_linear(xd, Pd, swd, out=od)
        gs = capture(launches, stream)
        ramp(gs, stream)
        r = 30
        t = time_graph(gs, r, stream) / (r * copies)
        per_shape[name] = {"N": N, "K": K, "us": t * 1e6, "gbs": gemv_bytes(1, N, K) / t / 1e9,
                           "bytes": gemv_bytes(1, N, K)}
        log(f"  {name:8s} N={N:6d} K={K:5d}: {t * 1e6:8.2f} us  {per_shape[name]['gbs']:8.1f} GB/s")
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

        def gemm_only():
            for Pd in Ps:
                tg.bitnet_gemm(q, Pd, sa, sw, out=o)

        def linear_full():
            for Pd in Ps:
                tg.bitnet_linear(x, Pd, sw, out=o, workspace=ws)

        def quant_only():
            for _ in Ps:
                tg.quantize_activation(x, out=q, scale=sa)

        res = {"N": N, "K": K}
        for tag, fn in (("gemm", gemm_only), ("linear", linear_full), ("quant", quant_only)):
            g = capture(fn, stream)
            ramp(g, stream)
            reps = 10
            t = time_graph(g, reps, stream) / (reps * rotate)
            res[tag + "_us"] = t * 1e6
        ops = 2.0 * M * N * K
        res["tops"] = ops / (res["gemm_us"] * 1e-6) / 1e12
        res["linear_tops"] = ops / (res["linear_us"] * 1e-6) / 1e12
        res["frac_int8_peak"] = res["tops"] / INT8_PEAK_TOPS
        out[name] = res
        log(f"  M={M} {name:8s} N={N:6d} K={K:5d}: gemm {res['gemm_us']:8.1f} us {res['tops']:7.1f} TOPS "
            f"({100 * res['frac_int8_peak']:.1f}% of peak); quant {res['quant_us']:.1f} us; "
            f"linear {res['linear_us']:.1f} us")
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

            def run():
                for Pd in Ps:
                    tg.bitnet_gemm(q, Pd, sa, sw, out=o)

            g = capture(run, stream)
            ramp(g, stream)
            t = time_graph(g, 3, stream) / (3 * copies)
            ops, nbytes = 2.0 * M * N * K, gemm_bytes(M, N, K)
            r = {"us": round(t * 1e6, 2), "gbs": round(nbytes / t / 1e9, 1), "tops": round(ops / t / 1e12, 1),
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
        reps = 20
        t = time_graph(g, reps, stream) / reps
        if M == 1:
            nbytes = sum(gemv_bytes(M, N, K) for _, N, K, _, _ in calls)
        else:  # quantise (2MK in, MK + 2M out) + GEMM
            nbytes = sum(gemm_bytes(M, N, K) + 3 * M * K + 2 * M for _, N, K, _, _ in calls)
        key = f"M{M}_rmsnorm" if rms else f"M{M}"
        res[key] = {"us_per_step": round(t * 1e6, 2), "tokens_per_s": round(M / t, 1),
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
            def run(x=x, b=b):
                for Pd in Ps:
                    tg.bitnet_linear(x, Pd, sw, out=o, workspace=ws, bias=b)
            g = capture(run, stream)
            ramp(g, stream)
            t = time_graph(g, 3, stream) / (3 * copies)
            r[tag + "_us"] = round(t * 1e6, 2)
        out[f"{name}_M{M}"] = r
        log(f"  {name:10s} M={M:5d} N={N:6d} K={K:5d}: bf16 {r['bf16_us']:8.2f} us, +bias {r['bf16_bias_us']:8.2f} us, "
            f"f32 input {r['f32_us']:8.2f} us")
        del Ps, xb, xf, o, ws
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

            def run(x=x, y=y):
                for qd in qs:
                    tg.w8a16_gemv(x, qd, sc, out=y)
            g = capture(run, stream)
            ramp(g, stream)
            t = time_graph(g, 3, stream) / (3 * copies)
            r[f"M{M}_us"] = round(t * 1e6, 2)
            r[f"M{M}_gbs"] = round(w8a16_bytes(M, N, K) / t / 1e9, 1)
        out[name] = r
        log(f"  {name:16s} N={N:6d} K={K:5d}: M=1 {r['M1_us']:8.2f} us {r['M1_gbs']:7.1f} GB/s, "
            f"M=16 {r['M16_us']:8.2f} us {r['M16_gbs']:7.1f} GB/s")
        del qs, q
        torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- CPU oracle

def run_cpu_baseline(host, shapes, budget_s, log):
    import oracle  # the oracle is only ever used here, for the CPU baseline leg
    packed = {name: oracle.pack(host[name][0]) for name, _, _ in shapes}
    t0 = time.perf_counter()
    n = 0
    while True:
        for name, N, K in shapes:
            _, _, sw, x = host[name]
            oracle.linear(x, packed[name], sw)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 1000:
            break
    step_bytes = sum(gemv_bytes(1, N, K) for _, N, K in shapes)
    gbs = step_bytes * n / el / 1e9
    log(f"cpu oracle: {n} steps in {el:.1f} s -> {gbs:.3f} GB/s on {oracle.num_threads()} threads")
    return {"value": gbs, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} full M=1 decode steps (all five BitNet-2B-4T projections), {el:.1f} s",
            "ms_per_step": el / n * 1e3}


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


TRACE_ARGS = "--steps 22 --warmup 5 --no-cpu-baseline"


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


GEMM_PMC_FILE = os.path.join(ROOT, "profiles", "gemm_m2048_qkvo_counters.md")
GEMM_PMC_PASSES = {  # pass name -> counters (each pass a run of its own)
    "a": "SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_VALU_MFMA_COEXEC_CYCLES",
    "b": "SQ_WAIT_INST_ANY SQ_WAVE_CYCLES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS SQ_BUSY_CYCLES",
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
}
GEMM_PMC_WARM, GEMM_PMC_REPS = 300, 20


def run_pmc_target_gemm(device):
    """Eager launches for counter passes over the prefill GEMM: a plain copy of
    CALIB_COPY_BYTES (byte-counter calibration), then GEMM_PMC_WARM +
    GEMM_PMC_REPS launches of bitnet_gemm on the LLaMA-7B qkvo shape at M=2048
    (pre-quantised activations); the summary keeps the last GEMM_PMC_REPS, when
    the clocks have settled."""
    a = torch.full((CALIB_COPY_BYTES,), 7, dtype=torch.uint8, device=device)
    b = torch.empty_like(a)
    i, (name, N, K) = next((i, sh) for i, sh in enumerate(synth.LLAMA7B_SHAPES) if sh[0] == "qkvo")
    M = 2048
    P = tg.pack_weights(torch.from_numpy(synth.ternary_weights(N, K, synth.seed_for(3, 16 * i + synth.T_WEIGHT)))).to(device)
    sw = dev_bf16(synth.weight_scale_bf16(N, K, synth.seed_for(3, 16 * i + synth.T_SCALE)), device)
    x = dev_bf16(synth.activations_bf16(M, K, synth.seed_for(3, 16 * i + synth.T_ACT), outlier_frac=0.01), device)
    q, sa = tg.quantize_activation(x)
    o = torch.empty((M, N), dtype=torch.bfloat16, device=device)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    for _ in range(GEMM_PMC_WARM + GEMM_PMC_REPS):
        tg.bitnet_gemm(q, P, sa, sw, out=o)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_target_gemm": "done", "M": M, "N": N, "K": K,
                      "launches": GEMM_PMC_WARM + GEMM_PMC_REPS}), flush=True)


def summarize_gemm_pmc(dirs):
    """Markdown summary of the four counter passes of run_pmc_target_gemm (the
    directories in GEMM_PMC_PASSES order): per-launch averages over the last
    GEMM_PMC_REPS GEMM dispatches of each pass."""
    vals, durs, calib, kname = {}, [], {}, set()
    for (pname, counters), folder in zip(GEMM_PMC_PASSES.items(), dirs):
        rows = _csv_rows(folder, "counter_collection.csv")
        gemm_ids = sorted({int(_col(r, "Dispatch_Id")) for r in rows if "gemm_mfma_kernel" in _col(r, "Kernel_Name")})
        keep = set(gemm_ids[-GEMM_PMC_REPS:])
        if len(keep) < GEMM_PMC_REPS:
            raise SystemExit(f"pass {pname}: only {len(keep)} GEMM dispatches in {folder}")
        seen_dur = set()
        for r in rows:
            did = int(_col(r, "Dispatch_Id"))
            cname = _col(r, "Counter_Name")
            v = float(_col(r, "Counter_Value"))
            if did in keep:
                vals.setdefault(cname, []).append(v)
                m = re.search(r"gemm_mfma_kernel<[^>]*>", _col(r, "Kernel_Name"))
                kname.add(m.group(0) if m else _col(r, "Kernel_Name"))
                if pname == "a" and did not in seen_dur:
                    seen_dur.add(did)
                    durs.append(float(_col(r, "End_Timestamp")) - float(_col(r, "Start_Timestamp")))
            elif "copyBuffer" in _col(r, "Kernel_Name") and cname in ("FETCH_SIZE", "WRITE_SIZE"):
                calib.setdefault(cname, []).append(v)
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    dur_ns = sum(durs) / len(durs)
    i, (name, N, K) = next((i, sh) for i, sh in enumerate(synth.LLAMA7B_SHAPES) if sh[0] == "qkvo")
    M = 2048
    simds, clk = 256 * 4, 2.4e9
    mfma_cycles = 32.0  # v_mfma_i32_32x32x32_i8 per SIMD
    busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"]
    factor = {c: CALIB_COPY_BYTES / (1024.0 * max(v)) for c, v in calib.items()}
    fetch_b = avg["FETCH_SIZE"] * 1024.0 * factor["FETCH_SIZE"]
    write_b = avg["WRITE_SIZE"] * 1024.0 * factor["WRITE_SIZE"]
    algo = gemm_bytes(M, N, K)
    cmds = [f"timeout -s KILL 90 rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_gemm_{p} -o run -- "
            "python3 bench.py --pmc-target-gemm" for p, c in GEMM_PMC_PASSES.items()]
    cmds.append("python bench.py --summarize-gemm-pmc " + " ".join(f"gpurun_out/pmc_gemm_{p}" for p in GEMM_PMC_PASSES))
    md = [f"# Counters of the prefill GEMM (bitnet_gemm, LLaMA-7B qkvo, M={M}, N={N}, K={K})", "",
          "Commands (each pass a run of its own, from the repository root after `cd /tmp && export TMPDIR=/tmp`):", ""]
    md += ["    " + c for c in cmds]
    md += ["", f"Per-launch averages over the last {GEMM_PMC_REPS} of {GEMM_PMC_WARM + GEMM_PMC_REPS} eager launches "
           f"(`{', '.join(sorted(kname))}`, 256 workgroups of 8 waves).", "",
           "| quantity | value |", "|---|---:|",
           f"| dispatch duration (profiled) | {dur_ns / 1e3:.2f} µs |",
           f"| SQ_INSTS_MFMA | {avg['SQ_INSTS_MFMA']:.0f} (2MNK / 65536 = {2 * M * N * K // 65536}) |",
           f"| SQ_VALU_MFMA_BUSY_CYCLES | {busy:.4g} ({busy / avg['SQ_INSTS_MFMA']:.1f} per MFMA) |",
           f"| MFMA busy / (duration × 2.4 GHz × {simds} SIMDs) | {busy / (dur_ns * 1e-9 * clk * simds):.3f} |",
           f"| VALU instructions per MFMA | {avg['SQ_INSTS_VALU'] / avg['SQ_INSTS_MFMA']:.2f} |",
           f"| MFMA cycles with VALU co-issued (COEXEC / MFMA busy) | {avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / busy:.3f} |",
           f"| LDS instructions per MFMA | {avg['SQ_INSTS_LDS'] / avg['SQ_INSTS_MFMA']:.2f} |",
           f"| LDS bank-conflict cycles per LDS instruction | {avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_INSTS_LDS']:.2f} |",
           f"| SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES | {avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.3f} |",
           f"| SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES | {avg['SQ_WAIT_INST_LDS'] / avg['SQ_WAVE_CYCLES']:.3f} |",
           f"| HBM bytes (FETCH_SIZE × {factor['FETCH_SIZE']:.3f} + WRITE_SIZE × {factor['WRITE_SIZE']:.3f}) | "
           f"{fetch_b + write_b:.4g} ({(fetch_b + write_b) / algo:.2f} × the {algo} algorithmic bytes) |"]
    md += ["", "The byte counters are scaled by what they read for a plain device copy of 256 MiB in the same run.",
           "The MFMA peak used for the fraction is the dense int8 rate at 2.4 GHz: 1024 SIMDs × 32768 MACs per",
           "32 cycles = 5.0 POPS."]
    with open(GEMM_PMC_FILE, "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2200)
    ap.add_argument("--warmup", type=int, default=660)
    ap.add_argument("--gemm-m", type=int, default=2048)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the small-batch GEMM and full decode-step lines")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--pmc-target", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR")
    ap.add_argument("--trace-args", default=TRACE_ARGS, help="the bench.py arguments of the traced run")
    ap.add_argument("--pmc-target-gemm", action="store_true")
    ap.add_argument("--summarize-gemm-pmc", nargs=4, metavar=("A_DIR", "B_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--gemv-scaling", action="store_true")
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

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path; run with --gpus 1", file=sys.stderr)
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
    stream = torch.cuda.Stream(device)
    if args.gemv_scaling:
        run_gemv_scaling(device, stream)
        return

    shapes, host, dev_sets = build_decode(device, log)
    log("decode GEMV M=1 (BitNet-2B-4T shapes):")
    dec = run_decode(shapes, dev_sets, args.steps, args.warmup, stream, log)
    log(f"decode step: {dec['ms_per_step'] * 1e3:.2f} us/step, {dec['gbs']:.1f} GB/s "
        f"({100 * dec['gbs'] / HBM_PEAK_GBS:.1f}% of HBM peak)")
    del dev_sets
    torch.cuda.empty_cache()

    gemm = None
    if not args.no_gemm:
        log(f"prefill GEMM M={args.gemm_m} (LLaMA-7B shapes):")
        gemm = run_gemm(device, stream, args.gemm_m, log)

    small = full = options = w8 = None
    if not args.no_extra:
        log("small-batch GEMM M=8..256 (LLaMA-7B layer shapes, pre-quantised):")
        small = run_small_batch(device, stream, log)
        log("full BitNet-2B-4T decode step (30 layers x 4 + lm_head = 121 calls):")
        full = run_decode_full(device, stream, log)
        log("bitnet_linear options (f32 activations, bias):")
        options = run_options(device, stream, log)
        log("INT8 weight-only matmul (W8A16), decode shapes:")
        w8 = run_w8a16(device, stream, log)

    lm = dec["per_shape"]["lm_head"]
    traffic = load_traffic(lm["bytes"])
    roofline = {"bound": "hbm", "achieved": round(lm["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(lm["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "gemv_stream_kernel (lm_head 128256x2560, M=1)",
                "bytes_per_launch": lm["bytes"], "avg_launch_us": round(lm["us"], 3)}

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
        "ms_per_step": round(dec["ms_per_step"], 5),
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
            "frac_hbm_peak": round(dec["gbs"] / HBM_PEAK_GBS, 4),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if gemm is not None:
        tot_ops = sum(2.0 * args.gemm_m * v["N"] * v["K"] for v in gemm.values())
        tot_t = sum(v["gemm_us"] for v in gemm.values()) * 1e-6
        line["gemm"] = {
            "metric": f"GEMM INT8 TOPS (M={args.gemm_m}), LLaMA-7B shapes, pre-quantised activations",
            "value": round(tot_ops / tot_t / 1e12, 1), "unit": "TOPS",
            "frac_int8_peak": round(tot_ops / tot_t / 1e12 / INT8_PEAK_TOPS, 4),
            "per_shape": {k: {"tops": round(v["tops"], 1), "gemm_us": round(v["gemm_us"], 2),
                              "quant_us": round(v["quant_us"], 2), "linear_us": round(v["linear_us"], 2)}
                          for k, v in gemm.items()},
        }
    if small is not None:
        line["small_batch_gemm"] = small
        line["decode_full_step"] = full
        line["linear_options"] = options
        line["w8a16_gemv"] = w8
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
