"""Parity at the full workload sizes, launched the way the benchmark launches them.

* Decode GEMV, M=1, at the BitNet-2B-4T projection shapes (the benchmark's
  weights and activations, same seeds): every output, the int32 accumulators
  and the activation scale against the oracle; also as replays of a captured
  graph, the benchmark's launch mode.
* The same shapes at M=16 (split quantise + GEMM path of bitnet_linear): every
  output against the oracle.
* The same shapes with RMSNorm fused before the call (bitnet_linear_rms, M=1
  and 16), and at M=1 with f32 activations and a bias (bitnet_linear_ex's one
  launch): every output against the oracle.
* Small-batch GEMM, M in {8..256}, LLaMA-7B shapes, pre-quantised activations:
  the int32 accumulators over the whole output against an exact float64 product
  (every partial sum is an integer below 2^53, so any summation order is exact),
  the whole bf16 output against the oracle's epilogue of that exact product, and
  sampled rows and columns of both against the oracle's own contraction.
* Prefill, M in {2048, 4096}, LLaMA-7B shapes, activations with 1% outlier
  channels: the quantised activations and scales over the whole input against
  the oracle, the accumulators against the exact float64 product of the
  oracle's quantised activations, the whole output of bitnet_linear against the
  oracle's epilogue of that product, and sampled rows and columns against the
  oracle's own contraction.
* Every weight matrix is packed by the library's host packer, whose bytes must
  equal the oracle's.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_int8_gemm_amd as tg

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bf16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def assert_bf16_equal(got, want, what):
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} outputs differ, first at {tuple(bad[0])}: {got[tuple(bad[0])]:#06x} vs {want[tuple(bad[0])]:#06x}"


def lib_pack(W):
    """The library's host packer, required to give the oracle's bytes."""
    P = tg.pack_weights(torch.from_numpy(np.ascontiguousarray(W))).numpy()
    assert np.array_equal(P, oracle.pack(W)), "bitnet_pack_weights differs from the oracle's pack"
    return P


def exact_product(q_dev, W_host):
    """acc = q @ W^T in float64 on the GPU: exact for |acc| < 2^53."""
    Wt = torch.from_numpy(W_host).to(DEV).to(torch.float64).t().contiguous()
    return torch.mm(q_dev.to(torch.float64), Wt)


def sample_rows_cols(M, N, seed, n_cols=48):
    g = synth.rng(seed)
    rows = sorted({0, M - 1, M // 2, int(g.integers(0, M))})
    cols = sorted({0, N - 1} | set(int(c) for c in g.choice(N, size=min(n_cols, N), replace=False)))
    return np.array(rows), np.array(cols)


def check_whole(out_dev, exact, sa, sw, what):
    """Every bf16 output against the oracle's epilogue applied to the exact
    accumulators (a float64 product whose partial sums are integers below 2^53,
    so it is the exact integer result; it is computed by torch, not by this
    library) with the oracle's activation scales."""
    acc_exact = exact.cpu().numpy()
    assert np.abs(acc_exact).max(initial=0) < 2 ** 31
    want = oracle.epilogue(acc_exact.astype(np.int32), sa, sw)
    assert_bf16_equal(host_bf16(out_dev), want, f"{what} (whole output)")


def check_samples(out_dev, acc_dev, q, sa, P, sw, seed, what):
    """Rows and columns of the bf16 output (and of the accumulators, if given) against the oracle."""
    M, N = out_dev.shape
    rows, cols = sample_rows_cols(M, N, seed)
    out = host_bf16(out_dev)
    acc_r = oracle.gemm_i32(q[rows], P)                      # whole rows
    acc_c = oracle.gemm_i32(q, P[cols])                      # whole columns
    assert_bf16_equal(out[rows], oracle.epilogue(acc_r, sa[rows], sw), f"{what} rows {rows.tolist()}")
    assert_bf16_equal(out[:, cols], oracle.epilogue(acc_c, sa, sw[cols]), f"{what} sampled columns")
    if acc_dev is not None:
        acc = acc_dev.cpu().numpy()
        assert np.array_equal(acc[rows], acc_r), f"{what}: accumulator rows"
        assert np.array_equal(acc[:, cols], acc_c), f"{what}: accumulator columns"


# ----------------------------------------------------------------------------- decode (BitNet-2B-4T)

@functools.lru_cache(maxsize=None)
def decode_problem(i):
    """Projection i of the decode step with the benchmark's seeds (workload 1)."""
    name, N, K = synth.BITNET_2B_DECODE[i]
    W = synth.ternary_weights(N, K, synth.seed_for(1, 16 * i + synth.T_WEIGHT))
    P = lib_pack(W)
    del W
    sw = synth.weight_scale_bf16(N, K, synth.seed_for(1, 16 * i + synth.T_SCALE))
    x = synth.activations_bf16(1, K, synth.seed_for(1, 16 * i + synth.T_ACT))
    return name, N, K, P, sw, x


DECODE_IDS = [s[0] for s in synth.BITNET_2B_DECODE]


@pytest.mark.parametrize("i", range(len(synth.BITNET_2B_DECODE)), ids=DECODE_IDS)
def test_decode_m1_full(i):
    name, N, K, P, sw, x = decode_problem(i)
    ref = oracle.linear(x, P, sw)
    xd, Pd, swd = dev_bf16(x), dev(P), dev_bf16(sw)
    out = tg.bitnet_linear(xd, Pd, swd)                      # M=1: the fused GEMV
    acc, sa = tg.bitnet_gemv_fused_i32(xd, Pd)
    assert np.array_equal(host_bf16(sa), ref["scale_act"]), name
    assert np.array_equal(acc.cpu().numpy(), ref["acc"]), name
    assert_bf16_equal(host_bf16(out), ref["out"], name)


def test_decode_step_graph_replays():
    """The five projections captured in one graph (as the benchmark runs them),
    replayed three times with eager work and synchronisation in between."""
    probs = [decode_problem(i) for i in range(len(synth.BITNET_2B_DECODE))]
    refs = [oracle.linear(x, P, sw)["out"] for _, _, _, P, sw, x in probs]
    ins = [(dev_bf16(x), dev(P), dev_bf16(sw), torch.empty((1, N), dtype=torch.bfloat16, device=DEV))
           for _, N, _, P, sw, x in probs]
    stream = torch.cuda.Stream()

    def step():
        for xd, Pd, swd, od in ins:
            tg.bitnet_linear(xd, Pd, swd, out=od)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    for rep in range(3):
        for _, _, _, od in ins:
            od.fill_(1.0)                                    # replays must rewrite every output
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for (name, *_), (_, _, _, od), ref in zip(probs, ins, refs):
            assert_bf16_equal(host_bf16(od), ref, f"replay {rep} {name}")


@pytest.mark.parametrize("i", range(len(synth.BITNET_2B_DECODE)), ids=DECODE_IDS)
def test_decode_m16_full(i):
    name, N, K, P, sw, _ = decode_problem(i)
    x = synth.activations_bf16(16, K, synth.seed_for(5, 16 * i + synth.T_ACT))
    ref = oracle.linear(x, P, sw)
    out = tg.bitnet_linear(dev_bf16(x), dev(P), dev_bf16(sw))   # M=16: quantise + GEMM
    assert_bf16_equal(host_bf16(out), ref["out"], f"{name} M=16")


@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("i", range(len(synth.BITNET_2B_DECODE)), ids=DECODE_IDS)
def test_decode_rmsnorm_full(i, M):
    """The decode step with the RMSNorm that precedes every BitLinear call fused
    in (no gain, torch's default eps), launched as the benchmark launches it:
    every output against the oracle, where rows whose fp32 mean another double
    summation order could round the other way may match the alternative."""
    name, N, K, P, sw, _ = decode_problem(i)
    x = synth.activations_bf16(M, K, synth.seed_for(6, 16 * i + synth.T_ACT) + M)
    ref = oracle.linear_rms(x, P, sw)
    amb = ref["ambiguous"]
    alt = oracle.linear_rms(x, P, sw, means=ref["mean_alt"]) if amb.any() else ref
    got = host_bf16(tg.bitnet_linear_rms(dev_bf16(x), dev(P), dev_bf16(sw)))
    ok = np.all(got == ref["out"], axis=1) | (np.all(got == alt["out"], axis=1) & amb)
    assert ok.all(), f"{name} M={M}: rows {np.nonzero(~ok)[0][:8].tolist()} differ (ambiguous: {int(amb.sum())})"


@pytest.mark.parametrize("i", range(len(synth.BITNET_2B_DECODE)), ids=DECODE_IDS)
def test_decode_f32_bias_full(i):
    """bitnet_linear_ex at M=1 with f32 activations and a bias (one launch: the
    f32 row quantised in the GEMV prologue, the bias in its epilogue): every
    output against the oracle."""
    name, N, K, P, sw, _ = decode_problem(i)
    x = synth.rng(synth.seed_for(7, 16 * i + synth.T_ACT)).standard_normal((1, K)).astype(np.float32)
    bias = synth.row_scales_bf16(N, synth.seed_for(7, 16 * i + synth.T_ROWSCALE), lo=-4.0, hi=4.0)
    want = oracle.add_bias(oracle.linear_f32(x, P, sw)["out"], bias)
    out = tg.bitnet_linear(torch.from_numpy(x).to(DEV), dev(P), dev_bf16(sw), bias=dev_bf16(bias))
    assert_bf16_equal(host_bf16(out), want, f"{name} f32 + bias")


# ----------------------------------------------------------------------------- LLaMA-7B GEMMs

@functools.lru_cache(maxsize=4)
def llama_weights(j):
    name, N, K = synth.LLAMA7B_SHAPES[j]
    W = synth.ternary_weights(N, K, synth.seed_for(3, 16 * j + synth.T_WEIGHT))
    P = lib_pack(W)
    sw = synth.weight_scale_bf16(N, K, synth.seed_for(3, 16 * j + synth.T_SCALE))
    return name, N, K, W, P, sw


SMALL_M = [8, 16, 32, 64, 128, 256]


@pytest.mark.parametrize("j", range(3), ids=[s[0] for s in synth.LLAMA7B_SHAPES[:3]])
def test_small_batch_gemm(j):
    name, N, K, W, P, _ = llama_weights(j)
    sw = synth.row_scales_bf16(N, synth.seed_for(2, 16 * j + synth.T_ROWSCALE))   # one scale per output row
    Pd, swd = dev(P), dev_bf16(sw)
    for M in SMALL_M:
        x = synth.activations_bf16(M, K, synth.seed_for(2, 16 * j + synth.T_ACT) + M)
        q, sa = oracle.quantize(x)                           # pre-quantised on the host
        qd, sad = dev(q), dev_bf16(sa)
        out = tg.bitnet_gemm(qd, Pd, sad, swd)
        acc = tg.bitnet_gemm_i32(qd, Pd)
        exact = exact_product(dev(q), W)
        assert torch.equal(acc.to(torch.float64), exact), f"{name} M={M}: accumulators"
        check_whole(out, exact, sa, sw, f"{name} M={M}")
        check_samples(out, acc, q, sa, P, sw, seed=M * 31 + j, what=f"{name} M={M}")


@pytest.mark.parametrize("M", [2048, 4096])
@pytest.mark.parametrize("j", range(4), ids=[s[0] for s in synth.LLAMA7B_SHAPES])
def test_prefill_linear(j, M):
    name, N, K, W, P, sw = llama_weights(j)
    x = synth.activations_bf16(M, K, synth.seed_for(3, 16 * j + synth.T_ACT) + M, outlier_frac=0.01)
    q_ref, sa_ref = oracle.quantize(x)
    xd, Pd, swd = dev_bf16(x), dev(P), dev_bf16(sw)
    q, sa = tg.quantize_activation(xd)
    assert np.array_equal(q.cpu().numpy(), q_ref), f"{name} M={M}: quantised activations"
    assert np.array_equal(host_bf16(sa), sa_ref), f"{name} M={M}: activation scales"
    exact = exact_product(dev(q_ref), W)                     # from the oracle's quantised activations
    acc = tg.bitnet_gemm_i32(q, Pd)
    assert torch.equal(acc.to(torch.float64), exact), f"{name} M={M}: accumulators"
    del acc
    ws = torch.empty((tg.linear_workspace_bytes(M, K),), dtype=torch.uint8, device=DEV)
    out = tg.bitnet_linear(xd, Pd, swd, workspace=ws)       # the benchmark's quantise + GEMM launch
    check_whole(out, exact, sa_ref, sw, f"{name} M={M}")
    del exact
    check_samples(out, None, q_ref, sa_ref, P, sw, seed=M + j, what=f"{name} M={M}")
    out2 = tg.bitnet_gemm(q, Pd, sa, swd)                    # pre-quantised launch: same bits
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16)), f"{name} M={M}: gemm vs linear"
    torch.cuda.empty_cache()
