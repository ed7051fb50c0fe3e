"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself:
hand-worked values of the pages' formulas (tests/golden/), closed forms,
invariants, exact arithmetic, library routines for the special cases that
reduce to them, and brute force on tiny inputs.
"""
import itertools

import numpy as np
import pytest
import torch

import synth
from conftest import read_golden


def bf16_bits(values):
    return torch.tensor(values, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------- packing

def test_pack_closed_forms(orc):
    rows = read_golden("pack_closed_forms.txt")
    assert len(rows) >= 8
    for r in rows:
        w = np.array([[int(t) for t in r["lhs"]]], dtype=np.int8)
        want = np.array([[int(t, 16) for t in r["rhs"]]], dtype=np.uint8)
        got = orc.pack(w)
        assert got.tolist() == want.tolist(), (r, got)


def test_pack_roundtrip_exhaustive_81(orc):
    tuples = np.array(list(itertools.product([-1, 0, 1], repeat=4)), dtype=np.int8)   # 81 x 4
    P = orc.pack(tuples)
    assert P.shape == (81, 1)
    assert len(set(P[:, 0].tolist())) == 81           # injective on valid tuples
    assert np.array_equal(orc.unpack(P, 4), tuples)   # exact round trip
    # every code field of a packed byte is 1, 2 or 3 (code 0 never produced)
    for b in P[:, 0].tolist():
        assert all(((b >> (2 * i)) & 3) != 0 for i in range(4))


def test_pack_roundtrip_random_and_size(orc):
    W = synth.ternary_weights(37, 96, seed=11)
    P = orc.pack(W)
    assert P.shape == (37, 24)
    assert P.nbytes * 8 == W.size * 2            # 2 bits per weight: 8x smaller than bf16
    assert np.array_equal(orc.unpack(P, 96), W)


def test_decode_of_unused_code_is_minus_two(orc):
    # reading: decode is w = code - 2 for every code, so 0b00 gives -2
    P = np.array([[0x00, 0xE4]], dtype=np.uint8)   # 0xE4 = codes 0,1,2,3 from low bits
    assert orc.unpack(P, 8).tolist() == [[-2, -2, -2, -2, -2, -1, 0, 1]]


def test_pack_rejects_bad_input(orc):
    with pytest.raises(orc.OracleError):
        orc.pack(np.zeros((2, 6), dtype=np.int8))          # K % 4 != 0
    with pytest.raises(orc.OracleError):
        orc.pack(np.array([[0, 2, 0, 0]], dtype=np.int8))  # value outside {-1,0,1}
    with pytest.raises(orc.OracleError):
        orc.pack(np.array([[-2, 0, 0, 0]], dtype=np.int8))


# --------------------------------------------------------------------------- bf16

def test_bf16_rounding_matches_torch(orc):
    g = synth.rng(5)
    vals = np.concatenate([
        g.standard_normal(2000).astype(np.float32) * np.float32(1000.0),
        np.array([257.0, 259.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -257.0, 0.0, -0.0, 1e-30, 3.0e38],
                 dtype=np.float32),
    ])
    want = bf16_bits(vals)
    got = np.array([orc.bf16_from_f32(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)
    for h in [0x3F80, 0xC284, 0x33A9, 0x7F7F, 0x0001]:
        assert np.float32(orc.f32_from_bf16(h)) == synth.bf16_bits_to_f32(np.array([h]))[0]


# --------------------------------------------------------------------------- quantisation

def test_quantize_golden_vectors(orc):
    rows = read_golden("quantize_vectors.txt")
    assert len(rows) >= 5
    for r in rows:
        x = bf16_bits([float(t) for t in r["x"]])
        # the fixture values are exactly representable in bf16
        assert np.array_equal(synth.bf16_bits_to_f32(x), np.array([float(t) for t in r["x"]], dtype=np.float32))
        q, sa = orc.quantize(x[None, :])
        assert q[0].tolist() == [int(t) for t in r["q"]], r
        assert int(sa[0]) == int(r["scale_bf16"][0], 16), (r, hex(sa[0]))


def _rows_for_quant_checks():
    a = synth.activations_bf16(48, 2560, seed=21)
    b = synth.activations_bf16(16, 4096, seed=22, outlier_frac=0.01)
    tiny = bf16_bits(np.array([[1e-7, -3e-8, 0.0, 2e-6]], dtype=np.float32))   # absmax below eps
    return [a, b, tiny]


def test_quantize_absmax_maps_to_127_and_range(orc):
    for x in _rows_for_quant_checks()[:2]:
        q, _ = orc.quantize(x)
        xf = synth.bf16_bits_to_f32(x)
        am = np.argmax(np.abs(xf), axis=1)
        assert np.all(np.abs(q[np.arange(len(q)), am]) == 127)
        assert np.all(np.sign(q[np.arange(len(q)), am]) == np.sign(xf[np.arange(len(q)), am]))
        assert q.min() >= -127 and q.max() <= 127


def test_quantize_double_division_identity(orc):
    # fp32(x / s) == fp32((double)x / (double)s): double rounding is harmless for a
    # quotient of two binary32 numbers (53 >= 2*24 + 2), so this is an independent
    # route to the same IEEE quotient.  s itself: fp32(absmax / 127) computed the
    # same way, eps = fp32(1e-5).
    for x in _rows_for_quant_checks():
        q, sa = orc.quantize(x)
        xf = synth.bf16_bits_to_f32(x).astype(np.float64)
        a = np.max(np.abs(xf), axis=1)
        a = np.maximum(a, np.float64(np.float32(1e-5)))
        s = (a / 127.0).astype(np.float32).astype(np.float64)
        y = (xf / s[:, None]).astype(np.float32)
        want = np.clip(np.rint(y), -127, 127).astype(np.int8)   # numpy rint: half to even
        assert np.array_equal(q, want)
        assert np.array_equal(sa, bf16_bits(s.astype(np.float32)))


def test_quantize_symmetry_and_power_of_two_scaling(orc):
    x = synth.activations_bf16(8, 512, seed=23)
    q, sa = orc.quantize(x)
    qn, san = orc.quantize(x ^ np.uint16(0x8000))            # negate every element
    assert np.array_equal(qn, -q) and np.array_equal(san, sa)
    x4 = bf16_bits(synth.bf16_bits_to_f32(x) * np.float32(4.0))   # exact
    q4, sa4 = orc.quantize(x4)
    assert np.array_equal(q4, q)
    assert np.array_equal(synth.bf16_bits_to_f32(sa4), synth.bf16_bits_to_f32(sa) * np.float32(4.0))


def test_quantize_rows_independent(orc):
    x = synth.activations_bf16(6, 256, seed=24)
    q, sa = orc.quantize(x)
    for m in range(6):
        qm, sam = orc.quantize(x[m:m + 1])
        assert np.array_equal(qm[0], q[m]) and sam[0] == sa[m]


# --------------------------------------------------------------------------- contraction

def test_gemm_hand_examples(orc):
    rows = read_golden("gemm_hand.txt")
    assert len(rows) >= 6
    for r in rows:
        q = np.array([[int(t) for t in r["q"]]], dtype=np.int8)
        w = np.array([[int(t) for t in r["w"]]], dtype=np.int8)
        acc = orc.gemm_i32(q, orc.pack(w))
        assert int(acc[0, 0]) == int(r["acc"][0]), r


def test_gemm_brute_force_tiny(orc):
    # int64 dense product of the unpacked ternary matrix, for every small shape
    seed = 100
    for M in range(1, 6):
        for N in range(1, 10):
            for K in range(4, 68, 4):
                seed += 1
                W = synth.ternary_weights(N, K, seed)
                q = synth.random_int8((M, K), seed + 7)
                want = q.astype(np.int64) @ W.astype(np.int64).T
                got = orc.gemm_i32(q, orc.pack(W))
                assert np.array_equal(got, want), (M, N, K)


def test_gemm_exhaustive_rows_k4_k8(orc):
    for K, seed in ((4, 7), (8, 8)):
        W = np.array(list(itertools.product([-1, 0, 1], repeat=K)), dtype=np.int8)   # 3^K rows
        q = synth.random_int8((3, K), seed)
        want = q.astype(np.int64) @ W.astype(np.int64).T
        assert np.array_equal(orc.gemm_i32(q, orc.pack(W)), want)


def test_gemm_closed_forms(orc):
    q = synth.random_int8((5, 256), 31)
    rowsum = q.astype(np.int64).sum(axis=1)
    for val, expect in ((1, rowsum), (-1, -rowsum), (0, 0 * rowsum)):
        W = np.full((7, 256), val, dtype=np.int8)
        acc = orc.gemm_i32(q, orc.pack(W))
        assert np.array_equal(acc, np.repeat(expect[:, None], 7, axis=1))


def test_gemm_invariants(orc):
    W = synth.ternary_weights(19, 320, seed=41)
    q = synth.random_int8((4, 320), 42)
    acc = orc.gemm_i32(q, orc.pack(W))
    perm = synth.rng(43).permutation(320)
    assert np.array_equal(orc.gemm_i32(q[:, perm], orc.pack(W[:, perm])), acc)   # permute K consistently
    assert np.array_equal(orc.gemm_i32(q, orc.pack(-W)), -acc)
    assert np.array_equal(orc.gemm_i32(-q, orc.pack(W)), -acc)
    assert np.abs(acc).max() <= 127 * 320
    # transposing the roles: row m of acc only depends on q[m], column n only on W[n]
    assert np.array_equal(orc.gemm_i32(q[2:3], orc.pack(W[5:9])), acc[2:3, 5:9])


# --------------------------------------------------------------------------- epilogue

def test_epilogue_golden(orc):
    rows = read_golden("epilogue_cases.txt")
    assert len(rows) >= 8
    for r in rows:
        got = orc.epilogue_one(int(r["acc"][0]), int(r["sa"][0], 16), int(r["sw"][0], 16))
        assert got == int(r["out"][0], 16), (r, hex(got))


def test_epilogue_exact_product_identity(orc):
    # (double)acc * (double)sa * (double)sw is exact in double (24 + 8 + 8 bits), so its
    # rounding to fp32 is the single fp32 rounding of the exact product, which the
    # epilogue must reproduce before its bf16 rounding.
    g = synth.rng(51)
    acc = g.integers(-(1 << 23), 1 << 23, size=4000).astype(np.int32)
    acc[:50] = g.integers(-300, 300, size=50)
    sa = bf16_bits(g.uniform(1e-3, 0.1, size=4000).astype(np.float32))
    sw = bf16_bits(g.uniform(1e-3, 0.05, size=4000).astype(np.float32))
    exact = acc.astype(np.float64) * synth.bf16_bits_to_f32(sa).astype(np.float64) \
        * synth.bf16_bits_to_f32(sw).astype(np.float64)
    want = bf16_bits(exact.astype(np.float32))
    got = orc.epilogue(acc[None, :], sa[:1], sw)[0]   # one row: sa broadcast
    got_rows = np.array([orc.epilogue_one(int(a), int(s1), int(s2)) for a, s1, s2 in zip(acc, sa, sw)],
                        dtype=np.uint16)
    assert np.array_equal(got_rows, want)
    exact0 = acc.astype(np.float64) * np.float64(synth.bf16_bits_to_f32(sa[:1])[0]) \
        * synth.bf16_bits_to_f32(sw).astype(np.float64)
    assert np.array_equal(got, bf16_bits(exact0.astype(np.float32)))


# --------------------------------------------------------------------------- whole layer

def test_linear_is_composition_and_k8_example(orc):
    x = bf16_bits([127, 2.5, -2.5, 1.5, -0.5, 0.5, -127, 64])[None, :]
    W = np.array([[1] * 8, [-1] * 8, [0] * 8, [1, -1, 0, 1, -1, 0, -1, 1]], dtype=np.int8)
    sw = np.full((4,), 0x3F80, dtype=np.uint16)
    r = orc.linear(x, orc.pack(W), sw)
    assert r["acc"].tolist() == [[66, -66, 0, 318]]
    assert r["out"].tolist() == [[0x4284, 0xC284, 0x0000, 0x439F]]
    # on a random problem: linear == epilogue(gemm(quantize))
    x = synth.activations_bf16(5, 384, seed=61)
    W = synth.ternary_weights(33, 384, seed=62)
    P = orc.pack(W)
    sw = synth.row_scales_bf16(33, seed=63)
    r = orc.linear(x, P, sw)
    q, sa = orc.quantize(x)
    acc = orc.gemm_i32(q, P)
    assert np.array_equal(r["q"], q) and np.array_equal(r["scale_act"], sa) and np.array_equal(r["acc"], acc)
    assert np.array_equal(r["out"], orc.epilogue(acc, sa, sw))
    for m, n in ((0, 0), (4, 32), (2, 17)):
        o, a = orc.linear_one(q[m], sa[m], P, sw, n)
        assert o == r["out"][m, n] and a == r["acc"][m, n]


# ----------------------------------------------------------------------------- f32 activations and bias

def _f32_from_hex(tokens):
    return np.array([int(t, 16) for t in tokens], dtype=np.uint32).view(np.float32)


def test_quantize_f32_golden(orc):
    for r in read_golden("quantize_f32_vectors.txt"):
        q, sa = orc.quantize_f32(_f32_from_hex(r["x"])[None, :])
        assert q[0].tolist() == [int(t) for t in r["q"]], r
        assert int(sa[0]) == int(r["scale_bf16"][0], 16), r


def test_quantize_f32_equals_bf16_path_on_bf16_values(orc):
    """On values that are exactly bf16, the f32 path is the bf16 path."""
    x = synth.activations_bf16(6, 640, seed=31, outlier_frac=0.02)
    q16, s16 = orc.quantize(x)
    q32, s32 = orc.quantize_f32(synth.bf16_bits_to_f32(x))
    assert np.array_equal(q16, q32) and np.array_equal(s16, s32)


def test_quantize_f32_absmax_and_double_division(orc):
    g = synth.rng(33)
    x = g.standard_normal((5, 300)).astype(np.float32) * np.float32(3.0)
    q, sa = orc.quantize_f32(x)
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(q[np.arange(5), am] == np.sign(x[np.arange(5), am]) * 127)
    # independent quantiser: fp32 division emulated in double (exact rounding, 53 >= 2*24+2)
    a = np.maximum(np.abs(x).max(axis=1), np.float32(1e-5)).astype(np.float32)
    s = (a.astype(np.float64) / 127.0).astype(np.float32)
    y = (x.astype(np.float64) / s.astype(np.float64)[:, None]).astype(np.float32)
    assert np.array_equal(q, np.clip(np.rint(y), -127, 127).astype(np.int8))


def test_add_bias_golden(orc):
    for r in read_golden("bias_cases.txt"):
        y = np.array([[int(r["y"][0], 16)]], dtype=np.uint16)
        b = np.array([int(r["bias"][0], 16)], dtype=np.uint16)
        assert int(orc.add_bias(y, b)[0, 0]) == int(r["out"][0], 16), r


def test_add_bias_is_per_column_and_matches_torch(orc):
    g = synth.rng(34)
    y = torch.from_numpy(g.standard_normal((4, 9)).astype(np.float32)).to(torch.bfloat16)
    b = torch.from_numpy(g.standard_normal((9,)).astype(np.float32)).to(torch.bfloat16)
    want = (y + b).view(torch.int16).numpy().view(np.uint16)   # torch adds bf16 in fp32, rounds once
    got = orc.add_bias(y.view(torch.int16).numpy().view(np.uint16), b.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(got, want)


def test_linear_f32_is_composition(orc):
    g = synth.rng(35)
    x = g.standard_normal((3, 128)).astype(np.float32)
    W = synth.ternary_weights(7, 128, seed=36)
    P = orc.pack(W)
    sw = synth.row_scales_bf16(7, seed=37)
    r = orc.linear_f32(x, P, sw)
    q, sa = orc.quantize_f32(x)
    assert np.array_equal(r["q"], q) and np.array_equal(r["scale_act"], sa)
    assert np.array_equal(r["acc"], q.astype(np.int64) @ W.astype(np.int64).T)
    assert np.array_equal(r["out"], orc.epilogue(r["acc"], sa, sw))


# ----------------------------------------------------------------------------- W8A16 decode matmul

def test_w8a16_hand_example(orc):
    # x = [1, 2, -0.5, 0.25] (bf16-exact), q rows [3, -1, 4, 8] and [-127, 0, 127, 1]:
    #   row 0: 3 - 2 - 2 + 2 = 1, times scale 0.5 -> 0.5
    #   row 1: -127 + 0 - 63.5 + 0.25 = -190.25, times scale 2 -> -380.5
    x = bf16_bits([1.0, 2.0, -0.5, 0.25])[None, :]
    q = np.array([[3, -1, 4, 8], [-127, 0, 127, 1]], dtype=np.int8)
    y, bound = orc.w8a16(x, q, np.array([0.5, 2.0], dtype=np.float32))
    assert y.tolist() == [[0.5, -380.5]]
    assert bound.tolist() == [[0.5 * (3 + 2 + 2 + 2), 2.0 * (127 + 0 + 63.5 + 0.25)]]


def test_w8a16_zero_weights_and_symmetries(orc):
    x = synth.activations_bf16(3, 256, seed=41)
    g = synth.rng(42)
    q = g.integers(-127, 128, size=(5, 256)).astype(np.int8)
    sc = g.uniform(0.001, 0.1, size=5).astype(np.float32)
    y, _ = orc.w8a16(x, q, sc)
    assert np.all(orc.w8a16(x, np.zeros_like(q), sc)[0] == 0.0)
    assert np.array_equal(orc.w8a16(x, -q, sc)[0], -y)
    x2 = bf16_bits(synth.bf16_bits_to_f32(x) * 2.0)          # exact doubling in bf16
    assert np.array_equal(orc.w8a16(x2, q, sc)[0], 2.0 * y)


def test_w8a16_brute_force_exact(orc):
    from fractions import Fraction
    x = synth.activations_bf16(2, 40, seed=43)
    g = synth.rng(44)
    q = g.integers(-127, 128, size=(3, 40)).astype(np.int8)
    sc = g.uniform(0.01, 1.0, size=3).astype(np.float32)
    y, _ = orc.w8a16(x, q, sc)
    xf = synth.bf16_bits_to_f32(x)
    for m in range(2):
        for n in range(3):
            exact = sum(Fraction(float(xf[m, k])) * int(q[n, k]) for k in range(40)) * Fraction(float(sc[n]))
            assert y[m, n] == float(exact)


# ----------------------------------------------------------------------------- RMSNorm before quantisation

def _torch_rms_norm_bits(x_bits, gain_bits, eps):
    """torch's own F.rms_norm on the same bf16 input (the library routine the reading follows)."""
    import torch
    import torch.nn.functional as F
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16)
    g = None if gain_bits is None else torch.from_numpy(gain_bits.view(np.int16)).view(torch.bfloat16)
    y = F.rms_norm(x, [x.shape[-1]], g, eps)
    return y.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("K", [256, 2560, 6912])
@pytest.mark.parametrize("with_gain", [False, True])
@pytest.mark.parametrize("eps", [None, 1e-5])
@pytest.mark.parametrize("magnitude", [1.0, 2.0 ** -12])
def test_rmsnorm_equals_torch_on_exact_rows(orc, K, with_gain, eps, magnitude):
    # Integer activations in [-8, 8] (times a power of two): every sum of squares
    # is an integer below 2^24 (times a power of two), exact in torch's fp32
    # reduction in any order, so the normalised values must agree bit for bit.
    # At 2^-12 the mean is comparable to eps, which makes eps's place visible.
    g = synth.rng(900 + K)
    x = bf16_bits((g.integers(-8, 9, size=(32, K)) * magnitude).astype(np.float32))
    gain = bf16_bits(g.uniform(0.5, 1.5, size=K).astype(np.float32)) if with_gain else None
    r = orc.rmsnorm_quantize(x, gain, orc.FP32_EPS if eps is None else eps)
    assert not r["ambiguous"].any()
    assert np.array_equal(r["xn"], _torch_rms_norm_bits(x, gain, eps))


def test_rmsnorm_close_to_torch_on_random_rows(orc):
    # Random bf16 rows: torch sums the squares in fp32, the oracle in double, so
    # an fp32 mean can differ in its last bit; the normalised values then differ
    # by at most one bf16 step, and rarely.
    x = synth.activations_bf16(64, 2560, seed=910)
    r = orc.rmsnorm_quantize(x)
    want = _torch_rms_norm_bits(x, None, None)
    a = r["xn"].astype(np.int32)
    b = want.astype(np.int32)
    oa = np.where(a & 0x8000, -(a & 0x7FFF), a & 0x7FFF)
    ob = np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    assert np.abs(oa - ob).max() <= 1
    assert (a != b).mean() < 1e-3


def test_rmsnorm_constant_and_zero_rows(orc):
    K = 512
    x = np.zeros((4, K), dtype=np.uint16)
    x[0] = bf16_bits(np.full(K, 0.5, dtype=np.float32))
    x[1] = bf16_bits(np.full(K, -3.0, dtype=np.float32))
    x[2] = bf16_bits(np.where(np.arange(K) % 2 == 0, 7.0, -7.0).astype(np.float32))
    r = orc.rmsnorm_quantize(x)
    # a row of constant magnitude c normalises to sign(x) * c / sqrt(c^2 + eps), i.e. +-1 in bf16
    assert np.all(r["xn"][0] == 0x3F80) and np.all(r["xn"][1] == 0xBF80)
    assert np.array_equal(r["xn"][2], np.where(np.arange(K) % 2 == 0, 0x3F80, 0xBF80))
    assert np.all(np.abs(r["q"][:3]) == 127)
    # all-zero row: zeros out, the quantiser's eps floor for the scale
    assert np.all(r["xn"][3] == 0) and np.all(r["q"][3] == 0) and r["mean"][3] == 0.0
    assert r["scale_act"][3] == 0x33A9


def test_rmsnorm_symmetries(orc):
    x = synth.activations_bf16(8, 1024, seed=920)
    xf = synth.bf16_bits_to_f32(x)
    base = orc.rmsnorm_quantize(x, eps=0.0)
    neg = orc.rmsnorm_quantize(bf16_bits(-xf), eps=0.0)
    assert np.array_equal(neg["xn"], base["xn"] ^ np.uint16(0x8000) * (base["xn"] != 0))
    for j in (-6, 5):                                        # exact power-of-two scaling, eps = 0
        sc = orc.rmsnorm_quantize(bf16_bits(xf * np.float32(2.0 ** j)), eps=0.0)
        assert np.array_equal(sc["xn"], base["xn"]) and np.array_equal(sc["q"], base["q"])
    two = orc.rmsnorm_quantize(x, bf16_bits(np.full(1024, 2.0, dtype=np.float32)), eps=0.0)
    assert np.array_equal(synth.bf16_bits_to_f32(two["xn"]), 2.0 * synth.bf16_bits_to_f32(base["xn"]))
    perm = synth.rng(921).permutation(1024)
    xi = bf16_bits(synth.rng(922).integers(-8, 9, size=(8, 1024)).astype(np.float32))   # exact sums
    a = orc.rmsnorm_quantize(xi)
    b = orc.rmsnorm_quantize(xi[:, perm])
    assert np.array_equal(b["xn"], a["xn"][:, perm]) and np.array_equal(b["q"], a["q"][:, perm])


def test_rmsnorm_unit_mean_square(orc):
    x = synth.activations_bf16(16, 4096, seed=930, outlier_frac=0.01)
    xn = synth.bf16_bits_to_f32(orc.rmsnorm_quantize(x)["xn"]).astype(np.float64)
    assert np.allclose((xn * xn).mean(axis=1), 1.0, rtol=2.0 ** -7)


def test_rmsnorm_ambiguous_mean_is_flagged(orc):
    # [2, 0, 0, 2^-11]: sum of squares 4 + 2^-22, mean 1 + 2^-24, exactly halfway
    # between the fp32 values 1 and 1 + 2^-23.  [2, 0, 0, 0]: mean exactly 1.
    x = bf16_bits(np.array([[2.0, 0.0, 0.0, 2.0 ** -11], [2.0, 0.0, 0.0, 0.0]], dtype=np.float32))
    r = orc.rmsnorm_quantize(x, eps=0.0)
    assert r["ambiguous"].tolist() == [True, False]
    assert r["mean"].tolist() == [1.0, 1.0]
    assert float(r["mean_alt"][0]) == 1.0 + 2.0 ** -23
    forced = orc.rmsnorm_quantize(x, eps=0.0, means=np.array([1.0 + 2.0 ** -23, 1.0], dtype=np.float32))
    assert forced["mean"].tolist() == [1.0 + 2.0 ** -23, 1.0] and not forced["ambiguous"].any()


def test_linear_rms_is_the_composition(orc):
    x = synth.activations_bf16(5, 512, seed=940)
    gain = synth.row_scales_bf16(512, seed=941, lo=0.5, hi=2.0)
    W = synth.ternary_weights(33, 512, seed=942)
    P = orc.pack(W)
    sw = synth.row_scales_bf16(33, seed=943)
    r = orc.linear_rms(x, P, sw, gain, 1e-6)
    ref = orc.linear(r["xn"], P, sw)
    assert np.array_equal(r["out"], ref["out"]) and np.array_equal(r["q"], ref["q"])
    assert np.array_equal(r["acc"], r["q"].astype(np.int64) @ W.astype(np.int64).T)
