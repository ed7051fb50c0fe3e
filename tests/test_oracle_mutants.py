"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each.

Each mutant is a copy of the oracle source with one textual change, compiled to a
temporary library.  The pin battery below (golden hand-worked values, exact-arithmetic
identities, brute force) must fail on every mutant and pass on the real oracle.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import read_golden
from oracle import build as obuild


def _bf16(values):
    return torch.tensor(values, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _pin_battery(lib):
    """Returns the names of the pins that fail for the library `lib`."""
    failed = []

    def check(name, fn):
        try:
            ok = fn()
        except oracle.OracleError:
            ok = False
        if not ok:
            failed.append(name)

    def pack_golden():
        for r in read_golden("pack_closed_forms.txt"):
            w = np.array([[int(t) for t in r["lhs"]]], dtype=np.int8)
            if oracle.pack(w, lib=lib)[0].tolist() != [int(t, 16) for t in r["rhs"]]:
                return False
        return True

    def unpack_roundtrip():
        W = synth.ternary_weights(9, 64, seed=3)
        return np.array_equal(oracle.unpack(oracle.pack(W, lib=lib), 64, lib=lib), W)

    def quant_golden():
        for r in read_golden("quantize_vectors.txt"):
            q, sa = oracle.quantize(_bf16([float(t) for t in r["x"]])[None, :], lib=lib)
            if q[0].tolist() != [int(t) for t in r["q"]] or int(sa[0]) != int(r["scale_bf16"][0], 16):
                return False
        return True

    def quant_absmax():
        x = synth.activations_bf16(8, 1024, seed=4)
        q, _ = oracle.quantize(x, lib=lib)
        xf = synth.bf16_bits_to_f32(x)
        am = np.argmax(np.abs(xf), axis=1)
        return bool(np.all(q[np.arange(8), am] == np.sign(xf[np.arange(8), am]) * 127))

    def gemm_hand():
        for r in read_golden("gemm_hand.txt"):
            q = np.array([[int(t) for t in r["q"]]], dtype=np.int8)
            w = np.array([[int(t) for t in r["w"]]], dtype=np.int8)
            if int(oracle.gemm_i32(q, oracle.pack(w, lib=lib), lib=lib)[0, 0]) != int(r["acc"][0]):
                return False
        return True

    def gemm_brute():
        for (M, N, K, s) in ((3, 5, 12, 1), (4, 7, 64, 2), (1, 3, 4, 3), (5, 2, 36, 4)):
            W = synth.ternary_weights(N, K, s)
            q = synth.random_int8((M, K), s + 9)
            if not np.array_equal(oracle.gemm_i32(q, oracle.pack(W, lib=lib), lib=lib),
                                  q.astype(np.int64) @ W.astype(np.int64).T):
                return False
        return True

    def epi_golden():
        for r in read_golden("epilogue_cases.txt"):
            got = oracle.epilogue_one(int(r["acc"][0]), int(r["sa"][0], 16), int(r["sw"][0], 16), lib=lib)
            if got != int(r["out"][0], 16):
                return False
        return True

    def epi_batch():
        g = synth.rng(8)
        acc = g.integers(-(1 << 20), 1 << 20, size=(3, 5)).astype(np.int32)
        sa = _bf16(g.uniform(1e-3, 0.1, size=3).astype(np.float32))
        sw = _bf16(g.uniform(1e-3, 0.05, size=5).astype(np.float32))
        exact = acc.astype(np.float64) * synth.bf16_bits_to_f32(sa).astype(np.float64)[:, None] \
            * synth.bf16_bits_to_f32(sw).astype(np.float64)[None, :]
        return np.array_equal(oracle.epilogue(acc, sa, sw, lib=lib), _bf16(exact.astype(np.float32)))

    def linear_k8():
        x = _bf16([127, 2.5, -2.5, 1.5, -0.5, 0.5, -127, 64])[None, :]
        W = np.array([[1] * 8, [1, -1, 0, 1, -1, 0, -1, 1]], dtype=np.int8)
        r = oracle.linear(x, oracle.pack(W, lib=lib), np.full((2,), 0x3F80, dtype=np.uint16), lib=lib)
        return r["out"].tolist() == [[0x4284, 0x439F]]

    def linear_shape():
        x = synth.activations_bf16(3, 64, seed=5)
        W = synth.ternary_weights(5, 64, seed=6)
        P = oracle.pack(W, lib=lib)
        r = oracle.linear(x, P, np.full((5,), 0x3F80, dtype=np.uint16), lib=lib)
        return np.array_equal(r["acc"], r["q"].astype(np.int64) @ W.astype(np.int64).T)

    def quant_f32_golden():
        for r in read_golden("quantize_f32_vectors.txt"):
            x = np.array([int(t, 16) for t in r["x"]], dtype=np.uint32).view(np.float32)[None, :]
            q, sa = oracle.quantize_f32(x, lib=lib)
            if q[0].tolist() != [int(t) for t in r["q"]] or int(sa[0]) != int(r["scale_bf16"][0], 16):
                return False
        return True

    def bias_golden():
        for r in read_golden("bias_cases.txt"):
            y = np.array([[int(r["y"][0], 16), 0]], dtype=np.uint16)
            b = np.array([int(r["bias"][0], 16), 0x3F80], dtype=np.uint16)
            got = oracle.add_bias(y, b, lib=lib)
            if int(got[0, 0]) != int(r["out"][0], 16) or int(got[0, 1]) != 0x3F80:
                return False
        return True

    def w8a16_hand():
        x = _bf16([1.0, 2.0, -0.5, 0.25])[None, :]
        q = np.array([[3, -1, 4, 8], [-127, 0, 127, 1]], dtype=np.int8)
        y, bound = oracle.w8a16(x, q, np.array([0.5, 2.0], dtype=np.float32), lib=lib)
        return y.tolist() == [[0.5, -380.5]] and bound.tolist() == [[4.5, 381.5]]

    def rms_torch_exact():
        # integer rows: exact sums in any order, so torch's F.rms_norm is matched bit for bit
        import torch.nn.functional as F
        g = synth.rng(77)
        x = _bf16(g.integers(-8, 9, size=(6, 256)).astype(np.float32).tolist())
        gain = _bf16(g.uniform(0.5, 1.5, size=256).astype(np.float32).tolist())
        r = oracle.rmsnorm_quantize(x, gain, lib=lib)
        xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
        gt = torch.from_numpy(gain.view(np.int16)).view(torch.bfloat16)
        want = F.rms_norm(xt, [256], gt).view(torch.int16).numpy().view(np.uint16)
        # small rows (x 2^-12, sums still exact): the mean is comparable to eps
        xs = _bf16((g.integers(-8, 9, size=(6, 256)) * 2.0 ** -12).astype(np.float32).tolist())
        rs = oracle.rmsnorm_quantize(xs, eps=1e-6, lib=lib)
        xst = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16)
        wants = F.rms_norm(xst, [256], None, 1e-6).view(torch.int16).numpy().view(np.uint16)
        return np.array_equal(r["xn"], want) and np.array_equal(rs["xn"], wants)

    def rms_tie_flagged():
        x = _bf16([[2.0, 0.0, 0.0, 2.0 ** -11]])
        r = oracle.rmsnorm_quantize(x, eps=0.0, lib=lib)
        return bool(r["ambiguous"][0]) and float(r["mean_alt"][0]) == 1.0 + 2.0 ** -23

    def rms_constant_row():
        r = oracle.rmsnorm_quantize(_bf16([[-3.0] * 64]), lib=lib)
        return bool(np.all(r["xn"] == 0xBF80)) and bool(np.all(r["q"] == -127))

    for name, fn in [("pack_golden", pack_golden), ("unpack_roundtrip", unpack_roundtrip),
                     ("rms_torch_exact", rms_torch_exact), ("rms_tie_flagged", rms_tie_flagged),
                     ("rms_constant_row", rms_constant_row),
                     ("quant_f32_golden", quant_f32_golden), ("bias_golden", bias_golden),
                     ("w8a16_hand", w8a16_hand),
                     ("quant_golden", quant_golden), ("quant_absmax", quant_absmax),
                     ("gemm_hand", gemm_hand), ("gemm_brute", gemm_brute), ("epi_golden", epi_golden), ("epi_batch", epi_batch),
                     ("linear_k8", linear_k8), ("linear_shape", linear_shape)]:
        check(name, fn)
    return failed


MUTANTS = [
    ("code_offset", "(unsigned)(W[n * K + 4 * j + i] + 2)", "(unsigned)(W[n * K + 4 * j + i] + 1)"),
    ("pack_bit_order", "byte |= code << (2 * i);", "byte |= code << (6 - 2 * i);"),
    ("decode_offset", "return code - 2;", "return code - 1;"),
    ("decode_bit_order", "(byte >> (2 * (k % 4))) & 3", "(byte >> (2 * (3 - k % 4))) & 3"),
    ("absmax_no_abs", "std::fabs(xf[k])", "(xf[k])"),
    ("scale_128", "const float s = a / 127.0f;", "const float s = a / 128.0f;"),
    ("eps_dropped", "if (a < eps) a = eps;", "(void)eps;"),
    ("round_half_away", "std::nearbyint(y)", "std::round(y)"),
    ("mul_by_reciprocal", "xf[k] / s;", "xf[k] * (127.0f / a);"),
    ("divide_by_bf16_scale", "xf[k] / s;", "xf[k] / oracle_f32_from_bf16(oracle_bf16_from_f32(s));"),
    ("scale_truncated", "*scale = oracle_bf16_from_f32(s);", "{ uint32_t u_; std::memcpy(&u_, &s, 4); *scale = (uint16_t)(u_ >> 16); }"),
    ("gemm_transposed_out", "acc[m * N + n] = (int32_t)s;", "acc[n * M + m] = (int32_t)s;"),
    ("gemm_dropped_term", "for (int64_t k = 0; k < K; ++k) s +=", "for (int64_t k = 1; k < K; ++k) s +="),
    ("epi_acc_sa_first", "const float y = (float)acc * scale;",
     "const float y = ((float)acc * oracle_f32_from_bf16(sa)) * oracle_f32_from_bf16(sw); (void)scale;"),
    ("epi_acc_sw_first", "const float y = (float)acc * scale;",
     "const float y = ((float)acc * oracle_f32_from_bf16(sw)) * oracle_f32_from_bf16(sa); (void)scale;"),
    ("bf16_round_half_up", "(lower == 0x8000u && (upper & 1u))", "(lower == 0x8000u)"),
    ("bf16_truncate", "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;", "(void)lower;"),
    ("epi_scale_index", "oracle_epilogue_one(acc[m * N + n], sa[m], sw[n])",
     "oracle_epilogue_one(acc[m * N + n], sa[m], sw[m])"),
    ("f32_via_bf16", "quantize_values(x, K, q, scale);  // the f32 values",
     "for (int64_t k = 0; k < K; ++k) ((float*)x)[k] = oracle_f32_from_bf16(oracle_bf16_from_f32(x[k]));\n    quantize_values(x, K, q, scale);  // the f32 values"),
    ("bf16_widen_wrong", "xf[k] = oracle_f32_from_bf16(x[k]);", "xf[k] = (float)(int16_t)x[k];"),
    ("bias_double_round", "const float y = oracle_f32_from_bf16(out[m * N + n]) + oracle_f32_from_bf16(bias[n]);",
     "const float y = oracle_f32_from_bf16(oracle_bf16_from_f32(oracle_f32_from_bf16(out[m * N + n]) + oracle_f32_from_bf16(bias[n]) * 0.5f)) + oracle_f32_from_bf16(bias[n]) * 0.5f;"),
    ("bias_row_index", "oracle_f32_from_bf16(bias[n])", "oracle_f32_from_bf16(bias[m])"),
    ("w8a16_scale_index", "y[m * N + n] = s * (double)scale[n];", "y[m * N + n] = s * (double)scale[0];"),
    ("w8a16_dropped_term", "for (int64_t k = 0; k < K; ++k) {\n                const double t",
     "for (int64_t k = 1; k < K; ++k) {\n                const double t"),
    ("w8a16_abs_bound", "a += std::fabs(t);", "a += t;"),
    ("rms_eps_after_sqrt", "const float v = mean + eps;\n    const float sd = std::sqrt(v);",
     "const float v = mean;\n    const float sd = std::sqrt(v) + eps;"),
    ("rms_sum_not_mean", "const double m64 = S / (double)K;", "const double m64 = S;"),
    ("rms_gain_after_round", "if (gain) t = t * oracle_f32_from_bf16(gain[k]);",
     "if (gain) t = oracle_f32_from_bf16(oracle_bf16_from_f32(t)) * oracle_f32_from_bf16(gain[k]);"),
    ("rms_gain_index", "oracle_f32_from_bf16(gain[k])", "oracle_f32_from_bf16(gain[0])"),
    ("rms_no_inverse", "const float r = 1.0f / sd;", "const float r = sd;"),
    ("rms_signed_square", "S += v * v;  // exact product", "S += v * std::fabs(v);  // exact product"),
    ("rms_no_margin", "const double delta = (2.0 * (double)(K - 1) + 4.0) * std::ldexp(1.0, -53) * 1.01;",
     "const double delta = 0.0;"),
]


def test_real_oracle_passes_battery():
    assert _pin_battery(oracle.load()) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/not found"
    mpath = os.path.join(tmp_path, f"m_{name}.cpp")
    with open(mpath, "w") as f:
        f.write(src.replace(old, new))
    so = obuild.build(src=mpath, out=os.path.join(tmp_path, f"m_{name}.so"), extra_flags=["-w"])
    lib = oracle.load(so)
    failed = _pin_battery(lib)
    assert failed, f"mutant {name} passed every pin"
