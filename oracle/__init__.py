"""CPU oracle of the W1.58A8 (ternary weight x INT8 activation) linear layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP library never
imports, links or calls it, and it shares no code with the library.

The arithmetic lives in bitnet_oracle.cpp (plain scalar C++); this module only
loads that library with ctypes and marshals numpy arrays.  bf16 values are
passed as their uint16 bit patterns.

Parity status of each function (what pins it is listed in the tests):
  pack / unpack / weight decode   pinned (closed-form bytes, exhaustive round trip)
  quantize                        pinned (hand-worked vectors, absmax -> +-127,
                                  double-division identity, reading discriminators)
  gemm_i32                        pinned (hand-worked K=4/K=8, brute force, closed forms)
  epilogue                        pinned (exact-product identity, tie cases)
  linear / linear_one             pinned through the three above and by composition
  quantize_f32 / linear_f32       pinned (hand-worked f32 vector; equal to the bf16 path on
                                  bf16-representable inputs; composition)
  add_bias                        pinned (hand-worked round-to-even ties; zero bias; zero rows)
  rmsnorm_quantize / linear_rms   pinned (bit-equal to torch's F.rms_norm on rows whose sums are exact;
                                  closed forms: constant rows, zero rows; sign, power-of-two scale
                                  and gain symmetries; the ambiguity flag on constructed ties)
  w8a16                           pinned (hand-worked example; zero weights; power-of-two scaling and
                                  sign symmetry; brute force against an exact rational sum)
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def load(path=None):
    """Load the compiled oracle (compiling it first if it has never been built)."""
    global _LIB
    if path is None and _LIB is not None:
        return _LIB
    lib_path = path or _build.LIB
    if not os.path.exists(lib_path):
        _build.build()
    lib = ctypes.CDLL(lib_path)
    lib.oracle_pack.argtypes = [_p, _i64, _i64, _p]
    lib.oracle_pack.restype = ctypes.c_int
    lib.oracle_weight_at.argtypes = [_p, _i64, _i64, _i64]
    lib.oracle_weight_at.restype = ctypes.c_int
    lib.oracle_unpack.argtypes = [_p, _i64, _i64, _p]
    lib.oracle_unpack.restype = None
    lib.oracle_f32_from_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_f32_from_bf16.restype = ctypes.c_float
    lib.oracle_bf16_from_f32.argtypes = [ctypes.c_float]
    lib.oracle_bf16_from_f32.restype = ctypes.c_uint16
    lib.oracle_quantize_row.argtypes = [_p, _i64, _p, _p]
    lib.oracle_quantize_row.restype = None
    lib.oracle_quantize.argtypes = [_p, _i64, _i64, _p, _p]
    lib.oracle_quantize.restype = ctypes.c_int
    lib.oracle_quantize_f32.argtypes = [_p, _i64, _i64, _p, _p]
    lib.oracle_quantize_f32.restype = ctypes.c_int
    lib.oracle_add_bias.argtypes = [_p, _p, _i64, _i64]
    lib.oracle_add_bias.restype = None
    lib.oracle_linear_f32.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p]
    lib.oracle_linear_f32.restype = ctypes.c_int
    lib.oracle_w8a16.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p]
    lib.oracle_rmsnorm_quantize.argtypes = [_p, _p, ctypes.c_float, _i64, _i64, _p, _p, _p, _p, _p, _p]
    lib.oracle_rmsnorm_quantize.restype = ctypes.c_int
    lib.oracle_w8a16.restype = None
    lib.oracle_dot_i64.argtypes = [_p, _p, _i64, _i64]
    lib.oracle_dot_i64.restype = ctypes.c_int64
    lib.oracle_gemm_i32.argtypes = [_p, _p, _i64, _i64, _i64, _p]
    lib.oracle_gemm_i32.restype = ctypes.c_int
    lib.oracle_epilogue_one.argtypes = [ctypes.c_int32, ctypes.c_uint16, ctypes.c_uint16]
    lib.oracle_epilogue_one.restype = ctypes.c_uint16
    lib.oracle_epilogue.argtypes = [_p, _p, _p, _i64, _i64, _p]
    lib.oracle_epilogue.restype = None
    lib.oracle_linear.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p]
    lib.oracle_linear.restype = ctypes.c_int
    lib.oracle_linear_one.argtypes = [_p, ctypes.c_uint16, _p, _p, _i64, _i64, _p]
    lib.oracle_linear_one.restype = ctypes.c_uint16
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    if path is None:
        _LIB = lib
    return lib


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: oracle status {rc}")


def num_threads():
    return load().oracle_num_threads()


def set_num_threads(n):
    load().oracle_set_num_threads(int(n))


def bf16_from_f32(x):
    return int(load().oracle_bf16_from_f32(float(x)))


def f32_from_bf16(h):
    return float(load().oracle_f32_from_bf16(int(h)))


def pack(W, lib=None):
    """int8 W[N,K] in {-1,0,1} -> uint8 P[N,K/4]."""
    lib = lib or load()
    W = np.ascontiguousarray(W, dtype=np.int8)
    N, K = W.shape
    P = np.zeros((N, K // 4 if K % 4 == 0 else 0), dtype=np.uint8)
    _check(lib.oracle_pack(_ptr(W), N, K, _ptr(P)), "pack")
    return P


def unpack(P, K, lib=None):
    lib = lib or load()
    P = np.ascontiguousarray(P, dtype=np.uint8)
    N = P.shape[0]
    W = np.zeros((N, K), dtype=np.int8)
    lib.oracle_unpack(_ptr(P), N, K, _ptr(W))
    return W


def quantize(x_bits, lib=None):
    """bf16 bits x[M,K] (uint16) -> (int8 q[M,K], uint16 bf16 scale_act[M])."""
    lib = lib or load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, K = x.shape
    q = np.zeros((M, K), dtype=np.int8)
    sa = np.zeros((M,), dtype=np.uint16)
    _check(lib.oracle_quantize(_ptr(x), M, K, _ptr(q), _ptr(sa)), "quantize")
    return q, sa


def gemm_i32(q, P, lib=None):
    """int8 q[M,K] x packed P[N,K/4] -> int32 acc[M,N]."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    P = np.ascontiguousarray(P, dtype=np.uint8)
    M, K = q.shape
    N = P.shape[0]
    acc = np.zeros((M, N), dtype=np.int32)
    _check(lib.oracle_gemm_i32(_ptr(q), _ptr(P), M, N, K, _ptr(acc)), "gemm_i32")
    return acc


def epilogue(acc, sa, sw, lib=None):
    """int32 acc[M,N], bf16 bits sa[M], sw[N] -> bf16 bits out[M,N]."""
    lib = lib or load()
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    sa = np.ascontiguousarray(sa, dtype=np.uint16)
    sw = np.ascontiguousarray(sw, dtype=np.uint16)
    M, N = acc.shape
    out = np.zeros((M, N), dtype=np.uint16)
    lib.oracle_epilogue(_ptr(acc), _ptr(sa), _ptr(sw), M, N, _ptr(out))
    return out


def epilogue_one(acc, sa, sw, lib=None):
    lib = lib or load()
    return int(lib.oracle_epilogue_one(int(acc), int(sa), int(sw)))


def linear(x_bits, P, sw, lib=None):
    """Whole layer.  Returns dict(out, q, scale_act, acc)."""
    lib = lib or load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    P = np.ascontiguousarray(P, dtype=np.uint8)
    sw = np.ascontiguousarray(sw, dtype=np.uint16)
    M, K = x.shape
    N = P.shape[0]
    out = np.zeros((M, N), dtype=np.uint16)
    q = np.zeros((M, K), dtype=np.int8)
    sa = np.zeros((M,), dtype=np.uint16)
    acc = np.zeros((M, N), dtype=np.int32)
    _check(lib.oracle_linear(_ptr(x), _ptr(P), _ptr(sw), M, N, K, _ptr(out), _ptr(q), _ptr(sa), _ptr(acc)),
           "linear")
    return {"out": out, "q": q, "scale_act": sa, "acc": acc}


def linear_one(q_row, sa, P, sw, n, lib=None):
    """One output element from a quantised row: returns (bf16 bits, int32 acc)."""
    lib = lib or load()
    q_row = np.ascontiguousarray(q_row, dtype=np.int8)
    P = np.ascontiguousarray(P, dtype=np.uint8)
    sw = np.ascontiguousarray(sw, dtype=np.uint16)
    acc = ctypes.c_int32(0)
    K = q_row.shape[0]
    out = lib.oracle_linear_one(_ptr(q_row), int(sa), _ptr(P), _ptr(sw), K, int(n), ctypes.byref(acc))
    return int(out), int(acc.value)


def quantize_f32(x, lib=None):
    """float32 x[M,K] -> (int8 q[M,K], uint16 bf16 scale_act[M])."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    q = np.zeros((M, K), dtype=np.int8)
    sa = np.zeros((M,), dtype=np.uint16)
    _check(lib.oracle_quantize_f32(_ptr(x), M, K, _ptr(q), _ptr(sa)), "quantize_f32")
    return q, sa


def add_bias(out_bits, bias_bits, lib=None):
    """bf16 bits out[M,N] + bf16 bits bias[N] -> new bf16 bits array."""
    lib = lib or load()
    out = np.array(out_bits, dtype=np.uint16, copy=True, order="C")
    bias = np.ascontiguousarray(bias_bits, dtype=np.uint16)
    M, N = out.shape
    lib.oracle_add_bias(_ptr(out), _ptr(bias), M, N)
    return out


def linear_f32(x, P, sw, lib=None):
    """Whole layer on float32 activations.  Returns dict(out, q, scale_act, acc)."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    P = np.ascontiguousarray(P, dtype=np.uint8)
    sw = np.ascontiguousarray(sw, dtype=np.uint16)
    M, K = x.shape
    N = P.shape[0]
    out = np.zeros((M, N), dtype=np.uint16)
    q = np.zeros((M, K), dtype=np.int8)
    sa = np.zeros((M,), dtype=np.uint16)
    acc = np.zeros((M, N), dtype=np.int32)
    _check(lib.oracle_linear_f32(_ptr(x), _ptr(P), _ptr(sw), M, N, K, _ptr(out), _ptr(q), _ptr(sa), _ptr(acc)),
           "linear_f32")
    return {"out": out, "q": q, "scale_act": sa, "acc": acc}


def w8a16(x_bits, q, scale, lib=None):
    """INT8 weight-only matmul: bf16 bits x[M,K], int8 q[N,K], float32 scale[N] ->
    (float64 y[M,N], float64 bound[M,N] = sum_k |x*q| * |scale|)."""
    lib = lib or load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    q = np.ascontiguousarray(q, dtype=np.int8)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    M, K = x.shape
    N = q.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    bound = np.zeros((M, N), dtype=np.float64)
    lib.oracle_w8a16(_ptr(x), _ptr(q), _ptr(scale), M, N, K, _ptr(y), _ptr(bound))
    return y, bound


FP32_EPS = 2.0 ** -23   # torch's default rms_norm eps for bf16 and f32 input


def rmsnorm_quantize(x_bits, gain_bits=None, eps=FP32_EPS, means=None, lib=None):
    """RMSNorm then per-token quantisation: bf16 bits x[M,K], optional bf16 gain[K].

    Returns a dict with xn (bf16 bits), q, scale_act, mean (fp32 per row),
    mean_alt (the other fp32 mean a different summation order could give;
    equal to mean when the row is unambiguous) and ambiguous (bool per row).
    means (fp32 [M]) forces the mean used for every row."""
    lib = lib or load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, K = x.shape
    g = None if gain_bits is None else np.ascontiguousarray(gain_bits, dtype=np.uint16)
    mi = None if means is None else np.ascontiguousarray(means, dtype=np.float32)
    xn = np.zeros((M, K), dtype=np.uint16)
    q = np.zeros((M, K), dtype=np.int8)
    sa = np.zeros(M, dtype=np.uint16)
    mean = np.zeros(M, dtype=np.float32)
    alt = np.zeros(M, dtype=np.float32)
    _check(lib.oracle_rmsnorm_quantize(_ptr(x), None if g is None else _ptr(g), ctypes.c_float(eps), M, K,
                                       None if mi is None else _ptr(mi), _ptr(xn), _ptr(q), _ptr(sa), _ptr(mean),
                                       _ptr(alt)), "oracle_rmsnorm_quantize")
    return {"xn": xn, "q": q, "scale_act": sa, "mean": mean, "mean_alt": alt, "ambiguous": mean != alt}


def linear_rms(x_bits, P, sw, gain_bits=None, eps=FP32_EPS, means=None, lib=None):
    """RMSNorm, quantise, ternary contraction, epilogue: bf16 bits out[M,N] and the intermediates."""
    r = rmsnorm_quantize(x_bits, gain_bits, eps, means, lib)
    acc = gemm_i32(r["q"], P, lib)
    r["acc"] = acc
    r["out"] = epilogue(acc, r["scale_act"], sw, lib)
    return r
