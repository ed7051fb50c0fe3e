// bitnet_oracle.cpp -- the CPU oracle for the W1.58A8 linear layer.
//
// TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
// statement of what the ternary x INT8 linear layer computes.  Only the test
// suite, the package's smoke check and the benchmark's CPU-baseline leg may
// load it.  It shares no code, header, table or helper with the HIP library
// under ternary_int8_gemm_amd/, and the library never calls it.
//
// Every step is written as the plain definition from the pages:
//
//   * "phanerozoic/bitnet-cpu v1, torch-ext/bitnet_cpu/__init__.py"
//       - function pack_weights        -> oracle_pack / oracle_unpack
//       - function quantize_activation -> oracle_quantize_row
//       - functions bitnet_gemm, bitnet_gemv_fused, bitnet_linear
//                                     -> oracle_gemm_i32, oracle_epilogue,
//                                        oracle_linear
//   * "kernels-community/README discussion #1 (bitnet-tc kernel request)",
//       numbers post: the product accumulates in int32.
//       - f32 activations (accepted by quantize_activation, bitnet_gemv_fused
//         and bitnet_linear)       -> oracle_quantize_row_f32, oracle_linear_f32
//       - class BitLinear, the bias added to the layer's output
//                                     -> oracle_add_bias
//   * "CoolDip00/tiny-llm src/tinyllm/kernels/int8_gemv.py", the W8A16 decode
//       matmul                     -> oracle_w8a16
//   * "kyegomez/BitNet issue #77", activation_norm_quant (RMSNorm, then the
//       per-token quantisation; a fused kernel is suggested there), and
//       bitnet-cpu's BitLinearKernel (its rms_norm module runs before
//       bitnet_linear)              -> oracle_rmsnorm_row, oracle_rmsnorm_quantize
//   * "CoolDip00/tiny-llm src/tinyllm/kernels/int8_gemv.py", docstring of
//       int8_matmul: the integer/matmul result is scaled without an
//       intermediate rounding to bf16.
//
// Readings taken where the pages leave a step open (each is listed with its
// reason in the design notes of the repository):
//   R1  the quantiser works in fp32 on the widened bf16 input (the f32 branch
//       of quantize_activation), not in bf16 arithmetic;
//   R2  q = round_half_even(fp32(x / s)) with s = fp32(absmax / 127), the
//       division done in IEEE fp32 (not a multiply by 127/absmax);
//   R3  scale_act is the bf16 round-to-nearest-even of the fp32 s, and s (not
//       its bf16 image) is what x is divided by;
//   R4  a 2-bit code of 0 (never produced by packing) decodes to -2, i.e. the
//       decode is w = code - 2 for every code;
//   R5  epilogue: out = bf16_rne( fp32( (float)acc * fp32( (float)sa * (float)sw ) ) ),
//       one fp32 product of the two scales (exact for bf16 inputs), one fp32
//       product with the exact (float)acc, then one bf16 rounding;
//   R6  the fused (M < 16) path and the split path compute the same thing, so
//       both are oracle_linear.
//
// Build: plain C++17 with the host compiler, no fast-math, no FP contraction.
// OpenMP is used only to run independent output rows on several host threads;
// it changes no arithmetic (each output is computed by one thread in order).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <cstdlib>
#ifdef _OPENMP
#include <omp.h>
#endif

extern "C" {

// Status codes of the oracle (its own; unrelated to the library's).
enum { ORC_OK = 0, ORC_ERR_SHAPE = 1, ORC_ERR_VALUE = 2, ORC_ERR_OVERFLOW = 3 };

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  A bf16 value is the top 16 bits of an IEEE binary32.
// Widening is exact.  Narrowing rounds to nearest, ties to even, on the
// discarded 16 bits (NaN inputs are outside the contract and are not used).
// ---------------------------------------------------------------------------
float oracle_f32_from_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_bf16_from_f32(float f) {
    uint32_t u;
    std::memcpy(&u, &f, sizeof u);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xFFFFu;
    // Round to nearest; on an exact tie (lower == 0x8000) round to the even upper.
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

// ---------------------------------------------------------------------------
// Packing (bitnet-cpu, pack_weights).  W is [N][K] int8 in {-1,0,+1}, K a
// multiple of 4.  Code c = w + 2 (so -1 -> 1, 0 -> 2, +1 -> 3).  Four codes go
// in one byte, the element with the lowest k in the two lowest bits:
//   P[n][j] = c(4j) | c(4j+1) << 2 | c(4j+2) << 4 | c(4j+3) << 6.
// Output P is [N][K/4] uint8.
// ---------------------------------------------------------------------------
int oracle_pack(const int8_t* W, int64_t N, int64_t K, uint8_t* P) {
    if (N < 0 || K < 0 || K % 4 != 0) return ORC_ERR_SHAPE;
    for (int64_t i = 0; i < N * K; ++i)
        if (W[i] < -1 || W[i] > 1) return ORC_ERR_VALUE;
    const int64_t KB = K / 4;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < KB; ++j) {
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i) {
                unsigned code = (unsigned)(W[n * K + 4 * j + i] + 2);
                byte |= code << (2 * i);
            }
            P[n * KB + j] = (uint8_t)byte;
        }
    }
    return ORC_OK;
}

// Decode of one weight: w = code - 2 where code is the 2-bit field holding
// element k (reading R4: a code of 0 gives -2).
int oracle_weight_at(const uint8_t* P, int64_t K, int64_t n, int64_t k) {
    const uint8_t byte = P[n * (K / 4) + k / 4];
    const int code = (byte >> (2 * (k % 4))) & 3;
    return code - 2;
}

void oracle_unpack(const uint8_t* P, int64_t N, int64_t K, int8_t* W) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            W[n * K + k] = (int8_t)oracle_weight_at(P, K, n, k);
}

// ---------------------------------------------------------------------------
// Per-token absmax INT8 quantisation (bitnet-cpu, quantize_activation, with
// readings R1-R3).  For one row x[0..K) of bf16 values:
//   xf    = (float) x                              (exact widening)
//   a     = max_k |xf[k]|, then a = max(a, 1e-5f)   (eps clamp from below)
//   s     = a / 127.0f                              (IEEE fp32 division)
//   q[k]  = clamp(round_half_even(xf[k] / s), -127, 127) as int8
//   scale = bf16_rne(s)
// ---------------------------------------------------------------------------
// One row of per-token absmax quantisation on fp32 values xf[0..K).
static void quantize_values(const float* xf, int64_t K, int8_t* q, uint16_t* scale) {
    float a = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        const float v = std::fabs(xf[k]);
        if (v > a) a = v;
    }
    const float eps = 1e-5f;
    if (a < eps) a = eps;
    const float s = a / 127.0f;
    for (int64_t k = 0; k < K; ++k) {
        const float y = xf[k] / s;
        float r = std::nearbyint(y);  // default rounding mode: to nearest, ties to even
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[k] = (int8_t)r;
    }
    *scale = oracle_bf16_from_f32(s);
}

// bf16 activations: widened exactly to fp32, then quantised.
void oracle_quantize_row(const uint16_t* x, int64_t K, int8_t* q, uint16_t* scale) {
    float* xf = (float*)std::malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
    for (int64_t k = 0; k < K; ++k) xf[k] = oracle_f32_from_bf16(x[k]);
    quantize_values(xf, K, q, scale);
    std::free(xf);
}

int oracle_quantize(const uint16_t* x, int64_t M, int64_t K, int8_t* q, uint16_t* scale) {
    if (M < 0 || K <= 0) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) oracle_quantize_row(x + m * K, K, q + m * K, scale + m);
    return ORC_OK;
}

// ---------------------------------------------------------------------------
// The ternary x int8 contraction (bitnet-cpu, bitnet_gemm; the int32
// accumulation of the bitnet-tc numbers post):
//   acc[m][n] = sum_k w[n][k] * q[m][k]
// summed exactly in int64, then required to fit in int32.
// ---------------------------------------------------------------------------
int64_t oracle_dot_i64(const int8_t* q_row, const uint8_t* P, int64_t K, int64_t n) {
    int64_t s = 0;
    for (int64_t k = 0; k < K; ++k) s += (int64_t)oracle_weight_at(P, K, n, k) * (int64_t)q_row[k];
    return s;
}

int oracle_gemm_i32(const int8_t* q, const uint8_t* P, int64_t M, int64_t N, int64_t K, int32_t* acc) {
    if (M < 0 || N < 0 || K <= 0 || K % 4 != 0) return ORC_ERR_SHAPE;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            const int64_t s = oracle_dot_i64(q + m * K, P, K, n);
            if (s > INT32_MAX || s < INT32_MIN) bad = 1;
            acc[m * N + n] = (int32_t)s;
        }
    }
    return bad ? ORC_ERR_OVERFLOW : ORC_OK;
}

// ---------------------------------------------------------------------------
// Epilogue (reading R5).  The two bf16 scales are widened and multiplied in
// fp32 first, then the widened accumulator is multiplied by that product in
// fp32, then the fp32 result is rounded to bf16.
// ---------------------------------------------------------------------------
uint16_t oracle_epilogue_one(int32_t acc, uint16_t sa, uint16_t sw) {
    const float scale = oracle_f32_from_bf16(sa) * oracle_f32_from_bf16(sw);
    const float y = (float)acc * scale;
    return oracle_bf16_from_f32(y);
}

void oracle_epilogue(const int32_t* acc, const uint16_t* sa, const uint16_t* sw, int64_t M, int64_t N,
                     uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) out[m * N + n] = oracle_epilogue_one(acc[m * N + n], sa[m], sw[n]);
}

// ---------------------------------------------------------------------------
// INT8 weight-only decode matmul (W8A16), as in "CoolDip00/tiny-llm,
// src/tinyllm/kernels/int8_gemv.py" (docstring of the module and of
// int8_matmul): y[m][n] = scale[n] * sum_k x[m][k] * q[n][k], with bf16 x,
// int8 q, fp32 scale, fp32 y.  The kernel accumulates in fp32 in an order of
// its own, so the oracle gives the reference value in double (every product
// x * q is exact in double, and so is the sum while it stays within 53 bits of
// its smallest term) together with sum_k |x * q| * |scale|, from which the
// tests bound the fp32 rounding of any summation order.
// ---------------------------------------------------------------------------
void oracle_w8a16(const uint16_t* x, const int8_t* q, const float* scale, int64_t M, int64_t N, int64_t K,
                  double* y, double* absbound) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double s = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double t = (double)oracle_f32_from_bf16(x[m * K + k]) * (double)q[n * K + k];
                s += t;
                a += std::fabs(t);
            }
            y[m * N + n] = s * (double)scale[n];
            absbound[m * N + n] = a * std::fabs((double)scale[n]);
        }
    }
}

// ---------------------------------------------------------------------------
// f32 activations.  bitnet-cpu's quantize_activation, bitnet_gemv_fused and
// bitnet_linear accept x in bf16 or f32; for f32 the same per-token absmax
// quantisation runs on the f32 values themselves (no rounding to bf16 first).
// ---------------------------------------------------------------------------
void oracle_quantize_row_f32(const float* x, int64_t K, int8_t* q, uint16_t* scale) {
    quantize_values(x, K, q, scale);  // the f32 values themselves, no rounding to bf16
}

int oracle_quantize_f32(const float* x, int64_t M, int64_t K, int8_t* q, uint16_t* scale) {
    if (M < 0 || K <= 0) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) oracle_quantize_row_f32(x + m * K, K, q + m * K, scale + m);
    return ORC_OK;
}

// Bias, as bitnet-cpu's BitLinear applies it: the layer's bf16 output y plus a
// bf16 bias per output column, added in fp32 and rounded to bf16 once:
//   out[m][n] = bf16_rne( fp32(y[m][n]) + fp32(bias[n]) ).
void oracle_add_bias(uint16_t* out, const uint16_t* bias, int64_t M, int64_t N) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            const float y = oracle_f32_from_bf16(out[m * N + n]) + oracle_f32_from_bf16(bias[n]);
            out[m * N + n] = oracle_bf16_from_f32(y);
        }
}

// ---------------------------------------------------------------------------
// RMSNorm before the quantisation ("kyegomez/BitNet issue #77",
// activation_norm_quant: F.rms_norm over the last dimension, then the int8
// quantisation; bitnet-cpu's BitLinearKernel applies its rms_norm module the
// same way before bitnet_linear).  Reading R22, torch's rms_norm on bf16 input,
// computed in fp32:
//   mean = fp32( sum_k x_k^2 / K )
//   r    = fp32( 1 / fp32( sqrt( fp32(mean + eps) ) ) )
//   xn_k = bf16_rne( fp32( fp32(x_k * r) * g_k ) )     (no multiply without a gain)
// with eps given in fp32 (torch's default is the fp32 epsilon, 2^-23).  Every
// square of a bf16 value is exact in double; the sum is taken in double, so an
// implementation may add the squares in any order.  Different orders can round
// the double sum differently, and in rare rows that moves the fp32 mean by one
// step: the oracle then returns both fp32 candidates (mean_out, mean_alt_out;
// equal when the row is unambiguous), and mean_in (when given) forces the mean
// used, so that each candidate's result can be formed.
// ---------------------------------------------------------------------------
void oracle_rmsnorm_row(const uint16_t* x, const uint16_t* gain, float eps, int64_t K, const float* mean_in,
                        uint16_t* xn, float* mean_out, float* mean_alt_out) {
    double S = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const double v = (double)oracle_f32_from_bf16(x[k]);
        S += v * v;  // exact product
    }
    const double m64 = S / (double)K;
    // Any summation order of K non-negative terms lies within (K - 1) * 2^-53
    // (relative, to first order) of the exact sum, as does this one; with the
    // division's rounding, an implementation's double mean lies within
    // delta of m64 (relative).
    const double delta = (2.0 * (double)(K - 1) + 4.0) * std::ldexp(1.0, -53) * 1.01;
    const float lo = (float)(m64 * (1.0 - delta));
    const float hi = (float)(m64 * (1.0 + delta));
    float mean = (float)m64;
    float alt = (lo != mean) ? lo : hi;
    if (mean_in) {
        mean = *mean_in;
        alt = mean;
    }
    if (mean_out) *mean_out = mean;
    if (mean_alt_out) *mean_alt_out = alt;
    const float v = mean + eps;
    const float sd = std::sqrt(v);
    const float r = 1.0f / sd;
    for (int64_t k = 0; k < K; ++k) {
        float t = oracle_f32_from_bf16(x[k]) * r;
        if (gain) t = t * oracle_f32_from_bf16(gain[k]);
        xn[k] = oracle_bf16_from_f32(t);
    }
}

// RMSNorm then quantise, row by row.  xn (bf16, [M][K]) receives the
// normalised activations the quantiser sees; mean_in may be NULL.
int oracle_rmsnorm_quantize(const uint16_t* x, const uint16_t* gain, float eps, int64_t M, int64_t K,
                            const float* mean_in, uint16_t* xn, int8_t* q, uint16_t* scale, float* mean_out,
                            float* mean_alt_out) {
    if (M < 0 || K <= 0) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        oracle_rmsnorm_row(x + m * K, gain, eps, K, mean_in ? mean_in + m : nullptr, xn + m * K, mean_out + m,
                           mean_alt_out + m);
        oracle_quantize_row(xn + m * K, K, q + m * K, scale + m);
    }
    return ORC_OK;
}

// ---------------------------------------------------------------------------
// The whole layer (bitnet-cpu, bitnet_linear and bitnet_gemv_fused; reading
// R6): quantise each row, contract, scale.  Fills q/scale_act/acc when the
// caller passes buffers for them (NULL to skip).
// ---------------------------------------------------------------------------
int oracle_linear(const uint16_t* x, const uint8_t* P, const uint16_t* sw, int64_t M, int64_t N, int64_t K,
                  uint16_t* out, int8_t* q_out, uint16_t* sa_out, int32_t* acc_out) {
    if (M < 0 || N < 0 || K <= 0 || K % 4 != 0) return ORC_ERR_SHAPE;
    int8_t* q = q_out ? q_out : (int8_t*)std::malloc((size_t)(M * K > 0 ? M * K : 1));
    uint16_t* sa = sa_out ? sa_out : (uint16_t*)std::malloc((size_t)(M > 0 ? M : 1) * sizeof(uint16_t));
    int32_t* acc = acc_out ? acc_out : (int32_t*)std::malloc((size_t)(M * N > 0 ? M * N : 1) * sizeof(int32_t));
    int rc = oracle_quantize(x, M, K, q, sa);
    if (rc == ORC_OK) rc = oracle_gemm_i32(q, P, M, N, K, acc);
    if (rc == ORC_OK) oracle_epilogue(acc, sa, sw, M, N, out);
    if (!q_out) std::free(q);
    if (!sa_out) std::free(sa);
    if (!acc_out) std::free(acc);
    return rc;
}

// The whole layer on f32 activations: quantise (f32), contract, scale.
int oracle_linear_f32(const float* x, const uint8_t* P, const uint16_t* sw, int64_t M, int64_t N, int64_t K,
                      uint16_t* out, int8_t* q_out, uint16_t* sa_out, int32_t* acc_out) {
    if (M < 0 || N < 0 || K <= 0 || K % 4 != 0) return ORC_ERR_SHAPE;
    int8_t* q = q_out ? q_out : (int8_t*)std::malloc((size_t)(M * K > 0 ? M * K : 1));
    uint16_t* sa = sa_out ? sa_out : (uint16_t*)std::malloc((size_t)(M > 0 ? M : 1) * sizeof(uint16_t));
    int32_t* acc = acc_out ? acc_out : (int32_t*)std::malloc((size_t)(M * N > 0 ? M * N : 1) * sizeof(int32_t));
    int rc = oracle_quantize_f32(x, M, K, q, sa);
    if (rc == ORC_OK) rc = oracle_gemm_i32(q, P, M, N, K, acc);
    if (rc == ORC_OK) oracle_epilogue(acc, sa, sw, M, N, out);
    if (!q_out) std::free(q);
    if (!sa_out) std::free(sa);
    if (!acc_out) std::free(acc);
    return rc;
}

// One output element of the layer from an already quantised row: used to
// check sampled outputs of full-size problems one by one.
uint16_t oracle_linear_one(const int8_t* q_row, uint16_t sa, const uint8_t* P, const uint16_t* sw, int64_t K,
                           int64_t n, int32_t* acc_out) {
    const int64_t s = oracle_dot_i64(q_row, P, K, n);
    if (acc_out) *acc_out = (int32_t)s;
    return oracle_epilogue_one((int32_t)s, sa, sw[n]);
}

}  // extern "C"
