// bitnet_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Everything here is written for CDNA4 (gfx950, wave64): DPP lane exchanges,
// v_dot4 integer dot products, v_cvt_pk_bf16_f32 rounding, and the exact
// per-token quantisation of "phanerozoic/bitnet-cpu v1,
// torch-ext/bitnet_cpu/__init__.py" (function quantize_activation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnet {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// 16-byte streaming load (nontemporal hint: data used once, keep it out of the caches' way).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ----------------------------------------------------------------- bf16

// bf16 bit pattern (low 16 bits of h) -> fp32, exact.
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __builtin_bit_cast(float, h << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (v_cvt_pk_bf16_f32 under the
// default round-to-nearest-even mode).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// ----------------------------------------------------------------- DPP

template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int DPP_ROW_MIRROR = 0x140;       // lane i <-> 15-i within each 16 lanes

// Sum over each aligned group of 8 lanes; every lane of the group gets the total.
__device__ __forceinline__ int group8_sum(int v) {
    v += dpp_mov<DPP_QUAD_XOR1>(v);
    v += dpp_mov<DPP_QUAD_XOR2>(v);
    v += dpp_mov<DPP_ROW_HALF_MIRROR>(v);
    return v;
}

// Maximum over each aligned group of 16 lanes (unsigned); every lane gets it.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = max(v, (uint32_t)dpp_mov<DPP_QUAD_XOR1>((int)v));
    v = max(v, (uint32_t)dpp_mov<DPP_QUAD_XOR2>((int)v));
    v = max(v, (uint32_t)dpp_mov<DPP_ROW_HALF_MIRROR>((int)v));
    v = max(v, (uint32_t)dpp_mov<DPP_ROW_MIRROR>((int)v));
    return v;
}

// Maximum over the whole wave; the result is wave-uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = row16_max_u32(v);
    uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

// Sum over the whole wave; the result is wave-uniform.
__device__ __forceinline__ int wave_sum_i32(int v) {
    v += dpp_mov<DPP_QUAD_XOR1>(v);
    v += dpp_mov<DPP_QUAD_XOR2>(v);
    v += dpp_mov<DPP_ROW_HALF_MIRROR>(v);
    v += dpp_mov<DPP_ROW_MIRROR>(v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
           __builtin_amdgcn_readlane(v, 48);
}

template <int CTRL>
__device__ __forceinline__ double dpp_mov_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)dpp_mov<CTRL>((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)dpp_mov<CTRL>((int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the whole wave in double, in a fixed order; the result is wave-uniform.
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_mov_f64<DPP_QUAD_XOR1>(v);
    v += dpp_mov_f64<DPP_QUAD_XOR2>(v);
    v += dpp_mov_f64<DPP_ROW_HALF_MIRROR>(v);
    v += dpp_mov_f64<DPP_ROW_MIRROR>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// ----------------------------------------------------------------- RMSNorm
//
// RMSNorm before the quantisation (F.rms_norm over the row, as the BitNet
// activation_norm_quant function of "kyegomez/BitNet issue #77" applies it),
// computed as torch computes it on bf16 input, in fp32:
//   mean = fp32( sum_k x_k^2 / K )     (squares exact, summed in double)
//   r    = fp32( 1 / fp32( sqrt( fp32(mean + eps) ) ) )
//   xn_k = bf16_rne( fp32( fp32(x_k * r) * g_k ) )
// The square root and the division are the correctly rounded IEEE operations
// (hipcc's default lowering of sqrtf and of '/').

__device__ __forceinline__ float rms_inv(double sum_sq, int K, float eps) {
    const float mean = (float)(sum_sq / (double)K);
    const float v = mean + eps;
    return 1.0f / __builtin_sqrtf(v);
}

// Sum of the squares of the eight bf16 values of a 16-byte group, in double,
// as a tree (each square is exact in double; the order of the additions is
// free within the bound the oracle allows for any order).
__device__ __forceinline__ double sum_sq_bf16x8(const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    double p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double a = (double)bf16_to_f32(w[i] & 0xFFFFu);
        const double b = (double)bf16_to_f32(w[i] >> 16);
        p[i] = a * a + b * b;
    }
    return (p[0] + p[1]) + (p[2] + p[3]);
}

// Two normalised bf16 values from two bf16 inputs and their two bf16 gains.
__device__ __forceinline__ uint32_t rms_apply_bf16x2(uint32_t xw, uint32_t gw, float r) {
    const float t0 = (bf16_to_f32(xw & 0xFFFFu) * r) * bf16_to_f32(gw & 0xFFFFu);
    const float t1 = (bf16_to_f32(xw >> 16) * r) * bf16_to_f32(gw >> 16);
    return (uint32_t)f32_to_bf16(t0) | ((uint32_t)f32_to_bf16(t1) << 16);
}

// The same without a gain: bf16(fp32(x * r)), which is what multiplying by a
// gain of exactly 1 gives.
__device__ __forceinline__ uint32_t rms_scale_bf16x2(uint32_t xw, float r) {
    const float t0 = bf16_to_f32(xw & 0xFFFFu) * r;
    const float t1 = bf16_to_f32(xw >> 16) * r;
    return (uint32_t)f32_to_bf16(t0) | ((uint32_t)f32_to_bf16(t1) << 16);
}

__device__ __forceinline__ uint4 rms_scale_bf16x8(const uint4& x, float r) {
    return make_uint4(rms_scale_bf16x2(x.x, r), rms_scale_bf16x2(x.y, r), rms_scale_bf16x2(x.z, r),
                      rms_scale_bf16x2(x.w, r));
}

__device__ __forceinline__ uint4 rms_apply_bf16x8(const uint4& x, const uint4& g, float r) {
    return make_uint4(rms_apply_bf16x2(x.x, g.x, r), rms_apply_bf16x2(x.y, g.y, r), rms_apply_bf16x2(x.z, g.z, r),
                      rms_apply_bf16x2(x.w, g.w, r));
}

// bf16 1.0 in both halves: the gain used when there is none (x * 1 is exact).
constexpr uint32_t BF16X2_ONE = 0x3F803F80u;

// ----------------------------------------------------------------- quantisation

// |x| of a bf16 value as an unsigned integer: for non-NaN inputs the order of
// these integers is the order of the magnitudes, so the row absmax can be taken
// on the raw bits.  Two bf16 values per 32-bit word.
__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t w) { return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu); }

struct QuantScale {
    float s;  // fp32(absmax / 127): the divisor
    float r;  // fp32(1 / s), correctly rounded: drives the quotient below
};

// From the row absmax (quant_scale_f32: an fp32 value; quant_scale: bf16
// magnitude bits): clamp below at fp32(1e-5), then the IEEE fp32 quotient by
// 127 and the IEEE reciprocal of that (the compiler's division is correctly
// rounded).  Both are computed once per row.
__device__ __forceinline__ QuantScale quant_scale_f32(float a) {
    a = a < 1e-5f ? 1e-5f : a;
    QuantScale q;
    q.s = a / 127.0f;
    q.r = 1.0f / q.s;
    return q;
}

__device__ __forceinline__ QuantScale quant_scale(uint32_t absmax_bits) {
    float a = bf16_to_f32(absmax_bits);
    a = a < 1e-5f ? 1e-5f : a;
    QuantScale q;
    q.s = a / 127.0f;
    q.r = 1.0f / q.s;
    return q;
}

// fp32(x / s), correctly rounded, from r = fp32(1 / s) with three FMAs and a
// multiply instead of a division (Markstein's FMA division):
//  * q0 = fp32(x r) has a relative error below 2^-23 + 2^-48, i.e. it is
//    within 2 ulp of x / s;
//  * q0 + fp32(x - s q0) r (one FMA, one rounding) differs from x / s by at
//    most about 2^-22 ulp, so its rounding q1 is faithful (one of the two fp32
//    neighbours of x / s);
//  * for a faithful q1 the residual x - s q1 is exact in fp32 (one FMA), and
//    with r within half an ulp of 1 / s, fp32(q1 + (x - s q1) r) is the
//    correctly rounded x / s (Markstein's theorem).
// Valid while no step underflows: whenever |x / s| >= 1/4 every intermediate is
// a normal number (s >= 1e-5 / 127), and below 1/4 the value rounds to 0 to
// an integer whatever the last bits are.  |x| <= absmax keeps |x / s| <= 127.5.
__device__ __forceinline__ float quotient_rn(float x, const QuantScale& q) {
    const float q0 = x * q.r;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, q.s, x), q.r, q0);
    return __builtin_fmaf(__builtin_fmaf(-q1, q.s, x), q.r, q1);
}

// q = clamp(round_half_even(fp32(x / s)), -127, 127), exactly.
__device__ __forceinline__ int quantize_one(float x, const QuantScale& q) {
    float t = __builtin_rintf(quotient_rn(x, q));
    t = __builtin_fminf(__builtin_fmaxf(t, -127.0f), 127.0f);
    return (int)t;
}

// Quantise four f32 values (one 16-byte group) with quantize_one; returns the
// four int8 in one word, low element first.
__device__ __forceinline__ uint32_t quantize_f32x4(const uint4& v, const QuantScale& q) {
    const uint32_t b0 = (uint32_t)quantize_one(__builtin_bit_cast(float, v.x), q) & 0xFFu;
    const uint32_t b1 = (uint32_t)quantize_one(__builtin_bit_cast(float, v.y), q) & 0xFFu;
    const uint32_t b2 = (uint32_t)quantize_one(__builtin_bit_cast(float, v.z), q) & 0xFFu;
    const uint32_t b3 = (uint32_t)quantize_one(__builtin_bit_cast(float, v.w), q) & 0xFFu;
    return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// Largest f32 magnitude bits of four values (the order of non-negative finite floats).
__device__ __forceinline__ uint32_t absmax_f32x4(const uint4& v) {
    return max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
}

// Quantise eight bf16 values (one 16-byte group) with the arithmetic of
// quantize_one; returns the eight int8 in two words, low element first.
//  * Rounding by addition: for |y| <= 2^22, y + 1.5 * 2^23 lands in [2^23,
//    2^24), where the spacing is 1, so the sum is 1.5 * 2^23 + rint(y) with
//    ties to even, and its low byte is rint(y) as a two's-complement int8.
//  * No clamp is needed: |x| <= absmax and s = fp32(absmax / 127), so
//    |fp32(x / s)| <= 127 * (1 + 2^-23) < 127.5 (also when absmax is clamped
//    to 1e-5, since then |x| < 1e-5).
//  * Branch-free: every element takes the same few FMAs (quotient_rn).
// Needs FP contraction off (the sum with 1.5 * 2^23 must see the rounded quotient).
__device__ __forceinline__ uint2 quantize_bf16x8(const uint4& v, const QuantScale& q) {
    constexpr float RND = 12582912.0f;  // 1.5 * 2^23
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = bf16_to_f32((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu));
        u[e] = __builtin_bit_cast(uint32_t, quotient_rn(x, q) + RND);
    }
    // byte 0 of each value: perm selects bytes 0 (second operand) and 4 (first)
    const uint32_t p01 = __builtin_amdgcn_perm(u[1], u[0], 0x0C0C0400u);
    const uint32_t p23 = __builtin_amdgcn_perm(u[3], u[2], 0x0C0C0400u);
    const uint32_t p45 = __builtin_amdgcn_perm(u[5], u[4], 0x0C0C0400u);
    const uint32_t p67 = __builtin_amdgcn_perm(u[7], u[6], 0x0C0C0400u);
    return make_uint2(p01 | (p23 << 16), p45 | (p67 << 16));
}

// Quantise two bf16 values held in one 32-bit word; returns them in the low
// two bytes (low element first).
__device__ __forceinline__ uint32_t quantize_bf16x2(uint32_t w, const QuantScale& q) {
    int a = quantize_one(bf16_to_f32(w & 0xFFFFu), q);
    int b = quantize_one(bf16_to_f32(w >> 16), q);
    return ((uint32_t)a & 0xFFu) | (((uint32_t)b & 0xFFu) << 8);
}

// ----------------------------------------------------------------- epilogue

// The bias on a bf16 layer output: bf16_rne(fp32(y) + fp32(bias)).
__device__ __forceinline__ uint16_t add_bias_bf16(uint32_t y, uint32_t b) {
    return f32_to_bf16(bf16_to_f32(y) + bf16_to_f32(b));
}

// out = bf16_rne( fp32( (float)acc * fp32(sa * sw) ) ).  sa * sw is exact (two
// bf16 significands fit in fp32), (float)acc is exact for |acc| < 2^24, so the
// result has a single fp32 rounding followed by the bf16 rounding.  There is
// no addition, so no contraction can change it.
__device__ __forceinline__ uint16_t epilogue_bf16(int acc, float sa, float sw) {
    const float scale = sa * sw;
    const float y = (float)acc * scale;
    return f32_to_bf16(y);
}

// The same for two outputs, rounded to bf16 by one v_cvt_pk_bf16_f32; the
// result holds the first in its low half.
__device__ __forceinline__ uint32_t epilogue_bf16x2(int acc0, float sa0, int acc1, float sa1, float sw) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const float y0 = (float)acc0 * (sa0 * sw);
    const float y1 = (float)acc1 * (sa1 * sw);
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y0, y1}, bf16x2));
}

// ----------------------------------------------------------------- 2-bit codes

// For a 32-bit word of packed weights (16 codes; byte r holds the elements
// 4r..4r+3, element e of the byte in bits 2e..2e+1), the byte-lane masks that
// isolate element e of every byte: (p >> 2e) & 0x03030303 gives, in byte r,
// the code of element 4r + e.
constexpr uint32_t CODE_MASK = 0x03030303u;

// 4x4 byte transpose: n_r holds elements 4r..4r+3; result t_e holds element e of
// every n_r (t_e byte r = element 4r + e).
__device__ __forceinline__ uint4 transpose4x4(uint32_t n0, uint32_t n1, uint32_t n2, uint32_t n3) {
    const uint32_t u01lo = __builtin_amdgcn_perm(n1, n0, 0x05010400u);  // n0.b0 n1.b0 n0.b1 n1.b1
    const uint32_t u01hi = __builtin_amdgcn_perm(n1, n0, 0x07030602u);  // n0.b2 n1.b2 n0.b3 n1.b3
    const uint32_t u23lo = __builtin_amdgcn_perm(n3, n2, 0x05010400u);
    const uint32_t u23hi = __builtin_amdgcn_perm(n3, n2, 0x07030602u);
    uint4 t;
    t.x = __builtin_amdgcn_perm(u23lo, u01lo, 0x05040100u);
    t.y = __builtin_amdgcn_perm(u23lo, u01lo, 0x07060302u);
    t.z = __builtin_amdgcn_perm(u23hi, u01hi, 0x05040100u);
    t.w = __builtin_amdgcn_perm(u23hi, u01hi, 0x07060302u);
    return t;
}

}  // namespace bitnet
