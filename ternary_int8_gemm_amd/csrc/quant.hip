// quant.hip -- per-token absmax INT8 quantisation (K-QUANT).
//
// Implements quantize_activation of "phanerozoic/bitnet-cpu v1,
// torch-ext/bitnet_cpu/__init__.py" in fp32 on the widened bf16 input:
// absmax per row clamped below at 1e-5, s = absmax / 127 (IEEE fp32 division),
// q = clamp(round_half_even(x / s), -127, 127), scale stored as bf16(s).
//
// Layout on gfx950.  The kernel is HBM-bound at 3 bytes per element, so what
// matters is keeping enough bytes in flight and the per-row work short:
//  * quantize_rows_block<CH> (rows of up to 2048 * CH elements, K % 8 == 0):
//    one 256-thread workgroup per row; each thread loads its CH 16-byte groups
//    of the row up front (consecutive threads, consecutive groups), the absmax
//    is reduced on the bf16 magnitude bits (an integer max; DPP inside each
//    wave, LDS across the four), and the row is quantised from registers: one
//    read of x, 8-byte int8 stores written through the L2.
//  * quantize_rows_vec (longer rows, K % 16 == 0): one wave per row, two
//    passes over the row, the second re-reading it from L2.
//  * quantize_rows_plain: any K and alignment, one element per lane.
//
// RMSNorm variants (the RMS flag of quantize_rows_block, and
// quantize_rows_rms_plain) normalise the row first, as the BitNet
// activation_norm_quant of "kyegomez/BitNet issue #77" does before quantising:
// the exact squares of the row are summed in double, every thread forms the
// normalised bf16 values of its registers (fp32 x * r, times the gain), and
// the absmax and quantisation then run on those values.
#include "bitnet_device.h"
#include "launch.h"

namespace bitnet {

namespace {

constexpr int QUANT_ROWS_PER_BLOCK = 4;
// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format,
// stride 0: offsets are checked against the byte count in word 2).
constexpr int QUANT_BUFFER_RSRC_WORD3 = 0x00020000;
// Cache policy of the int8 row stores: sc0 | sc1, written through the L2.
constexpr int QUANT_STORE_WT = 17;
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Vector path: K % 16 == 0, x and q 16-byte aligned.
__global__ __launch_bounds__(256) void quantize_rows_vec(int8_t* __restrict__ q, uint16_t* __restrict__ scale,
                                                         const uint16_t* __restrict__ x, int64_t M, int64_t K) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * QUANT_ROWS_PER_BLOCK + (threadIdx.x >> 6);
    if (m >= M) return;  // wave-uniform
    const uint4* xv = reinterpret_cast<const uint4*>(x + m * K);
    const int64_t n16 = K / 16;  // groups of 16 elements = 2 x 16 bytes of bf16

    uint32_t amax = 0;
    for (int64_t i = lane; i < n16; i += 64) {
        const uint4 a = xv[2 * i];
        const uint4 b = xv[2 * i + 1];
        amax = max(amax, max(max(absmax_bf16x2(a.x), absmax_bf16x2(a.y)), max(absmax_bf16x2(a.z), absmax_bf16x2(a.w))));
        amax = max(amax, max(max(absmax_bf16x2(b.x), absmax_bf16x2(b.y)), max(absmax_bf16x2(b.z), absmax_bf16x2(b.w))));
    }
    amax = wave_max_u32(amax);
    const QuantScale qs = quant_scale(amax);
    if (lane == 0) scale[m] = f32_to_bf16(qs.s);

    uint4* qv = reinterpret_cast<uint4*>(q + m * K);
    for (int64_t i = lane; i < n16; i += 64) {
        const uint4 a = xv[2 * i];
        const uint4 b = xv[2 * i + 1];
        uint4 o;
        const uint2 qa = quantize_bf16x8(a, qs);
        const uint2 qb = quantize_bf16x8(b, qs);
        o.x = qa.x;
        o.y = qa.y;
        o.z = qb.x;
        o.w = qb.y;
        qv[i] = o;
    }
}

// Register-resident path, one workgroup per row: the 256 threads of workgroup
// m hold the 8-element groups g = c * 256 + tid (c < CH) of row m, so a row's
// arithmetic is spread over four waves and its loads are all in flight at
// once.  (One wave per row, measured against it, was 1.3-2x slower at every M
// from 5 to 4096 on the BitNet-2B-4T and LLaMA-7B widths.)  The sum of squares
// and the absmax are reduced per wave (DPP), then over the four waves through
// LDS in a fixed order.  Needs K % 8 == 0, K <= 2048 * CH, 16-byte aligned x
// rows (and gain, xn_out) and 8-byte aligned q rows.  With RMS, xn_out (when
// not NULL) receives the normalised bf16 row; without a gain the absmax of
// the normalised row is bf16(fp32(max|x| * r)) (both roundings are monotonic,
// r > 0), so it is reduced together with the sum of squares.
template <int CH, bool RMS>
__global__ __launch_bounds__(256) void quantize_rows_block(int8_t* __restrict__ q, uint16_t* __restrict__ scale,
                                                           uint16_t* __restrict__ xn_out,
                                                           const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ gain, float eps,
                                                           int64_t /*M: one workgroup per row*/, int64_t K) {
    constexpr int WAVES = 4;
    __shared__ double red_d[WAVES];
    __shared__ uint32_t red_a[WAVES];  // absmax of x (RMS without a gain)
    __shared__ uint32_t red_b[WAVES];  // absmax of the values to quantise
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t m = blockIdx.x;
    const int groups = (int)(K >> 3);
    const uint4* xv = reinterpret_cast<const uint4*>(x + m * K);
    uint4 v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int g = c * 256 + tid;
        v[c] = g < groups ? xv[g] : make_uint4(0u, 0u, 0u, 0u);  // zeros change neither sum nor absmax
    }
    auto absmax = [&]() {
        uint32_t a = 0u;
#pragma unroll
        for (int c = 0; c < CH; ++c)
            a = max(a, max(max(absmax_bf16x2(v[c].x), absmax_bf16x2(v[c].y)),
                           max(absmax_bf16x2(v[c].z), absmax_bf16x2(v[c].w))));
        return wave_max_u32(a);
    };
    uint32_t amax = 0u;
    bool have_amax = false;
    if constexpr (RMS) {
        double ss = 0.0;
#pragma unroll
        for (int c = 0; c < CH; ++c) ss += sum_sq_bf16x8(v[c]);
        ss = wave_sum_f64(ss);
        const uint32_t a = gain == nullptr ? absmax() : 0u;  // wave-uniform
        if (lane == 0) {
            red_d[wave] = ss;
            red_a[wave] = a;
        }
        __syncthreads();
        const float r = rms_inv(((red_d[0] + red_d[1]) + red_d[2]) + red_d[3], (int)K, eps);
        const uint4* gv = reinterpret_cast<const uint4*>(gain);
        if (gain == nullptr) {  // the same bits as a gain of 1
#pragma unroll
            for (int c = 0; c < CH; ++c) v[c] = rms_scale_bf16x8(v[c], r);  // zero padding stays zero
        } else {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int g = c * 256 + tid;
                const uint4 gw = g < groups ? gv[g] : make_uint4(BF16X2_ONE, BF16X2_ONE, BF16X2_ONE, BF16X2_ONE);
                v[c] = rms_apply_bf16x8(v[c], gw, r);
            }
        }
        if (xn_out != nullptr) {
            uint4* xo = reinterpret_cast<uint4*>(xn_out + m * K);
#pragma unroll
            for (int c = 0; c < CH; ++c)
                if (c * 256 + tid < groups) xo[c * 256 + tid] = v[c];
        }
        if (gain == nullptr) {
            const uint32_t ax = max(max(red_a[0], red_a[1]), max(red_a[2], red_a[3]));
            amax = (uint32_t)f32_to_bf16(bf16_to_f32(ax) * r) & 0x7FFFu;
            have_amax = true;
        }
    }
    if (!have_amax) {  // workgroup-uniform
        const uint32_t a = absmax();
        if (lane == 0) red_b[wave] = a;
        __syncthreads();
        amax = max(max(red_b[0], red_b[1]), max(red_b[2], red_b[3]));
    }
    const QuantScale qs = quant_scale(amax);
    if (tid == 0) scale[m] = f32_to_bf16(qs.s);
    // 8-byte stores written through the L2 (sc0 sc1) instead of left dirty
    // there until the kernel ends: measured 5.45 -> 4.62 us for 2048 x 4096
    // (12.6 -> 11.8 us for 2048 x 11008), the same bits.
    const __amdgpu_buffer_rsrc_t q_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(q + m * K, (short)0, (int)K, QUANT_BUFFER_RSRC_WORD3);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int g = c * 256 + tid;
        const uint2 t = quantize_bf16x8(v[c], qs);
        if (g < groups) __builtin_amdgcn_raw_buffer_store_b64(v2u{t.x, t.y}, q_rsrc, g * 8, 0, QUANT_STORE_WT);
    }
}

// Plain path for any K and alignment: one element per lane per iteration.
__global__ __launch_bounds__(256) void quantize_rows_plain(int8_t* __restrict__ q, uint16_t* __restrict__ scale,
                                                           const uint16_t* __restrict__ x, int64_t M, int64_t K) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * QUANT_ROWS_PER_BLOCK + (threadIdx.x >> 6);
    if (m >= M) return;
    const uint16_t* xr = x + m * K;
    uint32_t amax = 0;
    for (int64_t k = lane; k < K; k += 64) amax = max(amax, (uint32_t)xr[k] & 0x7FFFu);
    amax = wave_max_u32(amax);
    const QuantScale qs = quant_scale(amax);
    if (lane == 0) scale[m] = f32_to_bf16(qs.s);
    int8_t* qr = q + m * K;
    for (int64_t k = lane; k < K; k += 64) qr[k] = (int8_t)quantize_one(bf16_to_f32(xr[k]), qs);
}

// RMSNorm then quantise, any K and alignment: the sum of squares, then the
// absmax of the normalised values, then the quantisation (each recomputing the
// normalised element, which is a pure function of x, r and the gain).
__global__ __launch_bounds__(256) void quantize_rows_rms_plain(int8_t* __restrict__ q, uint16_t* __restrict__ scale,
                                                               uint16_t* __restrict__ xn_out,
                                                               const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ gain, float eps,
                                                               int64_t M, int64_t K) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * QUANT_ROWS_PER_BLOCK + (threadIdx.x >> 6);
    if (m >= M) return;
    const uint16_t* xr = x + m * K;
    double ss = 0.0;
    for (int64_t k = lane; k < K; k += 64) {
        const double d = (double)bf16_to_f32(xr[k]);
        ss += d * d;
    }
    const float r = rms_inv(wave_sum_f64(ss), (int)K, eps);
    auto norm = [&](int64_t k) -> uint32_t {
        const uint32_t g = gain != nullptr ? (uint32_t)gain[k] : 0x3F80u;
        return rms_apply_bf16x2((uint32_t)xr[k], g, r) & 0xFFFFu;
    };
    uint32_t amax = 0;
    for (int64_t k = lane; k < K; k += 64) amax = max(amax, norm(k) & 0x7FFFu);
    amax = wave_max_u32(amax);
    const QuantScale qs = quant_scale(amax);
    if (lane == 0) scale[m] = f32_to_bf16(qs.s);
    int8_t* qr = q + m * K;
    for (int64_t k = lane; k < K; k += 64) {
        const uint32_t h = norm(k);
        qr[k] = (int8_t)quantize_one(bf16_to_f32(h), qs);
        if (xn_out != nullptr) xn_out[m * K + k] = (uint16_t)h;
    }
}

// ---------------------------------------------------------------- f32 input
//
// The same quantisation on f32 activations (quantize_activation accepts bf16
// or f32): the absmax is an integer max over the f32 magnitude bits (the
// order of non-negative finite floats), and q comes from the same exact
// division.  One 256-thread workgroup per row, as quantize_rows_block: thread
// t holds the 4-element groups g = c * 256 + t (c < CH).
template <int CH>
__global__ __launch_bounds__(256) void quantize_rows_f32_block(int8_t* __restrict__ q, uint16_t* __restrict__ scale,
                                                               const float* __restrict__ x,
                                                               int64_t /*M: one workgroup per row*/, int64_t K) {
    constexpr int WAVES = 4;
    __shared__ uint32_t red[WAVES];
    const int tid = threadIdx.x;
    const int64_t m = blockIdx.x;
    const int groups = (int)(K >> 2);
    const uint4* xv = reinterpret_cast<const uint4*>(x + m * K);
    uint4 v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int g = c * 256 + tid;
        v[c] = g < groups ? xv[g] : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t amax = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) amax = max(amax, absmax_f32x4(v[c]));
    amax = wave_max_u32(amax);
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = max(max(red[0], red[1]), max(red[2], red[3]));
    const QuantScale qs = quant_scale_f32(__builtin_bit_cast(float, amax));
    if (tid == 0) scale[m] = f32_to_bf16(qs.s);
    uint32_t* qv = reinterpret_cast<uint32_t*>(q + m * K);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int g = c * 256 + tid;
        if (g < groups) qv[g] = quantize_f32x4(v[c], qs);
    }
}

// Any K and alignment: one element per lane per iteration, two passes.
__global__ __launch_bounds__(256) void quantize_rows_f32_plain(int8_t* __restrict__ q, uint16_t* __restrict__ scale,
                                                               const float* __restrict__ x, int64_t M, int64_t K) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * QUANT_ROWS_PER_BLOCK + (threadIdx.x >> 6);
    if (m >= M) return;
    const float* xr = x + m * K;
    uint32_t amax = 0;
    for (int64_t k = lane; k < K; k += 64) amax = max(amax, __builtin_bit_cast(uint32_t, xr[k]) & 0x7FFFFFFFu);
    amax = wave_max_u32(amax);
    const QuantScale qs = quant_scale_f32(__builtin_bit_cast(float, amax));
    if (lane == 0) scale[m] = f32_to_bf16(qs.s);
    int8_t* qr = q + m * K;
    for (int64_t k = lane; k < K; k += 64) qr[k] = (int8_t)quantize_one(xr[k], qs);
}

}  // namespace

namespace {

template <bool RMS>
void launch_rows_block(hipStream_t s, int8_t* q, uint16_t* scale, uint16_t* xn, const uint16_t* x,
                       const uint16_t* gain, float eps, int64_t M, int64_t K) {
    const int64_t ch = (K / 8 + 255) / 256;
    const dim3 grid((unsigned)M), block(256);
    if (ch <= 1)
        hipLaunchKernelGGL((quantize_rows_block<1, RMS>), grid, block, 0, s, q, scale, xn, x, gain, eps, M, K);
    else if (ch <= 2)
        hipLaunchKernelGGL((quantize_rows_block<2, RMS>), grid, block, 0, s, q, scale, xn, x, gain, eps, M, K);
    else if (ch <= 4)
        hipLaunchKernelGGL((quantize_rows_block<4, RMS>), grid, block, 0, s, q, scale, xn, x, gain, eps, M, K);
    else
        hipLaunchKernelGGL((quantize_rows_block<8, RMS>), grid, block, 0, s, q, scale, xn, x, gain, eps, M, K);
}


}  // namespace

hipError_t launch_quantize(int8_t* q, uint16_t* scale, const uint16_t* x, int64_t M, int64_t K, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    const int64_t blocks = (M + QUANT_ROWS_PER_BLOCK - 1) / QUANT_ROWS_PER_BLOCK;
    const dim3 grid((unsigned)blocks), block(256);
    if (K % 8 == 0 && aligned16(x) && reinterpret_cast<uintptr_t>(q) % 8 == 0 && K <= 2048 * 8) {
        launch_rows_block<false>(s, q, scale, nullptr, x, nullptr, 0.0f, M, K);
    } else if (K % 16 == 0 && aligned16(x) && aligned16(q)) {
        hipLaunchKernelGGL(quantize_rows_vec, grid, block, 0, s, q, scale, x, M, K);
    } else {
        hipLaunchKernelGGL(quantize_rows_plain, grid, block, 0, s, q, scale, x, M, K);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_rms(int8_t* q, uint16_t* scale, uint16_t* xn, const uint16_t* x, const uint16_t* gain,
                               float eps, int64_t M, int64_t K, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    const int64_t blocks = (M + QUANT_ROWS_PER_BLOCK - 1) / QUANT_ROWS_PER_BLOCK;
    const dim3 grid((unsigned)blocks), block(256);
    const bool vec = K % 8 == 0 && K <= 2048 * 8 && aligned16(x) && (gain == nullptr || aligned16(gain)) &&
                     (xn == nullptr || aligned16(xn)) && reinterpret_cast<uintptr_t>(q) % 8 == 0;
    if (vec)
        launch_rows_block<true>(s, q, scale, xn, x, gain, eps, M, K);
    else
        hipLaunchKernelGGL(quantize_rows_rms_plain, grid, block, 0, s, q, scale, xn, x, gain, eps, M, K);
    return hipGetLastError();
}

hipError_t launch_quantize_f32(int8_t* q, uint16_t* scale, const float* x, int64_t M, int64_t K, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    const dim3 block(256);
    if (K % 4 == 0 && aligned16(x) && reinterpret_cast<uintptr_t>(q) % 4 == 0 && K <= 1024 * 16) {
        const dim3 grid((unsigned)M);
        const int64_t ch = (K / 4 + 255) / 256;  // 16-byte groups per thread
        if (ch <= 1)
            hipLaunchKernelGGL(quantize_rows_f32_block<1>, grid, block, 0, s, q, scale, x, M, K);
        else if (ch <= 2)
            hipLaunchKernelGGL(quantize_rows_f32_block<2>, grid, block, 0, s, q, scale, x, M, K);
        else if (ch <= 4)
            hipLaunchKernelGGL(quantize_rows_f32_block<4>, grid, block, 0, s, q, scale, x, M, K);
        else if (ch <= 8)
            hipLaunchKernelGGL(quantize_rows_f32_block<8>, grid, block, 0, s, q, scale, x, M, K);
        else
            hipLaunchKernelGGL(quantize_rows_f32_block<16>, grid, block, 0, s, q, scale, x, M, K);
    } else {
        const dim3 grid((unsigned)((M + QUANT_ROWS_PER_BLOCK - 1) / QUANT_ROWS_PER_BLOCK));
        hipLaunchKernelGGL(quantize_rows_f32_plain, grid, block, 0, s, q, scale, x, M, K);
    }
    return hipGetLastError();
}

}  // namespace bitnet
