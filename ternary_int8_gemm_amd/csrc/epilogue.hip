// epilogue.hip -- the standalone scale epilogue (K-EPI) for int32 accumulators.
//
// out[m][n] = bf16_rne( fp32( (float)acc[m][n] * fp32( (float)scale_act[m] * (float)scale_wt[n] ) ) )
//
// The scale step of bitnet_gemm in "phanerozoic/bitnet-cpu v1,
// torch-ext/bitnet_cpu/__init__.py" (per-row activation scale, per-output
// weight scale, bf16 result), applied to the exact integer accumulator without
// an intermediate bf16 rounding (docstring of int8_matmul in "CoolDip00/tiny-llm
// src/tinyllm/kernels/int8_gemv.py").  The same device function is fused into
// the GEMV and GEMM kernels; this kernel exists so the epilogue can be run on
// given accumulators.  Elementwise and HBM-bound (4 B in, 2 B out per element):
// each lane handles 4 consecutive outputs of one row with a 16-byte load and an
// 8-byte store when N % 4 == 0.
//
// Also here: the bias of the BitLinear module of the same page, added in place
// to the layer's bf16 output: out = bf16_rne(fp32(out) + fp32(bias[n])).
#include "bitnet_device.h"
#include "launch.h"

namespace bitnet {

namespace {

__global__ __launch_bounds__(256) void epilogue_vec4(uint16_t* __restrict__ out, const int32_t* __restrict__ acc,
                                                     const uint16_t* __restrict__ sa,
                                                     const uint16_t* __restrict__ sw, int64_t M, int64_t N) {
    const int64_t groups = M * (N / 4);
    for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < groups;
         gi += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = gi * 4;
        const int64_t m = i / N;
        const int64_t n = i - m * N;
        const int4 a = *reinterpret_cast<const int4*>(acc + i);
        const float fa = bf16_to_f32(sa[m]);
        const uint32_t o0 = epilogue_bf16(a.x, fa, bf16_to_f32(sw[n + 0]));
        const uint32_t o1 = epilogue_bf16(a.y, fa, bf16_to_f32(sw[n + 1]));
        const uint32_t o2 = epilogue_bf16(a.z, fa, bf16_to_f32(sw[n + 2]));
        const uint32_t o3 = epilogue_bf16(a.w, fa, bf16_to_f32(sw[n + 3]));
        uint2 o;
        o.x = o0 | (o1 << 16);
        o.y = o2 | (o3 << 16);
        *reinterpret_cast<uint2*>(out + i) = o;
    }
}

__global__ __launch_bounds__(256) void epilogue_plain(uint16_t* __restrict__ out, const int32_t* __restrict__ acc,
                                                      const uint16_t* __restrict__ sa,
                                                      const uint16_t* __restrict__ sw, int64_t M, int64_t N) {
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / N;
        const int64_t n = i - m * N;
        out[i] = epilogue_bf16(acc[i], bf16_to_f32(sa[m]), bf16_to_f32(sw[n]));
    }
}

__device__ __forceinline__ uint32_t add_bias_pair(uint32_t y2, uint32_t b2) {
    const uint32_t lo = add_bias_bf16(y2 & 0xFFFFu, b2 & 0xFFFFu);
    const uint32_t hi = add_bias_bf16(y2 >> 16, b2 >> 16);
    return lo | (hi << 16);
}

// 8 outputs per lane (16-byte accesses) when N % 8 == 0 and out, bias are 16-byte aligned.
__global__ __launch_bounds__(256) void add_bias_vec8(uint16_t* __restrict__ out, const uint16_t* __restrict__ bias,
                                                     int64_t M, int64_t N) {
    const int64_t groups = M * (N / 8);
    for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < groups;
         gi += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = gi * 8;
        const int64_t n = i % N;
        uint4 y = *reinterpret_cast<const uint4*>(out + i);
        const uint4 b = *reinterpret_cast<const uint4*>(bias + n);
        y.x = add_bias_pair(y.x, b.x);
        y.y = add_bias_pair(y.y, b.y);
        y.z = add_bias_pair(y.z, b.z);
        y.w = add_bias_pair(y.w, b.w);
        *reinterpret_cast<uint4*>(out + i) = y;
    }
}

__global__ __launch_bounds__(256) void add_bias_plain(uint16_t* __restrict__ out, const uint16_t* __restrict__ bias,
                                                      int64_t M, int64_t N) {
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x)
        out[i] = add_bias_bf16(out[i], bias[i % N]);
}

int64_t grid_for(int64_t work) {
    int64_t b = (work + 255) / 256;
    if (b > 8192) b = 8192;
    return b < 1 ? 1 : b;
}

}  // namespace

hipError_t launch_epilogue(uint16_t* out, const int32_t* acc, const uint16_t* scale_act, const uint16_t* scale_wt,
                           int64_t M, int64_t N, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const bool vec = (N % 4 == 0) && aligned16(acc) && (((uintptr_t)out & 7u) == 0);
    if (vec) {
        hipLaunchKernelGGL(epilogue_vec4, dim3((unsigned)grid_for(M * N / 4)), dim3(256), 0, s, out, acc, scale_act,
                           scale_wt, M, N);
    } else {
        hipLaunchKernelGGL(epilogue_plain, dim3((unsigned)grid_for(M * N)), dim3(256), 0, s, out, acc, scale_act,
                           scale_wt, M, N);
    }
    return hipGetLastError();
}

hipError_t launch_add_bias(uint16_t* out, const uint16_t* bias, int64_t M, int64_t N, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (N % 8 == 0 && aligned16(out) && aligned16(bias))
        hipLaunchKernelGGL(add_bias_vec8, dim3((unsigned)grid_for(M * N / 8)), dim3(256), 0, s, out, bias, M, N);
    else
        hipLaunchKernelGGL(add_bias_plain, dim3((unsigned)grid_for(M * N)), dim3(256), 0, s, out, bias, M, N);
    return hipGetLastError();
}

}  // namespace bitnet
