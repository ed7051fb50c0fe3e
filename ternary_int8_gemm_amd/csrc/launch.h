// launch.h -- internal kernel launchers of the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace bitnet {

// Per-token absmax INT8 quantisation of x [M][K] (bf16) into q [M][K] and the
// bf16 scales [M].
hipError_t launch_quantize(int8_t* q, uint16_t* scale, const uint16_t* x, int64_t M, int64_t K, hipStream_t s);

// Batched ternary x int8 product.  Exactly one of out (bf16 [M][N], scaled
// with scale_act / scale_wt) and acc (int32 [M][N], unscaled) is non-null.
hipError_t launch_gemm(uint16_t* out, int32_t* acc, const int8_t* x, const uint8_t* w, const uint16_t* scale_act,
                       const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K, hipStream_t s);

// Fused quantise + GEMV for M <= 15.  Exactly one of out (bf16 [M][N]) and acc
// (int32 [M][N]) is non-null; scale_act_out (bf16 [M]) may be null.
hipError_t launch_gemv_fused(uint16_t* out, int32_t* acc, uint16_t* scale_act_out, const uint16_t* x,
                             const uint8_t* w, const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K,
                             hipStream_t s);

// The fused quantise + product on int8 MFMA for 1 <= M <= 16 rows (used from
// five rows up), for shapes gemv_mfma_fits accepts; same outputs as
// launch_gemv_fused.
bool gemv_mfma_fits(int64_t M, int64_t N, int64_t K, const void* x, const void* w);
hipError_t launch_gemv_mfma(uint16_t* out, int32_t* acc, uint16_t* scale_act_out, const uint16_t* x,
                            const uint8_t* w, const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K,
                            hipStream_t s);

// out[m][n] = epilogue(acc[m][n], scale_act[m], scale_wt[n]).
hipError_t launch_epilogue(uint16_t* out, const int32_t* acc, const uint16_t* scale_act, const uint16_t* scale_wt,
                           int64_t M, int64_t N, hipStream_t s);

// The same quantisation of f32 activations x [M][K].
hipError_t launch_quantize_f32(int8_t* q, uint16_t* scale, const float* x, int64_t M, int64_t K, hipStream_t s);

// In place: out[m][n] = bf16(fp32(out[m][n]) + fp32(bias[n])).
hipError_t launch_add_bias(uint16_t* out, const uint16_t* bias, int64_t M, int64_t N, hipStream_t s);

// Fused decode GEMV with the RMSNorm prologue (1 <= M <= 4, K % 64 == 0,
// aligned operands, activations within the LDS budget: gemv_rms_fusable).
bool gemv_rms_fusable(int64_t M, int64_t K, const void* x, const void* w, const void* gain);
hipError_t launch_gemv_fused_rms(uint16_t* out, uint16_t* scale_act_out, const uint16_t* x, const uint16_t* gain,
                                 float eps, const uint8_t* w, const uint16_t* scale_wt, int64_t M, int64_t N,
                                 int64_t K, hipStream_t s);

// The fused GEMV for bitnet_linear_ex: bf16 or f32 (x_f32) activations, an
// optional bf16 bias on the outputs; M <= 4, shapes gemv_ex_fusable accepts.
bool gemv_ex_fusable(int64_t M, int64_t K, const void* x, const void* w);
hipError_t launch_gemv_fused_ex(uint16_t* out, const void* x, bool x_f32, const uint16_t* bias, const uint8_t* w,
                                const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K, hipStream_t s);

// RMSNorm over each row of bf16 x [M][K] (optional bf16 gain [K]), then the
// per-token quantisation of the normalised row; xn (optional) receives it.
hipError_t launch_quantize_rms(int8_t* q, uint16_t* scale, uint16_t* xn, const uint16_t* x, const uint16_t* gain,
                               float eps, int64_t M, int64_t K, hipStream_t s);

// INT8 weight-only matmul: y [M][N] (fp32) = scale[n] * sum_k x[m][k] * q[n][k],
// x bf16 [M][K] (M <= 64), q int8 [N][K], scale fp32 [N].
hipError_t launch_w8a16(float* y, const uint16_t* x, const int8_t* q, const float* scale, int64_t M, int64_t N,
                        int64_t K, hipStream_t s);

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Raise a kernel's dynamic LDS limit above the 64 KB default, once per device
// for each kernel instance (each instance has its own flag word; devices past
// 63 set the attribute on every launch).
template <typename Kern>
hipError_t raise_lds_limit(Kern kern, size_t lds) {
    static std::atomic<unsigned long long> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = (dev >= 0 && dev < 64) ? 1ull << dev : 0;
    if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
    return e;
}


}  // namespace bitnet
