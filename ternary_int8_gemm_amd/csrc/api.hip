// api.hip -- the exported C ABI (include/bitnet.h): argument checks, the
// gfx950 device check, dispatch by M, and kernel launches.  No entry point
// allocates, frees or synchronises; device work is enqueued on the caller's
// stream.
#include <atomic>
#include <cstring>

#include "../../include/bitnet.h"
#include "launch.h"

#define BITNET_API extern "C" __attribute__((visibility("default")))

namespace {

using bitnet::launch_epilogue;
using bitnet::launch_gemm;
using bitnet::launch_gemv_fused;
using bitnet::launch_quantize;
using bitnet::launch_quantize_f32;
using bitnet::launch_add_bias;
using bitnet::launch_w8a16;
using bitnet::launch_quantize_rms;
using bitnet::launch_gemv_fused_rms;
using bitnet::gemv_rms_fusable;
using bitnet::gemv_ex_fusable;
using bitnet::launch_gemv_fused_ex;

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_arch_ok[kMaxDevices];

bitnet_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return BITNET_ERR_DEVICE;
    if (dev >= kMaxDevices) return BITNET_ERR_DEVICE;
    int state = g_arch_ok[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BITNET_ERR_DEVICE;
        state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_ok[dev].store(state, std::memory_order_release);
    }
    return state == 1 ? BITNET_OK : BITNET_ERR_DEVICE;
}

bitnet_status check_k(int64_t K) {
    if (K <= 0 || K % 4 != 0 || K > BITNET_MAX_K) return BITNET_ERR_SHAPE;
    return BITNET_OK;
}

bitnet_status launched(hipError_t e) { return e == hipSuccess ? BITNET_OK : BITNET_ERR_LAUNCH; }

// Sizes that fit the kernels' 32-bit index arithmetic.
bool sizes_ok(int64_t M, int64_t N) { return M >= 0 && N >= 0 && M <= (int64_t)1 << 30 && N <= (int64_t)1 << 30; }

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

BITNET_API int bitnet_version(void) { return 100; }

BITNET_API const char* bitnet_status_string(bitnet_status status) {
    switch (status) {
        case BITNET_OK: return "ok";
        case BITNET_ERR_NULL: return "null pointer argument";
        case BITNET_ERR_SHAPE: return "invalid shape";
        case BITNET_ERR_VALUE: return "weight value outside {-1, 0, +1}";
        case BITNET_ERR_WORKSPACE: return "workspace too small";
        case BITNET_ERR_DEVICE: return "current device is not gfx950 (MI355X)";
        case BITNET_ERR_LAUNCH: return "kernel launch failed";
        case BITNET_ERR_TOO_LARGE: return "problem exceeds the static scratch of bitnet_linear_noalloc";
    }
    return "unknown status";
}

BITNET_API bitnet_status bitnet_pack_weights(uint8_t* w_packed, const int8_t* w, int64_t N, int64_t K) {
    if (N < 0 || K < 0 || K % 4 != 0) return BITNET_ERR_SHAPE;
    if (N == 0 || K == 0) return BITNET_OK;
    if (w_packed == nullptr || w == nullptr) return BITNET_ERR_NULL;
    const int64_t nbytes = N * (K / 4);
    // Four weights per byte; the code of weight e of the byte (w + 2) sits in
    // bits 2e..2e+1.  A lookup on (w + 1) in {0, 1, 2} is both the range check
    // and the encoding.
    for (int64_t i = 0; i < nbytes; ++i) {
        const int8_t* q = w + 4 * i;
        uint32_t byte = 0;
        for (int e = 0; e < 4; ++e) {
            const uint32_t u = (uint32_t)((int32_t)q[e] + 1);
            if (u > 2u) return BITNET_ERR_VALUE;
            byte |= (u + 1u) << (2 * e);
        }
        w_packed[i] = (uint8_t)byte;
    }
    return BITNET_OK;
}

BITNET_API bitnet_status bitnet_quantize_act(int8_t* x_int8, uint16_t* scale_act, const uint16_t* x, int64_t M,
                                             int64_t K, bitnet_stream_t stream) {
    if (!sizes_ok(M, 0)) return BITNET_ERR_SHAPE;
    if (bitnet_status st = check_k(K)) return st;
    if (M == 0) return BITNET_OK;
    if (!x_int8 || !scale_act || !x) return BITNET_ERR_NULL;
    if (bitnet_status st = check_device()) return st;
    return launched(launch_quantize(x_int8, scale_act, x, M, K, (hipStream_t)stream));
}

BITNET_API bitnet_status bitnet_gemm(uint16_t* out, const int8_t* x_int8, const uint8_t* w_packed,
                                     const uint16_t* scale_act, const uint16_t* scale_wt, int64_t M, int64_t N,
                                     int64_t K, bitnet_stream_t stream) {
    if (!sizes_ok(M, N)) return BITNET_ERR_SHAPE;
    if (bitnet_status st = check_k(K)) return st;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!out || !x_int8 || !w_packed || !scale_act || !scale_wt) return BITNET_ERR_NULL;
    if (bitnet_status st = check_device()) return st;
    return launched(launch_gemm(out, nullptr, x_int8, w_packed, scale_act, scale_wt, M, N, K, (hipStream_t)stream));
}

BITNET_API bitnet_status bitnet_gemm_i32(int32_t* acc, const int8_t* x_int8, const uint8_t* w_packed, int64_t M,
                                         int64_t N, int64_t K, bitnet_stream_t stream) {
    if (!sizes_ok(M, N)) return BITNET_ERR_SHAPE;
    if (bitnet_status st = check_k(K)) return st;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!acc || !x_int8 || !w_packed) return BITNET_ERR_NULL;
    if (bitnet_status st = check_device()) return st;
    return launched(launch_gemm(nullptr, acc, x_int8, w_packed, nullptr, nullptr, M, N, K, (hipStream_t)stream));
}

BITNET_API bitnet_status bitnet_gemv_fused(uint16_t* out, const uint16_t* x, const uint8_t* w_packed,
                                           const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K,
                                           bitnet_stream_t stream) {
    if (!sizes_ok(M, N) || M > BITNET_FUSED_MAX_M) return BITNET_ERR_SHAPE;
    if (bitnet_status st = check_k(K)) return st;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!out || !x || !w_packed || !scale_wt) return BITNET_ERR_NULL;
    if (bitnet_status st = check_device()) return st;
    return launched(launch_gemv_fused(out, nullptr, nullptr, x, w_packed, scale_wt, M, N, K, (hipStream_t)stream));
}

BITNET_API bitnet_status bitnet_gemv_fused_i32(int32_t* acc, uint16_t* scale_act, const uint16_t* x,
                                               const uint8_t* w_packed, int64_t M, int64_t N, int64_t K,
                                               bitnet_stream_t stream) {
    if (!sizes_ok(M, N) || M > BITNET_FUSED_MAX_M) return BITNET_ERR_SHAPE;
    if (bitnet_status st = check_k(K)) return st;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!acc || !scale_act || !x || !w_packed) return BITNET_ERR_NULL;
    if (bitnet_status st = check_device()) return st;
    return launched(launch_gemv_fused(nullptr, acc, scale_act, x, w_packed, nullptr, M, N, K, (hipStream_t)stream));
}

// Which path bitnet_linear takes.  Both give the same bits; the fused kernels
// quantise the activations in every workgroup, which is cheapest for one or
// two rows (or up to four that fit the streaming GEMV's LDS budget), and, on
// the matrix units, for five to eight rows of short K over moderate N, while
// otherwise one quantisation pass plus the GEMM is faster (measured on the
// BitNet-2B-4T and LLaMA-7B projection shapes).
// Longest K for which three or four rows stay on the fused GEMV (its streaming
// kernel holds 4 x K int8 activations in 32 KB of LDS).
constexpr int64_t LINEAR_FUSED_K_MAX_M4 = 8192;
// Five to eight rows take the fused matrix-unit kernel while every workgroup's
// share of quantising (M * K elements) stays this small and the columns do not
// ask for more workgroups than the GPU holds at once (an LM head does).
constexpr int64_t LINEAR_MFMA_MK_MAX = 8 * 2560;
constexpr int64_t LINEAR_MFMA_N_MAX = 65536;

static bool linear_takes_fused(int64_t M, int64_t K) {
    if (M <= 2) return true;
    return M <= 4 && K <= LINEAR_FUSED_K_MAX_M4;
}

static bool linear_takes_mfma(int64_t M, int64_t N, int64_t K, const void* x, const void* w) {
    return M >= 5 && M <= 8 && M * K <= LINEAR_MFMA_MK_MAX && N <= LINEAR_MFMA_N_MAX &&
           bitnet::gemv_mfma_fits(M, N, K, x, w);
}

BITNET_API size_t bitnet_linear_workspace_bytes(int64_t M, int64_t K) {
    if (M < 0 || K <= 0 || K % 4 != 0 || K > BITNET_MAX_K || !sizes_ok(M, 0)) return 0;
    if (linear_takes_fused(M, K)) return 0;
    return round256((size_t)M * (size_t)K) + round256((size_t)M * 2);
}

BITNET_API bitnet_status bitnet_linear(uint16_t* out, const uint16_t* x, const uint8_t* w_packed,
                                       const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K, void* workspace,
                                       size_t workspace_bytes, bitnet_stream_t stream) {
    if (!sizes_ok(M, N)) return BITNET_ERR_SHAPE;
    if (bitnet_status st = check_k(K)) return st;
    if (M == 0 || N == 0) return BITNET_OK;
    if (linear_takes_fused(M, K)) return bitnet_gemv_fused(out, x, w_packed, scale_wt, M, N, K, stream);
    if (!out || !x || !w_packed || !scale_wt) return BITNET_ERR_NULL;
    const size_t need = bitnet_linear_workspace_bytes(M, K);
    if (workspace == nullptr || workspace_bytes < need) return BITNET_ERR_WORKSPACE;
    if (bitnet_status st = check_device()) return st;
    if (linear_takes_mfma(M, N, K, x, w_packed))  // the workspace goes unused
        return launched(bitnet::launch_gemv_mfma(out, nullptr, nullptr, x, w_packed, scale_wt, M, N, K,
                                                 (hipStream_t)stream));
    int8_t* x_int8 = static_cast<int8_t*>(workspace);
    uint16_t* scale_act = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + round256((size_t)M * K));
    hipStream_t s = (hipStream_t)stream;
    if (hipError_t e = launch_quantize(x_int8, scale_act, x, M, K, s)) return launched(e);
    return launched(launch_gemm(out, nullptr, x_int8, w_packed, scale_act, scale_wt, M, N, K, s));
}

// ---------------------------------------------------------------- bitnet_linear without allocation
//
// bitnet_linear_noalloc keeps its workspace (the quantised activations and
// their scales) in this array instead of a caller buffer.  The array exists
// once per device, for as long as the library stays loaded; every call on a
// device shares it (overlapping calls on one device race).  Its host-side name
// is only a handle: the device address is looked up once per device with
// hipGetSymbolAddress and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[BITNET_NOALLOC_SCRATCH_BYTES];

namespace {
std::atomic<uint8_t*> g_scratch[kMaxDevices];

// This device's copy of `scratch` (the current device; check_device has run).
bitnet_status scratch_ptr(uint8_t** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BITNET_ERR_DEVICE;
    uint8_t* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return BITNET_ERR_DEVICE;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return BITNET_OK;
}
}  // namespace

BITNET_API bitnet_status bitnet_linear_noalloc(uint16_t* out, const uint16_t* x, const uint8_t* w_packed,
                                               const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K,
                                               bitnet_stream_t stream) {
    if (!sizes_ok(M, N)) return BITNET_ERR_SHAPE;
    if (bitnet_status st = check_k(K)) return st;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!out || !x || !w_packed || !scale_wt) return BITNET_ERR_NULL;
    const size_t need = bitnet_linear_workspace_bytes(M, K);
    if (need > (size_t)BITNET_NOALLOC_SCRATCH_BYTES) return BITNET_ERR_TOO_LARGE;
    if (need == 0) return bitnet_gemv_fused(out, x, w_packed, scale_wt, M, N, K, stream);
    if (bitnet_status st = check_device()) return st;
    uint8_t* ws = nullptr;
    if (bitnet_status st = scratch_ptr(&ws)) return st;
    // Every byte the GEMM reads is written by the quantiser first, so nothing
    // of the previous call's contents needs clearing.
    return bitnet_linear(out, x, w_packed, scale_wt, M, N, K, ws, need, stream);
}

BITNET_API bitnet_status bitnet_quantize_act_f32(int8_t* x_int8, uint16_t* scale_act, const float* x, int64_t M,
                                                 int64_t K, bitnet_stream_t stream) {
    if (!sizes_ok(M, 0)) return BITNET_ERR_SHAPE;
    if (bitnet_status st = check_k(K)) return st;
    if (M == 0) return BITNET_OK;
    if (!x_int8 || !scale_act || !x) return BITNET_ERR_NULL;
    if (bitnet_status st = check_device()) return st;
    return launched(launch_quantize_f32(x_int8, scale_act, x, M, K, (hipStream_t)stream));
}

BITNET_API size_t bitnet_linear_ex_workspace_bytes(int64_t M, int64_t K, int x_dtype) {
    if (x_dtype == BITNET_DTYPE_BF16) return bitnet_linear_workspace_bytes(M, K);
    if (x_dtype != BITNET_DTYPE_F32) return 0;
    if (M < 0 || K <= 0 || K % 4 != 0 || K > BITNET_MAX_K || !sizes_ok(M, 0)) return 0;
    return round256((size_t)M * (size_t)K) + round256((size_t)M * 2);
}

BITNET_API bitnet_status bitnet_linear_ex(uint16_t* out, const void* x, int x_dtype, const uint8_t* w_packed,
                                          const uint16_t* scale_wt, const uint16_t* bias, int64_t M, int64_t N,
                                          int64_t K, void* workspace, size_t workspace_bytes,
                                          bitnet_stream_t stream) {
    if (x_dtype != BITNET_DTYPE_BF16 && x_dtype != BITNET_DTYPE_F32) return BITNET_ERR_VALUE;
    if (!sizes_ok(M, N)) return BITNET_ERR_SHAPE;
    if (bitnet_status st = check_k(K)) return st;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!out || !x || !w_packed || !scale_wt) return BITNET_ERR_NULL;
    bitnet_status st;
    const size_t need = bitnet_linear_ex_workspace_bytes(M, K, x_dtype);
    if (x_dtype == BITNET_DTYPE_F32 && (workspace == nullptr || workspace_bytes < need)) return BITNET_ERR_WORKSPACE;
    if (linear_takes_fused(M, K) && gemv_ex_fusable(M, K, x, w_packed)) {
        // one launch: the activations (either type) quantised in the GEMV's
        // prologue, the bias in its epilogue; the workspace is not touched
        if ((st = check_device())) return st;
        return launched(launch_gemv_fused_ex(out, x, x_dtype == BITNET_DTYPE_F32, bias, w_packed, scale_wt, M, N, K,
                                             (hipStream_t)stream));
    }
    if (x_dtype == BITNET_DTYPE_BF16) {
        st = bitnet_linear(out, static_cast<const uint16_t*>(x), w_packed, scale_wt, M, N, K, workspace,
                           workspace_bytes, stream);
    } else {
        if ((st = check_device())) return st;
        int8_t* x_int8 = static_cast<int8_t*>(workspace);
        uint16_t* scale_act = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + round256((size_t)M * K));
        hipStream_t s = (hipStream_t)stream;
        if (hipError_t e = launch_quantize_f32(x_int8, scale_act, static_cast<const float*>(x), M, K, s))
            return launched(e);
        st = launched(launch_gemm(out, nullptr, x_int8, w_packed, scale_act, scale_wt, M, N, K, s));
    }
    if (st != BITNET_OK || bias == nullptr) return st;
    return launched(launch_add_bias(out, bias, M, N, (hipStream_t)stream));
}

static bool eps_ok(float eps) { return eps >= 0.0f && eps <= 3.4028234e38f; }  // false for NaN and +inf

BITNET_API bitnet_status bitnet_rmsnorm_quantize(int8_t* x_int8, uint16_t* scale_act, uint16_t* x_norm,
                                                 const uint16_t* x, const uint16_t* gain, float eps, int64_t M,
                                                 int64_t K, bitnet_stream_t stream) {
    if (!sizes_ok(M, 0)) return BITNET_ERR_SHAPE;
    if (bitnet_status st = check_k(K)) return st;
    if (!eps_ok(eps)) return BITNET_ERR_VALUE;
    if (M == 0) return BITNET_OK;
    if (!x_int8 || !scale_act || !x) return BITNET_ERR_NULL;
    if (bitnet_status st = check_device()) return st;
    return launched(launch_quantize_rms(x_int8, scale_act, x_norm, x, gain, eps, M, K, (hipStream_t)stream));
}

BITNET_API size_t bitnet_linear_rms_workspace_bytes(int64_t M, int64_t K) {
    if (M < 0 || K <= 0 || K % 4 != 0 || K > BITNET_MAX_K || !sizes_ok(M, 0)) return 0;
    return round256((size_t)M * (size_t)K) + round256((size_t)M * 2);
}

BITNET_API bitnet_status bitnet_linear_rms(uint16_t* out, const uint16_t* x, const uint16_t* gain, float eps,
                                           const uint8_t* w_packed, const uint16_t* scale_wt, int64_t M, int64_t N,
                                           int64_t K, void* workspace, size_t workspace_bytes,
                                           bitnet_stream_t stream) {
    if (!sizes_ok(M, N)) return BITNET_ERR_SHAPE;
    if (bitnet_status st = check_k(K)) return st;
    if (!eps_ok(eps)) return BITNET_ERR_VALUE;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!out || !x || !w_packed || !scale_wt) return BITNET_ERR_NULL;
    const size_t need = bitnet_linear_rms_workspace_bytes(M, K);
    if (workspace == nullptr || workspace_bytes < need) return BITNET_ERR_WORKSPACE;
    if (bitnet_status st = check_device()) return st;
    hipStream_t s = (hipStream_t)stream;
    if (gemv_rms_fusable(M, K, x, w_packed, gain))
        return launched(launch_gemv_fused_rms(out, nullptr, x, gain, eps, w_packed, scale_wt, M, N, K, s));
    int8_t* x_int8 = static_cast<int8_t*>(workspace);
    uint16_t* scale_act = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + round256((size_t)M * K));
    if (hipError_t e = launch_quantize_rms(x_int8, scale_act, nullptr, x, gain, eps, M, K, s)) return launched(e);
    return launched(launch_gemm(out, nullptr, x_int8, w_packed, scale_act, scale_wt, M, N, K, s));
}

BITNET_API bitnet_status bitnet_w8a16_gemv(float* y, const uint16_t* x, const int8_t* q, const float* scale,
                                           int64_t M, int64_t N, int64_t K, bitnet_stream_t stream) {
    if (!sizes_ok(M, N) || M > BITNET_W8A16_MAX_M || K <= 0 || K > BITNET_MAX_K) return BITNET_ERR_SHAPE;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!y || !x || !q || !scale) return BITNET_ERR_NULL;
    if (bitnet_status st = check_device()) return st;
    return launched(launch_w8a16(y, x, q, scale, M, N, K, (hipStream_t)stream));
}

BITNET_API bitnet_status bitnet_scale_epilogue(uint16_t* out, const int32_t* acc, const uint16_t* scale_act,
                                               const uint16_t* scale_wt, int64_t M, int64_t N,
                                               bitnet_stream_t stream) {
    if (!sizes_ok(M, N)) return BITNET_ERR_SHAPE;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!out || !acc || !scale_act || !scale_wt) return BITNET_ERR_NULL;
    if (bitnet_status st = check_device()) return st;
    return launched(launch_epilogue(out, acc, scale_act, scale_wt, M, N, (hipStream_t)stream));
}
