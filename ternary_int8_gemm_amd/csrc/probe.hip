// probe.hip -- machine-ceiling microbenchmarks used by the benchmark script
// (libbitnet_probe.so, separate from the layer's library and its C ABI).
//
// The layer's kernels are measured against MI355X's published peaks (HBM3E
// 8 TB/s, dense int8 MFMA 5.0 POPS).  These kernels measure what this box
// actually delivers for the same two resources, so that a kernel's fraction of
// the published peak can be read against a practical ceiling:
//   probe_read      streams a buffer with 16-byte loads and reduces it (HBM read)
//   probe_copy      copies a buffer with 16-byte loads and stores (HBM read + write)
//   probe_mfma_i8   back-to-back v_mfma_i32_32x32x32_i8 on register operands
//   probe_gemm_loop the ternary GEMM's inner loop alone (LDS fragment reads,
//                   weight-code expansion, MFMAs) on operand data distributed
//                   like the prefill workload's
// The two MFMA probes also read the shader-clock counter (s_memtime) and the
// constant 100 MHz counter (s_memrealtime) around their loops in one wave,
// which gives the shader clock while the matrix units are loaded.  The
// matrix units' power depends on the operand bits: probe_mfma_i8 repeats a
// few small register operands, probe_gemm_loop changes them every MFMA as the
// GEMM does, and the clock the chip sustains differs accordingly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define PROBE_API extern "C" __attribute__((visibility("default")))

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int PR_UNROLL = 8;               // 16-byte loads in flight per lane

// Each wave takes whole segments of 64 lanes x PR_UNROLL x 16 bytes (8 KB),
// grid-stride; a tail shorter than a segment is read 16 bytes per lane.  The
// XOR of everything read is written once per thread into sink (so the loads
// cannot be dropped).
__global__ __launch_bounds__(256) void probe_read_kernel(const v4u* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t segs = n16 / (64 * PR_UNROLL);
    uint32_t x = 0;
    for (int64_t s = wave; s < segs; s += waves) {
        const v4u* p = src + s * (64 * PR_UNROLL) + lane;
        v4u v[PR_UNROLL];
#pragma unroll
        for (int i = 0; i < PR_UNROLL; ++i) v[i] = __builtin_nontemporal_load(p + 64 * i);
#pragma unroll
        for (int i = 0; i < PR_UNROLL; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    for (int64_t i = segs * (64 * PR_UNROLL) + wave * 64 + lane; i < n16; i += waves * 64) {
        const v4u v = src[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

__global__ __launch_bounds__(256) void probe_copy_kernel(v4u* __restrict__ dst, const v4u* __restrict__ src,
                                                         int64_t n16) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t segs = n16 / (64 * PR_UNROLL);
    for (int64_t s = wave; s < segs; s += waves) {
        const int64_t base = s * (64 * PR_UNROLL) + lane;
        v4u v[PR_UNROLL];
#pragma unroll
        for (int i = 0; i < PR_UNROLL; ++i) v[i] = __builtin_nontemporal_load(src + base + 64 * i);
#pragma unroll
        for (int i = 0; i < PR_UNROLL; ++i) __builtin_nontemporal_store(v[i], dst + base + 64 * i);
    }
    for (int64_t i = segs * (64 * PR_UNROLL) + wave * 64 + lane; i < n16; i += waves * 64) dst[i] = src[i];
}

// Four independent accumulator chains per wave; operands depend on the lane
// so that nothing folds.  Block 0's wave 0 records both counters.
__global__ __launch_bounds__(256) void probe_mfma_i8_kernel(int32_t* __restrict__ out, int iters,
                                                            uint64_t* __restrict__ clk) {
    const int lane = threadIdx.x & 63;
    const v4i a = {lane, lane * 3, lane ^ 5, 7};
    const v4i b = {lane * 5, 1, lane + 2, lane ^ 9};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const bool timer = blockIdx.x == 0 && threadIdx.x < 64;
    uint64_t t0 = 0, r0 = 0;
    if (timer) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    if (timer) {
        const uint64_t t1 = __builtin_amdgcn_s_memtime();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        if (lane == 0) {
            clk[0] = t1 - t0;
            clk[1] = r1 - r0;
        }
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c0[j] ^ c1[j] ^ c2[j] ^ c3[j];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// A 32-bit integer mixer (murmur3's finaliser), for synthetic operand data.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x85ebca6bu;
    x ^= x >> 13;
    x *= 0xc2b2ae35u;
    x ^= x >> 16;
    return x;
}

// Four signed activation bytes, bell-shaped in -22 .. 23 with standard
// deviation about 8: like the per-token absmax int8 codes of N(0, 1)
// activations whose rows hold outlier channels eight times larger (the
// prefill workload: the absmax is set by an outlier, the mean |code| is about
// 6 and 96 % of the codes lie within +-15).
__device__ __forceinline__ uint32_t activation_bytes(uint32_t h) {
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t a = mix32(h * 4u + j);
        const int code = (int)(a & 15) + (int)((a >> 4) & 15) + (int)((a >> 8) & 15) - 22;
        v |= (uint32_t)(code & 0xff) << (8 * j);
    }
    return v;
}

// Sixteen packed 2-bit weight codes (w + 2 for w in {-1, 0, +1}), P(w = 0) = 0.4.
__device__ __forceinline__ uint32_t weight_codes(uint32_t h) {
    uint32_t p = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t r = mix32(h * 16u + j) % 10u;
        p |= (r < 3 ? 1u : (r < 7 ? 2u : 3u)) << (2 * j);
    }
    return p;
}

// The inner loop of the tiled GEMM for one 128 x 64 wave tile (4 x 2 MFMA
// tiles): per 128-element stage the packed weight dwords of the two column
// tiles and, per 32-element k-step, the four activation fragments are read
// from LDS, each weight dword is expanded into four code dwords, and eight
// MFMAs are issued.  LDS holds one stage; the lanes rotate over it every
// iteration, so operand data changes every MFMA.  No global loads, no
// barriers: the rate this loop reaches bounds the GEMM's.
constexpr int GL_MT = 4, GL_NT = 2;
__global__ __launch_bounds__(256) void probe_gemm_loop_kernel(int32_t* __restrict__ out, int iters,
                                                              uint64_t* __restrict__ clk) {
    constexpr int A_BYTES = GL_MT * 4 * 1024;
    __shared__ __align__(16) uint8_t lds[A_BYTES + GL_NT * 1024];
    const int tid = threadIdx.x, lane = tid & 63;
    for (int i = tid * 4; i < (int)sizeof(lds); i += 256 * 4) {
        const uint32_t h = mix32((uint32_t)i * 2654435761u + blockIdx.x);
        *reinterpret_cast<uint32_t*>(lds + i) = i < A_BYTES ? activation_bytes(h) : weight_codes(h);
    }
    __syncthreads();
    v16i acc[GL_MT][GL_NT];
#pragma unroll
    for (int t = 0; t < GL_MT; ++t)
#pragma unroll
        for (int u = 0; u < GL_NT; ++u) acc[t][u] = v16i{};
    const bool timer = blockIdx.x == 0 && threadIdx.x < 64;
    uint64_t t0 = 0, r0 = 0;
    if (timer) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int it = 0; it < iters; ++it) {
        const int slot = ((lane ^ it) & 63) * 16;
        v4u pb[GL_NT];
#pragma unroll
        for (int u = 0; u < GL_NT; ++u) pb[u] = *reinterpret_cast<const v4u*>(lds + A_BYTES + u * 1024 + slot);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            v4i af[GL_MT];
#pragma unroll
            for (int t = 0; t < GL_MT; ++t) af[t] = *reinterpret_cast<const v4i*>(lds + (t * 4 + s) * 1024 + slot);
#pragma unroll
            for (int u = 0; u < GL_NT; ++u) {
                const uint32_t p = pb[u][s];
                const v4i bf = {(int)(p & 0x03030303u), (int)((p >> 2) & 0x03030303u), (int)((p >> 4) & 0x03030303u),
                                (int)((p >> 6) & 0x03030303u)};
#pragma unroll
                for (int t = 0; t < GL_MT; ++t)
                    acc[t][u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[t], bf, acc[t][u], 0, 0, 0);
            }
        }
    }
    if (timer) {
        const uint64_t t1 = __builtin_amdgcn_s_memtime();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        if (lane == 0) {
            clk[0] = t1 - t0;
            clk[1] = r1 - r0;
        }
    }
    int sum = 0;
#pragma unroll
    for (int t = 0; t < GL_MT; ++t)
#pragma unroll
        for (int u = 0; u < GL_NT; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j) sum += acc[t][u][j];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

}  // namespace

// Reads n_bytes (a multiple of 16, 16-byte aligned src) with `blocks`
// workgroups of 256 threads; sink holds blocks * 256 uint32 (written).
PROBE_API int probe_read(const void* src, int64_t n_bytes, uint32_t* sink, int blocks, void* stream) {
    if (n_bytes % 16 != 0 || ((uintptr_t)src & 15) != 0 || blocks <= 0) return 2;
    hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const v4u*>(src), n_bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

// Copies n_bytes (a multiple of 16, 16-byte aligned buffers) from src to dst.
PROBE_API int probe_copy(void* dst, const void* src, int64_t n_bytes, int blocks, void* stream) {
    if (n_bytes % 16 != 0 || ((uintptr_t)src & 15) != 0 || ((uintptr_t)dst & 15) != 0 || blocks <= 0) return 2;
    hipLaunchKernelGGL(probe_copy_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, static_cast<v4u*>(dst),
                       static_cast<const v4u*>(src), n_bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

// blocks workgroups of 4 waves, each wave 4 * iters MFMAs (32 x 32 x 32 int8,
// 65536 ops each); out holds blocks * 256 int32, clk two uint64 (written):
// shader-clock ticks and 100 MHz ticks across one wave's loop.
PROBE_API int probe_mfma_i8(int32_t* out, int iters, uint64_t* clk, int blocks, void* stream) {
    if (iters <= 0 || blocks <= 0) return 2;
    hipLaunchKernelGGL(probe_mfma_i8_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, clk);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

// blocks workgroups of 4 waves, each wave iters x 32 MFMAs (32 x 32 x 32 int8);
// out holds blocks * 256 int32, clk two uint64 (written), as for probe_mfma_i8.
PROBE_API int probe_gemm_loop(int32_t* out, int iters, uint64_t* clk, int blocks, void* stream) {
    if (iters <= 0 || blocks <= 0) return 2;
    hipLaunchKernelGGL(probe_gemm_loop_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, clk);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}
