// w8a16.hip -- INT8 weight-only decode matmul (W8A16).
//
// Computes int8_matmul of "CoolDip00/tiny-llm, src/tinyllm/kernels/int8_gemv.py":
//   y[m][n] = scale[n] * sum_k x[m][k] * q[n][k]
// with bf16 activations x [M][K] (M <= 64), int8 weights q [N][K], fp32 scales
// [N] and fp32 output y [M][N].  As on that page, each int8 weight is read once
// and converted in registers (exact: |q| <= 127 fits a bf16 significand), the
// products accumulate in fp32, and the per-row scale is applied at the end.
//
// At decode the call is bound by reading q (one byte per weight), so it is laid
// out like the split-K path of the ternary GEMM: a block owns 32 output columns
// and 32 * MT rows (MT = 1 for M <= 32, else 2; rows past M read as zeros), and
// its KW waves split K into 64-element chunks.  Operands go from global memory
// straight into v_mfma_f32_32x32x16_bf16 registers: lane (r, h) loads, per chunk,
// the 32 int8 weights 32h .. 32h + 31 of column r (two 16-byte loads) and for
// each of the four MFMA k-steps s the 8 activations 32h + 8s .. 32h + 8s + 7 of
// row r (one 16-byte load), so both operands see the same k order.  A ring of D
// chunks keeps loads in flight.  The waves' partial fp32 tiles are summed in
// LDS in a fixed order (deterministic results), scaled and stored.
//
// Fast path: K % 64 == 0 and 16-byte aligned x and q; otherwise w8a16_plain,
// one wave per output column.
#include "bitnet_device.h"
#include "launch.h"

namespace bitnet {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WQ_CHUNK = 64;  // K elements per chunk (four MFMA k-steps of 16)
// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format;
// stride 0, so bounds are checked against the byte count in word 2).
constexpr int BUFFER_RSRC_WORD3_W8 = 0x00020000;

// Two int8 values (bytes b and b + 1 of p) as a bf16 pair, low element first.
// int8 -> fp32 is exact and leaves the low 16 bits zero, so the bf16 is the
// high half of the fp32 bits.
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t p, int b) {
    const float f0 = (float)(int8_t)(p >> (8 * b));
    const float f1 = (float)(int8_t)(p >> (8 * b + 8));
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1), __builtin_bit_cast(uint32_t, f0), 0x07060302u);
}

__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t p0, uint32_t p1) {
    const v4u v = {i8x2_to_bf16x2(p0, 0), i8x2_to_bf16x2(p0, 2), i8x2_to_bf16x2(p1, 0), i8x2_to_bf16x2(p1, 2)};
    return __builtin_bit_cast(bf16x8, v);
}

template <int MT, int KW, int D>
__global__ __launch_bounds__(64 * KW) void w8a16_kernel(float* __restrict__ y, const uint16_t* __restrict__ x,
                                                        const int8_t* __restrict__ q, const float* __restrict__ scale,
                                                        int M, int N, int K) {
    constexpr int BM = 32 * MT;
    constexpr int LDC = 33;  // padded LDS row of a partial tile
    __shared__ float part[KW][BM * LDC];

    const int n0 = blockIdx.x * 32;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nc = K / WQ_CHUNK;
    const int r = lane & 31, h = lane >> 5;

    // rows past M and columns past N lie past the end of their buffers: zeros
    const __amdgpu_buffer_rsrc_t x_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0, M * K * 2, BUFFER_RSRC_WORD3_W8);
    const __amdgpu_buffer_rsrc_t q_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(q), (short)0, N * K, BUFFER_RSRC_WORD3_W8);
    int a_voff[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) a_voff[t] = ((32 * t + r) * K + 32 * h) * 2;
    const int b_voff = (n0 + r) * K + 32 * h;

    struct Chunk {
        v4u a[MT][4];
        v4u b[2];
    };
    auto load = [&](int j, Chunk& C) {
        const int c = min(wave + KW * j, nc - 1);  // clamped repeats past the end are never used
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                C.a[t][s] = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, a_voff[t], (c * WQ_CHUNK + 8 * s) * 2, 0);
        C.b[0] = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, b_voff, c * WQ_CHUNK, 0);
        C.b[1] = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, b_voff, c * WQ_CHUNK + 16, 0);
    };

    f32x16 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x16{};
    auto compute = [&](const Chunk& C) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v4u& bw = C.b[s >> 1];
            const bf16x8 bop = (s & 1) ? i8x8_to_bf16x8(bw.z, bw.w) : i8x8_to_bf16x8(bw.x, bw.y);
#pragma unroll
            for (int t = 0; t < MT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, C.a[t][s]), bop, acc[t],
                                                                  0, 0, 0);
        }
    };

    const int nj = (nc - 1 - wave) / KW + 1;  // the host guarantees nc >= KW
    Chunk ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i) load(i, ring[i]);
    int j = 0;
    for (; j + D <= nj; j += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            compute(ring[i]);
            load(j + D + i, ring[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (j + i < nj) compute(ring[i]);

    // ---- partial tiles to LDS (register q of lane l: row 8(q/4) + 4(l/32) + q%4,
    //      column l%32), then a fixed-order sum over the waves, the scale, the store
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int qq = 0; qq < 16; ++qq) {
            const int row = 32 * t + 8 * (qq >> 2) + 4 * h + (qq & 3);
            part[wave][row * LDC + r] = acc[t][qq];
        }
    __syncthreads();
    for (int e = tid; e < BM * 32; e += 64 * KW) {
        const int row = e >> 5, col = e & 31;
        const int gn = n0 + col;
        if (row < M && gn < N) {
            float v = part[0][row * LDC + col];
#pragma unroll
            for (int w = 1; w < KW; ++w) v += part[w][row * LDC + col];
            y[(int64_t)row * N + gn] = v * scale[gn];
        }
    }
}

// Any shape: one wave per output column, fp32 partial sums per lane, a fixed
// DPP/readlane tree across the wave.
__global__ __launch_bounds__(64) void w8a16_plain(float* __restrict__ y, const uint16_t* __restrict__ x,
                                                  const int8_t* __restrict__ q, const float* __restrict__ scale,
                                                  int M, int N, int K) {
    const int n = blockIdx.x;
    const int lane = threadIdx.x;
    for (int m = 0; m < M; ++m) {
        float s = 0.0f;
        for (int k = lane; k < K; k += 64)
            s += bf16_to_f32(x[(int64_t)m * K + k]) * (float)q[(int64_t)n * K + k];
        s += __builtin_bit_cast(float, dpp_mov<DPP_QUAD_XOR1>(__builtin_bit_cast(int, s)));
        s += __builtin_bit_cast(float, dpp_mov<DPP_QUAD_XOR2>(__builtin_bit_cast(int, s)));
        s += __builtin_bit_cast(float, dpp_mov<DPP_ROW_HALF_MIRROR>(__builtin_bit_cast(int, s)));
        s += __builtin_bit_cast(float, dpp_mov<DPP_ROW_MIRROR>(__builtin_bit_cast(int, s)));
        const float t0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 0));
        const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 16));
        const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 32));
        const float t3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 48));
        if (lane == 0) y[(int64_t)m * N + n] = ((t0 + t1) + (t2 + t3)) * scale[n];
    }
}

}  // namespace

hipError_t launch_w8a16(float* y, const uint16_t* x, const int8_t* q, const float* scale, int64_t M, int64_t N,
                        int64_t K, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    constexpr int KW = 4;
    const int64_t nc = K / WQ_CHUNK;
    // 32-bit buffer offsets: weights and activations below 2 GiB
    const bool fast = K % WQ_CHUNK == 0 && nc >= KW && aligned16(x) && aligned16(q) &&
                      (N + 31) * K < ((int64_t)1 << 31) && 64 * K * 2 < ((int64_t)1 << 31);
    if (!fast) {
        hipLaunchKernelGGL(w8a16_plain, dim3((unsigned)N), dim3(64), 0, s, y, x, q, scale, (int)M, (int)N, (int)K);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((N + 31) / 32)), block(64 * KW);
    if (M <= 32)
        hipLaunchKernelGGL((w8a16_kernel<1, KW, 2>), grid, block, 0, s, y, x, q, scale, (int)M, (int)N, (int)K);
    else
        hipLaunchKernelGGL((w8a16_kernel<2, KW, 2>), grid, block, 0, s, y, x, q, scale, (int)M, (int)N, (int)K);
    return hipGetLastError();
}

}  // namespace bitnet
