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
// out like the split-K path of the ternary GEMM: a block owns 32 (or 64) output
// columns and 32 * MT rows (MT = 1 for M <= 32, else 2; rows past M read as
// zeros), and its KW waves split K into chunks on v_mfma_f32_32x32x16_bf16.
// The main kernel for M >= 3, w8a16_lds_kernel (K % 128 == 0), stages each
// wave's 128-element chunk of both operands through a private LDS region and
// reads the MFMA fragments from there (see its own comment).  w8a16_kernel,
// for other K % 64 == 0 shapes, loads 64- or 128-element chunks straight into
// MFMA registers instead: lane (r, h) loads the int8 weights of its half of
// the chunk of column r and, per MFMA k-step, the matching 8 activations of
// row r, so both operands see the same k order; a ring of D chunks keeps loads
// in flight.  Either way the waves' partial fp32 tiles are summed in LDS in a
// fixed order (deterministic results), scaled and stored.
//
// w8a16_stream_kernel (M <= 2, the decode case).  Padding M to an MFMA tile
// forces the lanes of one load onto 32 different weight rows; for a handful of
// activation rows the multiply-adds are cheap on the vector ALUs instead, so
// the weights are streamed the way the ternary decode GEMV streams them: units
// of 8 rows, 8 lanes per row, each lane 16 contiguous int8 weights per step, so
// one wave instruction reads 8 whole 128-byte lines, with a ring of D loads in
// flight per wave.  The activations are widened to fp32 once per workgroup into
// LDS; each weight is converted exactly to fp32 and fed to one fp32 FMA per
// activation row (every product exact, one rounding per add).  A row's eight
// lane sums are combined by a fixed DPP tree.  When there are too few units of
// rows to fill the GPU (the smaller projections), groups of 2 or 4 waves share
// each unit, every wave taking a contiguous range of its steps, and the groups'
// row sums are added in LDS in a fixed order before the scale.
//
// Fast paths need 16-byte aligned x and q; the stream kernel K % 16 == 0 and
// M * K small enough for LDS, the MFMA kernel K % 64 == 0.  Anything else goes
// to w8a16_plain, one wave per output column.
#include "bitnet_device.h"
#include "launch.h"

namespace bitnet {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// MFMA kernel: 16-byte weight loads per lane and chunk, and the chunk ring
// depth for one and two 32-row activation tiles.  (Chunks of 128 elements, so
// that a wave reads whole 128-byte weight lines, measured slower from M = 8 on:
// the loads are bound by the 32 rows each instruction touches, not by lines
// shared between waves.)
constexpr int64_t W8_LDS_KW8_MAX_N = 8192;  // eight waves per column block up to this N
// Two column tiles per workgroup halve the activation staging per weight byte,
// which dominates once M is large; they pay while there are still enough column
// blocks to fill the chip (measured on the BitNet-2B and LLaMA-7B decode shapes).
constexpr int64_t W8_LDS_NT2_MIN_N = 16384;      // from this N at any M
constexpr int64_t W8_LDS_NT2_MIN_N_M16 = 10240;  // from this N at M >= 16
constexpr int W8_MFMA_NB = 2;
constexpr int W8_MFMA_D = 2;
constexpr int W8_MFMA_D2 = 2;
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

template <int MT, int KW, int D, int NB>
__global__ __launch_bounds__(64 * KW) void w8a16_kernel(float* __restrict__ y, const uint16_t* __restrict__ x,
                                                        const int8_t* __restrict__ q, const float* __restrict__ scale,
                                                        int M, int N, int K) {
    constexpr int BM = 32 * MT;
    constexpr int LDC = 33;  // padded LDS row of a partial tile
    constexpr int CK = 32 * NB;  // K elements per chunk: NB 16-byte weight loads per lane
    constexpr int NS = 2 * NB;   // MFMA k-steps of 16 per chunk
    __shared__ float part[KW][BM * LDC];

    const int n0 = blockIdx.x * 32;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nc = K / CK;
    const int r = lane & 31, h = lane >> 5;

    // rows past M and columns past N lie past the end of their buffers: zeros
    const __amdgpu_buffer_rsrc_t x_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0, M * K * 2, BUFFER_RSRC_WORD3_W8);
    const __amdgpu_buffer_rsrc_t q_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(q), (short)0, N * K, BUFFER_RSRC_WORD3_W8);
    // lane half h owns the chunk's weights 16 * NB * h .. 16 * NB * (h + 1) - 1
    int a_voff[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) a_voff[t] = ((32 * t + r) * K + 16 * NB * h) * 2;
    const int b_voff = (n0 + r) * K + 16 * NB * h;

    struct Chunk {
        v4u a[MT][NS];
        v4u b[NB];
    };
    auto load = [&](int j, Chunk& C) {
        const int c = min(wave + KW * j, nc - 1);  // clamped repeats past the end are never used
#pragma unroll
        for (int i = 0; i < NB; ++i) C.b[i] = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, b_voff, c * CK + 16 * i, 0);
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int s = 0; s < NS; ++s)
                C.a[t][s] = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, a_voff[t], (c * CK + 8 * s) * 2, 0);
    };

    f32x16 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x16{};
    auto compute = [&](const Chunk& C) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
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

// ---------------------------------------------------------------- MFMA kernel, LDS-staged operands
//
// Loading MFMA fragments straight from memory makes each 16-byte-per-lane
// instruction touch 32 rows; that, not the bytes, bounds w8a16_kernel.  Here
// each wave stages its 128-element chunk of both operands in a private LDS
// region, loading the weights as 8 whole 128-byte rows and the activations as
// 4 rows x 256 bytes per instruction, and reads the fragments from padded LDS
// rows (distinct banks): lane (r, h), k-step s, holds elements 64h + 8s ..
// 64h + 8s + 7 of the chunk for both operands.  The next chunk's loads are in
// flight while the current one is multiplied; no barrier is needed until the
// fixed-order sum over the waves.
constexpr int WL_KS = 128;                 // K elements per chunk
constexpr int WL_XROW = WL_KS * 2 + 16;    // bytes per staged activation row (bf16, padded)
constexpr int WL_WROW = WL_KS + 16;        // bytes per staged weight row (int8, padded)

// XR: activation rows staged per chunk (a multiple of 4, at most 32 * MT);
// with XR < 32 * MT (M <= XR, one row tile) the wave zeroes the other rows of
// its stage once and never loads them.
template <int MT, int NT, int KW, int XR>
__global__ __launch_bounds__(64 * KW) void w8a16_lds_kernel(float* __restrict__ y, const uint16_t* __restrict__ x,
                                                            const int8_t* __restrict__ q,
                                                            const float* __restrict__ scale, int M, int N, int K) {
    constexpr int BM = 32 * MT;
    constexpr int BN = 32 * NT;  // NT column tiles share each staged activation chunk
    constexpr int LDC = BN + 1;
    constexpr int XB = BM * WL_XROW;
    constexpr int WB = BN * WL_WROW;
    // With two column tiles the partial tiles reuse the stages' memory after the K
    // loop (two workgroups per CU rather than one); otherwise they have their own.
    constexpr bool OVERLAY = NT > 1;
    constexpr int STAGE_BYTES = KW * (XB + WB);
    constexpr int PART_BYTES = KW * BM * LDC * 4;
    __shared__ __align__(16) uint8_t
        smem[OVERLAY ? (STAGE_BYTES > PART_BYTES ? STAGE_BYTES : PART_BYTES) : STAGE_BYTES + PART_BYTES];
    auto stage = reinterpret_cast<uint8_t(*)[XB + WB]>(smem);
    auto part = reinterpret_cast<float(*)[BM * LDC]>(smem + (OVERLAY ? 0 : STAGE_BYTES));

    const int n0 = blockIdx.x * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nc = K / WL_KS;
    const int r = lane & 31, h = lane >> 5;

    // rows past M and columns past N lie past the end of their buffers: zeros
    const __amdgpu_buffer_rsrc_t x_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0, M * K * 2, BUFFER_RSRC_WORD3_W8);
    const __amdgpu_buffer_rsrc_t q_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(q), (short)0, N * K, BUFFER_RSRC_WORD3_W8);
    // this lane's global pieces: activation rows 4i + lane/16 (16 bytes at
    // lane%16 of the row's 256), weight rows 8i + lane/8 (16 bytes at lane%8)
    const int xr_l = lane >> 4, xp_l = lane & 15;
    const int wr_l = lane >> 3, wp_l = lane & 7;
    uint8_t* const xs = stage[wave];
    uint8_t* const ws = stage[wave] + XB;

    static_assert(XR % 4 == 0 && XR <= BM && (XR == BM || MT == 1), "staged rows: whole load instructions of one tile");
    constexpr int XI = XR / 4;
    if constexpr (XR < BM) {  // rows XR .. BM-1 of this wave's activation stage stay zero
        constexpr int ZW = (BM - XR) * WL_XROW / 16;
        for (int i = lane; i < ZW; i += 64)
            *reinterpret_cast<v4u*>(xs + XR * WL_XROW + 16 * i) = v4u{0u, 0u, 0u, 0u};
    }
    constexpr int WI = BN / 8;
    v4u xg[XI], wg[WI];
    auto load = [&](int c) {
#pragma unroll
        for (int i = 0; i < XI; ++i)
            xg[i] = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, ((4 * i + xr_l) * K) * 2 + 16 * xp_l,
                                                          c * WL_KS * 2, 0);
#pragma unroll
        for (int i = 0; i < WI; ++i)
            wg[i] = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, (n0 + 8 * i + wr_l) * K + 16 * wp_l, c * WL_KS, 0);
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < XI; ++i)
            *reinterpret_cast<v4u*>(xs + (4 * i + xr_l) * WL_XROW + 16 * xp_l) = xg[i];
#pragma unroll
        for (int i = 0; i < WI; ++i)
            *reinterpret_cast<v4u*>(ws + (8 * i + wr_l) * WL_WROW + 16 * wp_l) = wg[i];
    };

    f32x16 acc[MT][NT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u) acc[t][u] = f32x16{};
    auto compute = [&]() {
        v4u bw[NT][4];  // this lane's 64 weights of the chunk per column tile: elements 64h .. 64h + 63
#pragma unroll
        for (int u = 0; u < NT; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                bw[u][i] = *reinterpret_cast<const v4u*>(ws + (32 * u + r) * WL_WROW + 64 * h + 16 * i);
#pragma unroll
        for (int s = 0; s < WL_KS / 16; ++s) {
            bf16x8 af[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t)
                af[t] = __builtin_bit_cast(bf16x8,
                                           *reinterpret_cast<const v4u*>(xs + (32 * t + r) * WL_XROW + 128 * h + 16 * s));
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                const v4u& b = bw[u][s >> 1];
                const bf16x8 bop = (s & 1) ? i8x8_to_bf16x8(b.z, b.w) : i8x8_to_bf16x8(b.x, b.y);
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t], bop, acc[t][u], 0, 0, 0);
            }
        }
    };

    // Nothing is loaded past the wave's last chunk: such a load would only
    // delay the barrier of the partial-tile sum below, which waits for every
    // load in flight.
    const int nj = (nc - 1 - wave) / KW + 1;  // the host guarantees nc >= KW
    load(wave);
    for (int j = 0; j < nj; ++j) {
        store();  // after the previous chunk's fragment reads (same wave: in order)
        if (j + 1 < nj) load(wave + KW * (j + 1));
        compute();
    }

    // ---- partial tiles to LDS (register q of lane l: row 8(q/4) + 4(l/32) + q%4,
    //      column l%32), then a fixed-order sum over the waves, the scale, the store
    if constexpr (OVERLAY) __syncthreads();  // every wave is done with its stage before the tiles overwrite it
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u)
#pragma unroll
            for (int qq = 0; qq < 16; ++qq) {
                const int row = 32 * t + 8 * (qq >> 2) + 4 * h + (qq & 3);
                part[wave][row * LDC + 32 * u + r] = acc[t][u][qq];
            }
    __syncthreads();
    for (int e = tid; e < BM * BN; e += 64 * KW) {
        const int row = e / BN, col = e - row * BN;
        const int gn = n0 + col;
        if (row < M && gn < N) {
            float v = part[0][row * LDC + col];
#pragma unroll
            for (int w = 1; w < KW; ++w) v += part[w][row * LDC + col];
            y[(int64_t)row * N + gn] = v * scale[gn];
        }
    }
}

// ---------------------------------------------------------------- stream kernel (M <= 2)

constexpr int W8_STEP = 128;                // weights of a row per wave step (8 lanes x 16)
constexpr int W8_LDS_BYTES = 65536;         // fp32 activations held per workgroup
constexpr int W8_MAX_STEPS = W8_LDS_BYTES / (W8_STEP * 4);
// Workgroup cap: every workgroup stages all activations, so mid-sized split
// problems run best with fewer, longer workgroups (measured on the BitNet and
// LLaMA decode shapes).
constexpr int W8_STREAM_MAX_BLOCKS = 1024;
constexpr int W8_STREAM_MAX_BLOCKS_SPLIT = 512;  // when units x K parts <= W8_SPLIT_WORK
constexpr int W8_SPLIT_WORK = 8192;
constexpr int W8_STREAM_MAX_M = 2;          // from 3 rows on the MFMA kernel is as fast or faster
// Split K further while (units x K parts) stays below this (fewer for two
// activation rows, whose LDS staging costs twice as much per workgroup).
constexpr int W8_SPLIT_UNITS_M1 = 16384;
constexpr int W8_SPLIT_UNITS_M2 = 4096;

// Loads past a wave's work read this small, always-cached pad instead of
// weight lines (every ring slot is issued unconditionally).
__device__ __align__(256) uint8_t w8_pad[W8_MAX_STEPS * W8_STEP + 64 * 16];

// LDS float index of activation (m, k): 16-element pieces of 64 bytes, whose
// four 16-byte quarters are swapped pairwise in every other group of four
// pieces, so that the eight lanes of a row read eight distinct bank groups.
__device__ __forceinline__ int w8_lds_index(int m, int k, int row_floats) {
    const int p = k >> 4;
    const int i = (k >> 2) & 3;
    return m * row_floats + p * 16 + 4 * (i ^ ((p >> 2) & 1)) + (k & 3);
}

__device__ __forceinline__ float group8_sum_f32(float v) {
    v += __builtin_bit_cast(float, dpp_mov<DPP_QUAD_XOR1>(__builtin_bit_cast(int, v)));
    v += __builtin_bit_cast(float, dpp_mov<DPP_QUAD_XOR2>(__builtin_bit_cast(int, v)));
    v += __builtin_bit_cast(float, dpp_mov<DPP_ROW_HALF_MIRROR>(__builtin_bit_cast(int, v)));
    return v;
}

template <int MT, int D, int KS>
__global__ __launch_bounds__(256) void w8a16_stream_kernel(float* __restrict__ y, const uint16_t* __restrict__ x,
                                                           const int8_t* __restrict__ q,
                                                           const float* __restrict__ scale, int M, int N, int K,
                                                           int steps, int units, int upb) {
    constexpr int WAVES = 4;
    constexpr int NT = WAVES * 64;
    constexpr int WG = WAVES / KS;  // wave groups; the KS waves of a group split K
    extern __shared__ __align__(16) float lds_xf[];  // [MT][steps * W8_STEP], zero past K
    __shared__ float sc_lds[NT];
    __shared__ float part[KS > 1 ? KS : 1][KS > 1 ? NT * MT : 1];  // per-wave row sums when K is split

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wg = wave / KS;  // the wave's group: units wg, wg + WG, ... of the workgroup
    const int kp = wave % KS;  // the wave's part of K: steps [s_begin, s_end)
    const int g = lane >> 3;   // row of the unit
    const int sl = lane & 7;   // 16-weight piece of the step
    const int row_floats = steps * W8_STEP;
    const int s_begin = kp * steps / KS;
    const int s_end = (kp + 1) * steps / KS;  // the host guarantees steps >= KS

    const int ub0 = blockIdx.x * upb;
    const int ub1 = min(ub0 + upb, units);
    const int my_units = (ub0 + wg < ub1) ? (ub1 - 1 - ub0 - wg) / WG + 1 : 0;
    const int items = my_units * (s_end - s_begin);

    // ---- the weight ring (first loads go out before the activation prologue)
    const int last_step = steps - 1;
    const bool ktail = (K % W8_STEP) != 0;
    const uint32_t piece = (uint32_t)(sl * 16);
    // in a partial last step, lanes past the row's end re-read its last 16
    // bytes; their activations in LDS are zero
    const uint32_t piece_last = (uint32_t)min(sl * 16, K - last_step * W8_STEP - 16);
    int lj = 0, lt = s_begin;
    const int8_t* unit_ptr;
    uint32_t voff, voff_last;
    auto set_unit = [&]() {
        const bool live = lj < my_units;  // wave-uniform
        const int u = min(ub0 + wg + WG * min(lj, max(my_units - 1, 0)), units - 1);
        const uint32_t lane_row = (uint32_t)((min(u * 8 + g, N - 1) - u * 8) * K);
        unit_ptr = live ? q + (int64_t)u * 8 * K : reinterpret_cast<const int8_t*>(w8_pad);
        voff = live ? lane_row + piece : (uint32_t)(lane * 16);
        voff_last = live ? lane_row + piece_last : (uint32_t)(lane * 16);
    };
    set_unit();
    auto issue = [&](uint4& dst) {
        const int8_t* b = unit_ptr + lt * W8_STEP;
        dst = load_stream16(b + ((ktail && lt == last_step) ? voff_last : voff));
        if (++lt == s_end) {
            lt = s_begin;
            ++lj;
            set_unit();
        }
    };
    uint4 buf[D];
#pragma unroll
    for (int i = 0; i < D; ++i) issue(buf[i]);

    // ---- activations to LDS as fp32 (8 per thread and pass), weight scales
    const int per_row8 = steps * (W8_STEP / 8);
    for (int idx = tid; idx < MT * per_row8; idx += NT) {
        const int m = idx / per_row8;
        const int k = (idx - m * per_row8) * 8;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (m < M && k < K) v = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + k);
        const float4 lo = make_float4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                                      bf16_to_f32(v.y >> 16));
        const float4 hi = make_float4(bf16_to_f32(v.z & 0xFFFFu), bf16_to_f32(v.z >> 16), bf16_to_f32(v.w & 0xFFFFu),
                                      bf16_to_f32(v.w >> 16));
        *reinterpret_cast<float4*>(lds_xf + w8_lds_index(m, k, row_floats)) = lo;
        *reinterpret_cast<float4*>(lds_xf + w8_lds_index(m, k + 4, row_floats)) = hi;
    }
    const int row0 = ub0 * 8;
    const int nrows = min(ub1 * 8, N) - row0;
    sc_lds[tid] = tid < nrows ? scale[row0 + tid] : 0.0f;
    __syncthreads();

    // ---- stream
    float acc0[MT], acc1[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc0[m] = acc1[m] = 0.0f;
    const int swz = 4 * ((sl >> 2) & 1);
    const float* lds_a = lds_xf + sl * 16 + swz;       // quarters 0 and 2 of this lane's piece
    const float* lds_b = lds_xf + sl * 16 + 4 - swz;   // quarters 1 and 3
    int cj = 0, ct = s_begin;
    auto consume = [&](const uint4& v) {
        float wf[16];
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) wf[j] = (float)(int8_t)(wd[j >> 2] >> (8 * (j & 3)));
        const int off = ct * (8 * 16);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float4 x0 = *reinterpret_cast<const float4*>(lds_a + m * row_floats + off);
            const float4 x1 = *reinterpret_cast<const float4*>(lds_b + m * row_floats + off);
            const float4 x2 = *reinterpret_cast<const float4*>(lds_a + m * row_floats + off + 8);
            const float4 x3 = *reinterpret_cast<const float4*>(lds_b + m * row_floats + off + 8);
            acc0[m] = __builtin_fmaf(x0.x, wf[0], acc0[m]);
            acc1[m] = __builtin_fmaf(x0.y, wf[1], acc1[m]);
            acc0[m] = __builtin_fmaf(x0.z, wf[2], acc0[m]);
            acc1[m] = __builtin_fmaf(x0.w, wf[3], acc1[m]);
            acc0[m] = __builtin_fmaf(x1.x, wf[4], acc0[m]);
            acc1[m] = __builtin_fmaf(x1.y, wf[5], acc1[m]);
            acc0[m] = __builtin_fmaf(x1.z, wf[6], acc0[m]);
            acc1[m] = __builtin_fmaf(x1.w, wf[7], acc1[m]);
            acc0[m] = __builtin_fmaf(x2.x, wf[8], acc0[m]);
            acc1[m] = __builtin_fmaf(x2.y, wf[9], acc1[m]);
            acc0[m] = __builtin_fmaf(x2.z, wf[10], acc0[m]);
            acc1[m] = __builtin_fmaf(x2.w, wf[11], acc1[m]);
            acc0[m] = __builtin_fmaf(x3.x, wf[12], acc0[m]);
            acc1[m] = __builtin_fmaf(x3.y, wf[13], acc1[m]);
            acc0[m] = __builtin_fmaf(x3.z, wf[14], acc0[m]);
            acc1[m] = __builtin_fmaf(x3.w, wf[15], acc1[m]);
        }
        if (++ct == s_end) {  // unit complete: combine the row's 8 lanes, then scale and write
            const int ul = wg + WG * cj;
            const int n = (ub0 + ul) * 8 + g;
            const float sc = sc_lds[ul * 8 + g];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float tot = group8_sum_f32(acc0[m] + acc1[m]);
                acc0[m] = acc1[m] = 0.0f;
                if (KS == 1) {
                    if (m == sl && n < N && m < M) y[(int64_t)m * N + n] = tot * sc;
                } else if (m == sl) {
                    part[kp][(ul * 8 + g) * MT + m] = tot;  // combined below
                }
            }
            ct = s_begin;
            ++cj;
        }
    };

    int base = 0;
    for (; base + D <= items; base += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            consume(buf[i]);
            issue(buf[i]);
        }
    }
    const int rem = items - base;
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (i < rem) consume(buf[i]);

    if (KS > 1) {  // the parts of K in a fixed order, then the scale
        __syncthreads();
        for (int idx = tid; idx < nrows * MT; idx += NT) {
            const int r = idx / MT;
            const int m = idx - r * MT;
            float v = part[0][idx];
#pragma unroll
            for (int p = 1; p < KS; ++p) v += part[p][idx];
            if (m < M) y[(int64_t)m * N + row0 + r] = v * sc_lds[r];
        }
    }
}

template <int MT, int D>
hipError_t launch_w8a16_stream_ks(int ks, dim3 grid, size_t lds, hipStream_t s, float* y, const uint16_t* x,
                                  const int8_t* q, const float* scale, int M, int N, int K, int steps, int units,
                                  int upb) {
    if (ks == 4)
        hipLaunchKernelGGL((w8a16_stream_kernel<MT, D, 4>), grid, dim3(256), lds, s, y, x, q, scale, M, N, K, steps,
                           units, upb);
    else if (ks == 2)
        hipLaunchKernelGGL((w8a16_stream_kernel<MT, D, 2>), grid, dim3(256), lds, s, y, x, q, scale, M, N, K, steps,
                           units, upb);
    else
        hipLaunchKernelGGL((w8a16_stream_kernel<MT, D, 1>), grid, dim3(256), lds, s, y, x, q, scale, M, N, K, steps,
                           units, upb);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_w8a16_stream(float* y, const uint16_t* x, const int8_t* q, const float* scale, int M, int N, int K,
                               hipStream_t s) {
    const int steps = (K + W8_STEP - 1) / W8_STEP;
    const int units = (N + 7) / 8;
    // Split K inside the workgroup when there are too few units to give every
    // CU several waves of whole rows.
    int ks = 1;
    const int split_units = MT == 1 ? W8_SPLIT_UNITS_M1 : W8_SPLIT_UNITS_M2;
    while (ks < 4 && units * ks < split_units && steps >= 4 * ks) ks *= 2;
    const int groups = 4 / ks;
    // at most 32 units (256 rows, one scale per thread) per workgroup;
    // otherwise as few workgroups as keep the GPU full
    int blocks = (units + groups - 1) / groups;
    const int max_blocks = units * ks <= W8_SPLIT_WORK ? W8_STREAM_MAX_BLOCKS_SPLIT : W8_STREAM_MAX_BLOCKS;
    if (blocks > max_blocks) blocks = max_blocks;
    if (blocks < (units + 31) / 32) blocks = (units + 31) / 32;
    const int upb = (units + blocks - 1) / blocks;
    blocks = (units + upb - 1) / upb;
    const size_t lds = (size_t)MT * steps * W8_STEP * 4;
    if (steps / ks >= 12)
        return launch_w8a16_stream_ks<MT, MT == 1 ? 16 : 8>(ks, dim3(blocks), lds, s, y, x, q, scale, M, N, K, steps,
                                                            units, upb);
    return launch_w8a16_stream_ks<MT, 8>(ks, dim3(blocks), lds, s, y, x, q, scale, M, N, K, steps, units, upb);
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

// The LDS-staged kernel.  With one row tile and one column tile the activation
// rows staged are rounded up to 4, 8 or 16 only: measured on the BitNet-2B-4T
// and LLaMA-7B shapes 8-18% faster at M = 3-4, 2-8% at M = 8, 1-3% at M = 16;
// with two column tiles (LM heads, wide layers at M >= 16) it was 0.5-4%
// slower, so those stage all 32 rows.
template <int MT, int NT, int KW>
hipError_t launch_w8_lds(dim3 grid, hipStream_t s, float* y, const uint16_t* x, const int8_t* q, const float* scale,
                         int64_t M, int64_t N, int64_t K) {
    const dim3 block(64 * KW);
    if constexpr (MT == 1 && NT == 1) {
        if (M <= 4) {
            hipLaunchKernelGGL((w8a16_lds_kernel<1, NT, KW, 4>), grid, block, 0, s, y, x, q, scale, (int)M, (int)N, (int)K);
            return hipGetLastError();
        }
        if (M <= 8) {
            hipLaunchKernelGGL((w8a16_lds_kernel<1, NT, KW, 8>), grid, block, 0, s, y, x, q, scale, (int)M, (int)N, (int)K);
            return hipGetLastError();
        }
        if (M <= 16) {
            hipLaunchKernelGGL((w8a16_lds_kernel<1, NT, KW, 16>), grid, block, 0, s, y, x, q, scale, (int)M, (int)N, (int)K);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((w8a16_lds_kernel<MT, NT, KW, 32 * MT>), grid, block, 0, s, y, x, q, scale, (int)M, (int)N, (int)K);
    return hipGetLastError();
}

hipError_t launch_w8a16(float* y, const uint16_t* x, const int8_t* q, const float* scale, int64_t M, int64_t N,
                        int64_t K, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int64_t steps = (K + W8_STEP - 1) / W8_STEP;
    if (M <= W8_STREAM_MAX_M && K % 16 == 0 && M * steps <= W8_MAX_STEPS && aligned16(x) && aligned16(q)) {
        if (M == 1) return launch_w8a16_stream<1>(y, x, q, scale, (int)M, (int)N, (int)K, s);
        return launch_w8a16_stream<2>(y, x, q, scale, (int)M, (int)N, (int)K, s);
    }
    constexpr int KW = 4;
    // 32-bit buffer offsets: weight rows up to the last 64-column block's padding, activation rows up to 64
    const bool fits = aligned16(x) && aligned16(q) && (N + 63) * K < ((int64_t)1 << 31) && 64 * K * 2 < ((int64_t)1 << 31);
    const dim3 grid((unsigned)((N + 31) / 32)), block(64 * KW);
    if (fits && K % WL_KS == 0 && K / WL_KS >= KW) {
        constexpr int KW8 = 8;
        const dim3 grid2((unsigned)((N + 63) / 64));
        if (N >= W8_LDS_NT2_MIN_N || (M >= 16 && N >= W8_LDS_NT2_MIN_N_M16)) {
            if (M <= 32) return launch_w8_lds<1, 2, KW>(grid2, s, y, x, q, scale, M, N, K);
            return launch_w8_lds<2, 2, KW>(grid2, s, y, x, q, scale, M, N, K);
        }
        if (M <= 32 && N <= W8_LDS_KW8_MAX_N && K / WL_KS >= KW8) return launch_w8_lds<1, 1, KW8>(grid, s, y, x, q, scale, M, N, K);
        if (M <= 32) return launch_w8_lds<1, 1, KW>(grid, s, y, x, q, scale, M, N, K);
        return launch_w8_lds<2, 1, KW>(grid, s, y, x, q, scale, M, N, K);
    }
    if (fits && K % (32 * W8_MFMA_NB) == 0 && K / (32 * W8_MFMA_NB) >= KW) {
        // whole 128-byte weight lines per wave and chunk
        if (M <= 32)
            hipLaunchKernelGGL((w8a16_kernel<1, KW, W8_MFMA_D, W8_MFMA_NB>), grid, block, 0, s, y, x, q, scale, (int)M,
                               (int)N, (int)K);
        else
            hipLaunchKernelGGL((w8a16_kernel<2, KW, W8_MFMA_D2, W8_MFMA_NB>), grid, block, 0, s, y, x, q, scale,
                               (int)M, (int)N, (int)K);
        return hipGetLastError();
    }
    if (fits && K % 64 == 0 && K / 64 >= KW) {
        if (M <= 32)
            hipLaunchKernelGGL((w8a16_kernel<1, KW, 2, 2>), grid, block, 0, s, y, x, q, scale, (int)M, (int)N, (int)K);
        else
            hipLaunchKernelGGL((w8a16_kernel<2, KW, 2, 2>), grid, block, 0, s, y, x, q, scale, (int)M, (int)N, (int)K);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(w8a16_plain, dim3((unsigned)N), dim3(64), 0, s, y, x, q, scale, (int)M, (int)N, (int)K);
    return hipGetLastError();
}

}  // namespace bitnet
