// gemv_mfma.hip -- fused quantise + ternary product for a few activation rows
// on int8 MFMA (K-GEMV, 5 <= M <= 16).
//
// Computes bitnet_gemv_fused of "phanerozoic/bitnet-cpu v1,
// torch-ext/bitnet_cpu/__init__.py" (the fused decode path of the request post
// of "kernels-community/README discussion #1 (bitnet-tc kernel request)") with
// the same bits as quantize_activation followed by bitnet_gemm:
//   q = quantize_activation(x)                          (per row, in-kernel)
//   acc[m][n] = sum_k (code[n][k] - 2) * q[m][k]        (exact int32)
//   out[m][n] = epilogue(acc, bf16(s_m), scale_wt[n])
//
// Why a second fused kernel.  The dot4 streaming GEMV reads every quantised
// activation word from LDS once per activation row and weight word: at 16 rows
// that is 64 bytes of LDS per byte of weights, far more than the LDS delivers
// at HBM rate.  On the matrix units the same product costs one 1 KB fragment
// read per 32 x 32 x 32 MFMA, i.e. 2-3 bytes of LDS per weight byte.
//
// Layout on gfx950:
//  * One 1024-thread workgroup (16 waves) quantises the activation rows once:
//    the row absmax (each wave reduces its lanes per row with DPP, then one lane
//    per row takes an LDS max), then each thread quantises 16-element groups
//    into LDS as int8, every group 4x4-byte transposed (the k order of the
//    expanded weight dwords, as in the GEMM), with the row sums of q for the
//    -2 * sum_k q correction.  K is held in chunks of
//    at most 8192 elements (128 KB of LDS; the first chunk's activations stay
//    in registers between the absmax and the quantisation).
//  * Each wave owns one 32-column tile and one of KS interleaved parts of its
//    128-element K stages.  Per stage a lane loads the 16 packed bytes of its
//    column (lane (n, h): bytes 32 st + 16 h of row n0 + n), which hold its B
//    operand dwords for the stage's four k-steps; a ring of D stages is kept in
//    flight from the kernel's start, so the weights stream during the prologue
//    (slots past a wave's last stage read gq_pad, a small array that stays
//    cached, so that every ring load is still issued).
//  * v_mfma_i32_32x32x32_i8 with rows 0..M-1 from LDS (lanes of the other rows
//    feed zeros and read nothing), the codes (1, 2, 3) as B; the accumulator
//    rows 0..M-1 are the output rows.
//  * With KS > 1 the parts of a tile are added through LDS (int32, exact,
//    order-free), then the block writes the epilogue row-major.
// Needs K % 128 == 0, 16-byte aligned x and w, and N * K / 4 < 2^31 (32-bit
// buffer offsets).
#include "bitnet_device.h"
#include "launch.h"

namespace bitnet {

namespace {

constexpr int GQ_WAVES = 16;
constexpr int GQ_THREADS = GQ_WAVES * 64;
constexpr int GQ_ROWS = 16;                  // activation rows held (rows past M are zero)
constexpr int GQ_KC_MAX = 8192;              // K elements of quantised activations per chunk
constexpr int GQ_STAGE = 128;                // K elements per weight load (4 MFMA k-steps)
constexpr int GQ_PAD = 16;                   // bytes of padding per LDS row (bank spread)
constexpr int GQ_XG = GQ_ROWS * GQ_KC_MAX / 16 / GQ_THREADS;  // 16-element groups per thread (4)
constexpr int GQ_RSRC_WORD3 = 0x00020000;    // raw buffer resource, 32-bit data, bounds-checked

// Target of the ring's loads past a wave's last stage (never consumed): one
// 16-byte piece per lane of a small array that stays in the CU's cache, so the
// barrier after the last stage does not wait on weight lines for them.
__device__ __align__(256) uint8_t gq_pad[64 * 16];

// LDS byte offset of 16-element group g of activation row m (row stride kc + GQ_PAD).
__device__ __forceinline__ int gq_slot(int m, int g, int kc) { return m * (kc + GQ_PAD) + g * 16; }

template <int KS, int D, bool OUT_I32>
__global__ __launch_bounds__(GQ_THREADS) void gemv_mfma_kernel(uint16_t* __restrict__ out,
                                                               int32_t* __restrict__ acc_out,
                                                               uint16_t* __restrict__ sa_out,
                                                               const uint16_t* __restrict__ x,
                                                               const uint8_t* __restrict__ w,
                                                               const uint16_t* __restrict__ sw, int M, int N, int K,
                                                               int KC) {
    constexpr int TPB = GQ_WAVES / KS;  // column tiles per workgroup
    extern __shared__ __align__(16) uint8_t lds[];  // [GQ_ROWS][KC + GQ_PAD] quantised x; reused for the K parts
    __shared__ uint32_t s_amax[GQ_ROWS];
    __shared__ int s_rsum[GQ_ROWS];
    __shared__ float s_saf[GQ_ROWS];
    __shared__ QuantScale s_qs[GQ_ROWS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kp = wave % KS;        // K part of this wave
    const int tl = wave / KS;        // tile within the workgroup
    const int r = lane & 31, h = lane >> 5;
    const int n0 = (blockIdx.x * TPB + tl) * 32;  // first column of the tile (may lie past N: zeros, dropped)
    const int KB = K >> 2;
    const int nst = K / GQ_STAGE;
    const int nchunks = (K + KC - 1) / KC;
    const int gpr = KC / 16;  // 16-element groups per row in a chunk

    if (tid < GQ_ROWS) {
        s_amax[tid] = 0u;
        s_rsum[tid] = 0;
    }

    // ---- chunk 0 of x: this thread's 16-element groups (row gi / gpr), two 16-byte loads each
    const int len0 = min(K, KC);
    v4u xr[GQ_XG][2];
#pragma unroll
    for (int i = 0; i < GQ_XG; ++i) {
        const int gi = tid + GQ_THREADS * i;
        const int m = gi / gpr, g = gi - m * gpr;
        if (m < M && g * 16 < len0) {
            const v4u* src = reinterpret_cast<const v4u*>(x + (int64_t)m * K + g * 16);
            xr[i][0] = src[0];
            xr[i][1] = src[1];
        } else {
            xr[i][0] = xr[i][1] = v4u{0u, 0u, 0u, 0u};
        }
    }
    const uint16_t sw_lane = (!OUT_I32 && n0 + r < N) ? sw[n0 + r] : (uint16_t)0;

    // ---- weight ring: item j of chunk c is stage c * (KC / 128) + kp + KS * j
    const int w_voff = (n0 + r) * KB + 16 * h;  // rows past N lie past the buffer's end: zeros
    const int spc = KC / GQ_STAGE;               // stages per chunk
    auto items_of = [&](int c) {
        const int s0 = c * spc, s1 = min(s0 + spc, nst);
        return s1 - s0 > kp ? (s1 - s0 - kp + KS - 1) / KS : 0;
    };
    // item i of chunk c; items past the wave's last one of the chunk read
    // gq_pad instead (never consumed: they keep every ring load unconditional,
    // so the compiler's waits stay exact).  Uniform selects, no branch.
    auto issue = [&](int c, int i, int items) -> v4u {
        const bool live = i < items;  // wave-uniform
        const int st = c * spc + kp + KS * (live ? i : 0);
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            live ? const_cast<uint8_t*>(w) : gq_pad, (short)0, live ? N * KB : (int)sizeof(gq_pad), GQ_RSRC_WORD3);
        return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rsrc, live ? w_voff : lane * 16,
                                                                             live ? st * (GQ_STAGE / 4) : 0, 0));
    };
    v4u buf[D];
    int items = items_of(0);
#pragma unroll
    for (int i = 0; i < D; ++i) buf[i] = issue(0, i, items);

    __syncthreads();  // s_amax / s_rsum cleared

    // Row reductions: the 64 lanes of a wave hold consecutive groups, i.e. a few
    // consecutive rows; each row's lanes are combined in the wave (DPP) and one
    // lane per row updates LDS, instead of every lane hitting one LDS word.
    auto rows_of_wave = [&](int m, int& lo, int& hi) {  // rows past M hold nothing to reduce
        lo = __builtin_amdgcn_readfirstlane(m);
        hi = min(__builtin_amdgcn_readlane(m, 63), M - 1);
    };
    auto row_max = [&](int m, uint32_t v) {
        int lo, hi;
        rows_of_wave(m, lo, hi);
        for (int mm = lo; mm <= hi; ++mm) {
            const uint32_t u = wave_max_u32(m == mm ? v : 0u);
            if (lane == 0) atomicMax(&s_amax[mm], u);
        }
    };
    auto row_sum = [&](int m, int v) {
        int lo, hi;
        rows_of_wave(m, lo, hi);
        for (int mm = lo; mm <= hi; ++mm) {
            const int u = wave_sum_i32(m == mm ? v : 0);
            if (lane == 0 && u != 0) atomicAdd(&s_rsum[mm], u);
        }
    };

    // ---- row absmax: chunk 0 from registers, later chunks read (not kept)
    auto group_absmax = [&](const v4u& a, const v4u& b) {
        return max(max(max(absmax_bf16x2(a.x), absmax_bf16x2(a.y)), max(absmax_bf16x2(a.z), absmax_bf16x2(a.w))),
                   max(max(absmax_bf16x2(b.x), absmax_bf16x2(b.y)), max(absmax_bf16x2(b.z), absmax_bf16x2(b.w))));
    };
#pragma unroll
    for (int i = 0; i < GQ_XG; ++i) {
        const int gi = tid + GQ_THREADS * i;
        row_max(gi / gpr, group_absmax(xr[i][0], xr[i][1]));  // padding groups hold zeros
    }
    // later chunks: wave-uniform trip counts (every lane takes part in the reductions)
    for (int c = 1; c < nchunks; ++c) {
        const int len = min(K - c * KC, KC);
        for (int base = wave * 64; base < M * gpr; base += GQ_THREADS) {
            const int gi = base + lane;
            const int m = gi / gpr, g = gi - m * gpr;
            uint32_t v = 0u;
            if (m < M && g * 16 < len) {
                const v4u* src = reinterpret_cast<const v4u*>(x + (int64_t)m * K + c * KC + g * 16);
                v = group_absmax(src[0], src[1]);
            }
            row_max(m, v);
        }
    }
    __syncthreads();  // row absmax final
    if (tid < GQ_ROWS) {  // the row scales, once per workgroup
        const QuantScale qs = quant_scale(s_amax[tid]);
        const uint16_t sb = f32_to_bf16(qs.s);
        s_qs[tid] = qs;
        s_saf[tid] = bf16_to_f32(sb);
        if (sa_out != nullptr && blockIdx.x == 0 && tid < M) sa_out[tid] = sb;
    }
    __syncthreads();

    // Quantise one group of a row below M into LDS; returns its byte sum (for
    // the row sums of q).  Nothing is written for other groups: rows M .. 15
    // are never read, nor are groups past K.
    auto put_group = [&](int m, int g, const v4u& a, const v4u& b, bool live) -> int {
        int sq = 0;
        if (live) {
            const QuantScale qs = s_qs[m];
            const uint2 qa = quantize_bf16x8(make_uint4(a.x, a.y, a.z, a.w), qs);
            const uint2 qb = quantize_bf16x8(make_uint4(b.x, b.y, b.z, b.w), qs);
            sq = __builtin_amdgcn_sdot4((int)qa.x, 0x01010101, 0, false);
            sq = __builtin_amdgcn_sdot4((int)qa.y, 0x01010101, sq, false);
            sq = __builtin_amdgcn_sdot4((int)qb.x, 0x01010101, sq, false);
            sq = __builtin_amdgcn_sdot4((int)qb.y, 0x01010101, sq, false);
            *reinterpret_cast<uint4*>(lds + gq_slot(m, g, KC)) = transpose4x4(qa.x, qa.y, qb.x, qb.y);
        }
        return sq;
    };

    // chunk 0 from the registers loaded above
#pragma unroll
    for (int i = 0; i < GQ_XG; ++i) {
        const int gi = tid + GQ_THREADS * i;
        const int m = gi / gpr, g = gi - m * gpr;
        row_sum(m, put_group(m, g, xr[i][0], xr[i][1], m < M));
        __builtin_amdgcn_sched_barrier(0);  // one group's temporaries at a time
    }

    v16i acc = v16i{};
    const int a_rd = (r < GQ_ROWS) ? gq_slot(r, 4 * h, KC) : 0;  // this lane's row, lane-half group offset
    for (int c = 0; c < nchunks; ++c) {
        if (c > 0) {
            const int len = min(K - c * KC, KC);
            __syncthreads();  // every wave is done with chunk c - 1
            for (int base = wave * 64; base < M * gpr; base += GQ_THREADS) {
                const int gi = base + lane;
                const int m = gi / gpr, g = gi - m * gpr;
                const bool live = m < M && g * 16 < len;
                v4u a = v4u{0u, 0u, 0u, 0u}, b = a;
                if (live) {
                    const v4u* src = reinterpret_cast<const v4u*>(x + (int64_t)m * K + c * KC + g * 16);
                    a = src[0];
                    b = src[1];
                }
                row_sum(m, put_group(m, g, a, b, live));
            }
        }
        __syncthreads();  // chunk c quantised

        // ---- this wave's stages of chunk c
        auto consume = [&](const v4u& pw, int i) {
            const int gbase = (kp + KS * i) * 8;  // first group of the stage within the chunk
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t p = pw[s];
                const v4i bf = {(int)(p & CODE_MASK), (int)((p >> 2) & CODE_MASK), (int)((p >> 4) & CODE_MASK),
                                (int)((p >> 6) & CODE_MASK)};
                v4i af = v4i{0, 0, 0, 0};
                if (r < M) af = *reinterpret_cast<const v4i*>(lds + a_rd + (gbase + s) * 16);
                acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf, acc, 0, 0, 0);
            }
        };
        int base = 0;
        for (; base + D <= items; base += D) {
#pragma unroll
            for (int i = 0; i < D; ++i) {
                consume(buf[i], base + i);
                buf[i] = issue(c, base + i + D, items);
            }
        }
        const int rem = items - base;
#pragma unroll
        for (int i = 0; i < D; ++i)
            if (i < rem) consume(buf[i], base + i);
        if (c + 1 < nchunks) {  // refill the ring with the next chunk's first stages
            items = items_of(c + 1);
#pragma unroll
            for (int i = 0; i < D; ++i) buf[i] = issue(c + 1, i, items);
        }
    }

    // ---- accumulator register j of lane l: row 8 (j / 4) + 4 h + j % 4, column l % 32.
    // Rows 0..15 are registers 0..7.
    if constexpr (KS == 1) {
        const int n = n0 + r;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int m = 8 * (j >> 2) + 4 * h + (j & 3);
            if (m < M && n < N) {
                const int v = acc[j] - 2 * s_rsum[m];
                if (OUT_I32)
                    acc_out[(int64_t)m * N + n] = v;
                else
                    out[(int64_t)m * N + n] = epilogue_bf16(v, s_saf[m], bf16_to_f32(sw_lane));
            }
        }
    } else {
        // The K parts of each tile meet in LDS (the activation chunk is no
        // longer read): part kp of tile t stores its rows 0..15 in slot
        // [t][kp], and the parts are added in a fixed order.
        int* red = reinterpret_cast<int*>(lds);  // [TPB][KS][GQ_ROWS][32]
        __syncthreads();                         // every wave is done reading the chunk
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int m = 8 * (j >> 2) + 4 * h + (j & 3);
            red[((tl * KS + kp) * GQ_ROWS + m) * 32 + r] = acc[j];
        }
        __syncthreads();
        for (int i = tid; i < TPB * M * 32; i += GQ_THREADS) {
            const int t = i / (M * 32);
            const int e = i - t * (M * 32);
            const int m = e >> 5, col = e & 31;
            const int n = (blockIdx.x * TPB + t) * 32 + col;
            if (n < N) {
                int v = -2 * s_rsum[m];
#pragma unroll
                for (int q = 0; q < KS; ++q) v += red[((t * KS + q) * GQ_ROWS + m) * 32 + col];
                if (OUT_I32)
                    acc_out[(int64_t)m * N + n] = v;
                else
                    out[(int64_t)m * N + n] = epilogue_bf16(v, s_saf[m], bf16_to_f32(sw[n]));
            }
        }
    }
}

// Bytes of dynamic LDS: the activation chunk, or the K parts' tiles if larger.
constexpr size_t gq_lds_bytes(int KC, int KS) {
    const size_t xq = (size_t)GQ_ROWS * (KC + GQ_PAD);
    const size_t parts = KS > 1 ? (size_t)GQ_WAVES * GQ_ROWS * 32 * 4 : 0;
    return xq > parts ? xq : parts;
}

template <int KS, bool OUT_I32>
hipError_t launch_ks(uint16_t* out, int32_t* acc, uint16_t* sa_out, const uint16_t* x, const uint8_t* w,
                     const uint16_t* sw, int M, int N, int K, int KC, hipStream_t s) {
    constexpr int TPB = GQ_WAVES / KS;
    const int tiles = (N + 31) / 32;
    const unsigned blocks = (unsigned)((tiles + TPB - 1) / TPB);
    const size_t lds = gq_lds_bytes(KC, KS);
    auto kern = gemv_mfma_kernel<KS, 4, OUT_I32>;
    if (lds > 65536) {
        const hipError_t e = raise_lds_limit(kern, lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(GQ_THREADS), lds, s, out, acc, sa_out, x, w, sw, M, N, K, KC);
    return hipGetLastError();
}

}  // namespace

bool gemv_mfma_fits(int64_t M, int64_t N, int64_t K, const void* x, const void* w) {
    return M >= 1 && M <= GQ_ROWS && K % GQ_STAGE == 0 && aligned16(x) && aligned16(w) &&
           N * (K / 4) < ((int64_t)1 << 31);
}

hipError_t launch_gemv_mfma(uint16_t* out, int32_t* acc, uint16_t* scale_act_out, const uint16_t* x,
                            const uint8_t* w, const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K,
                            hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (!gemv_mfma_fits(M, N, K, x, w)) return hipErrorInvalidValue;
    const int m = (int)M, n = (int)N, k = (int)K;
    const int KC = k < GQ_KC_MAX ? k : GQ_KC_MAX;
    // K parts per tile: as many as keep the workgroups (one per CU: 16 waves
    // of at most 80 registers) within one round of 256 CUs, and at least one
    // stage per part.
    const int tiles = (n + 31) / 32;
    const int nst = k / GQ_STAGE;
    int ks = 1;
    while (ks < 16 && nst >= 2 * ks && (tiles * 2 * ks + GQ_WAVES - 1) / GQ_WAVES <= 256) ks *= 2;
    if (acc != nullptr) {
        switch (ks) {
            case 1: return launch_ks<1, true>(nullptr, acc, scale_act_out, x, w, scale_wt, m, n, k, KC, s);
            case 2: return launch_ks<2, true>(nullptr, acc, scale_act_out, x, w, scale_wt, m, n, k, KC, s);
            case 4: return launch_ks<4, true>(nullptr, acc, scale_act_out, x, w, scale_wt, m, n, k, KC, s);
            case 8: return launch_ks<8, true>(nullptr, acc, scale_act_out, x, w, scale_wt, m, n, k, KC, s);
            default: return launch_ks<16, true>(nullptr, acc, scale_act_out, x, w, scale_wt, m, n, k, KC, s);
        }
    }
    switch (ks) {
        case 1: return launch_ks<1, false>(out, nullptr, scale_act_out, x, w, scale_wt, m, n, k, KC, s);
        case 2: return launch_ks<2, false>(out, nullptr, scale_act_out, x, w, scale_wt, m, n, k, KC, s);
        case 4: return launch_ks<4, false>(out, nullptr, scale_act_out, x, w, scale_wt, m, n, k, KC, s);
        case 8: return launch_ks<8, false>(out, nullptr, scale_act_out, x, w, scale_wt, m, n, k, KC, s);
        default: return launch_ks<16, false>(out, nullptr, scale_act_out, x, w, scale_wt, m, n, k, KC, s);
    }
}

}  // namespace bitnet
