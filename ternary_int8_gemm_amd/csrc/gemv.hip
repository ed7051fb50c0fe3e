// gemv.hip -- fused quantise + ternary GEMV for the decode case (K-GEMV).
//
// Computes bitnet_gemv_fused of "phanerozoic/bitnet-cpu v1,
// torch-ext/bitnet_cpu/__init__.py" (the fused decode path named in the
// request post of "kernels-community/README discussion #1 (bitnet-tc kernel
// request)") for M <= 15 activation rows:
//   q = quantize_activation(x)            (in-kernel, bit-identical to K-QUANT)
//   acc[m][n] = sum_k (code[n][k] - 2) * q[m][k]     (exact int32)
//   out[m][n] = epilogue(acc, bf16(s_m), scale_wt[n])
//
// The decode GEMV is bound by streaming the packed weights from HBM (2 bits per
// weight, read once), so the design keeps every other cost off that stream.
//
// gemv_stream_kernel (activations fit in LDS: M * K <= 32768):
//  * Activations.  Every 256-thread workgroup quantises x itself (at most 15
//    rows; they stay in L2) into LDS as int8, each 16-element group stored as
//    the 4x4 byte transpose the unpack needs, in 64-element segments padded to
//    80 bytes so that the eight sub-lanes of a step hit distinct LDS banks.
//    Each thread first issues its loads of x, then the weight ring's first D
//    loads, and only then waits for x to compute the absmax and quantise, so
//    the weights are in flight during the prologue.  Where every wave has a
//    single short unit (the smaller decode projections), the ring goes out
//    after the absmax barrier instead, so that no workgroup's weight loads
//    hold up another's activations.
//  * Weights.  Work is split into units of 8 output rows; a workgroup owns up
//    to 32 consecutive units and its 4 waves take them round-robin.  Eight
//    consecutive lanes share a row and read 8 x 16 B = 128 contiguous bytes of
//    it per step (512 weights), so one wave instruction fetches 8 whole
//    128-byte lines.  Each wave keeps a ring of D loads in flight, every one of
//    them issued unconditionally (loads past the wave's work read a small,
//    always-cached pad), so the compiler's waits stay exact.
//  * Unpack without a lookup.  For a 32-bit word p of codes, p & 0x03030303,
//    p & 0x0C0C0C0C, p & 0x30303030 and (p >> 6) & 0x03030303 hold, in byte r,
//    the code of element 4r+e times 1, 4, 16 and 1 (e = 0..3).  Each is fed to
//    v_dot4_i32_i8 against the activations pre-permuted into the same byte
//    order, with separate accumulators for the x4 and x16 lanes; the exact
//    total sum(code * q) then loses 2 * sum_k q[m][k] to give sum((code-2) * q).
//    That is 5 logic ops + 4 dot4 per 16 weights.
//  * Reduction.  A row's eight partial sums are combined with three DPP adds
//    (quad_perm xor 1, quad_perm xor 2, row_half_mirror); the epilogue is fused.
//
// With RMS (the fused RMSNorm prologue of "kyegomez/BitNet issue #77"'s
// activation_norm_quant), every workgroup first normalises its activation rows:
// the exact squares are summed in double (per thread, then per wave with DPP,
// then the four waves in a fixed order through LDS), and each thread turns its
// bf16 words into the normalised bf16 values before the absmax and quantisation
// above.  The weight loads are already in flight meanwhile.
//
// With one activation row and few units of long rows (fewer than 4096 units x
// parts, at least 4 steps a part), groups of 2 or 4 waves share each unit, each
// wave taking a contiguous range of its steps; the exact int32 partial sums
// meet in LDS before the correction and the epilogue.
//
// For bitnet_linear_ex the same kernel takes f32 activations (XF32: the f32
// rows quantised as they are, with the f32 absmax) and a bias on the bf16
// outputs (BIAS: each workgroup stages its rows' bias values in LDS beside the
// weight scales); both are template variants, so a plain call runs the
// unchanged kernel.
//
// gemv_chunked_kernel (longer activations): each wave owns 8*RB rows and K is
// processed in LDS-sized chunks, with the same unpack and reduction.
//
// Shapes the fast kernels take: K % 64 == 0 and 16-byte aligned x and w (every
// BitNet/LLaMA projection).  Anything else goes to gemv_fused_plain, a direct
// one-wave-per-row kernel with the same arithmetic.
#include "bitnet_device.h"
#include "launch.h"

namespace bitnet {

namespace {

constexpr int GV_STEP = 512;            // weights per row per wave step (8 lanes x 64)
constexpr int GV_MAX_KS = 4;            // waves that can share one unit's K range
constexpr int GV_SPLIT_UNITS = 4096;    // split K while units x parts stays below this
constexpr int GV_LDS_BUDGET = 32768;    // bytes of quantised activations held per chunk
constexpr int GV_MFMA_MIN_M = 5;        // rows from which the fused product runs on the matrix units

__device__ __forceinline__ int lds_word_offset(int word) {
    // word = 16-element group within a chunk; seg = 64-element segment
    const int seg = word >> 2;
    const int j = word & 3;
    return (seg << 6) + ((j ^ ((seg >> 1) & 3)) << 4);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int j) {
    return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// ---------------------------------------------------------------- prologue helpers

// Row scales of the MT activation rows (rows >= M count as all-zero), computed
// by the whole workgroup: integer absmax over the bf16 magnitude bits, then
// quant_scale.  Block 0 also writes the bf16 scales when sa_out is given.
template <int MT, int WAVES>
__device__ __forceinline__ void block_row_scales(const uint16_t* __restrict__ x, int M, int K, uint32_t (*red_u)[MT],
                                                 float* s_scale, float* s_recip, uint16_t* __restrict__ sa_out,
                                                 QuantScale (&qsc)[MT]) {
    constexpr int NT = WAVES * 64;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    uint32_t am[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) am[m] = 0u;
    const int n8 = K >> 3;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (m < M) {
            const uint4* xv = reinterpret_cast<const uint4*>(x + (int64_t)m * K);
            for (int i = tid; i < n8; i += NT) {
                const uint4 v = xv[i];
                am[m] = max(am[m], max(max(absmax_bf16x2(v.x), absmax_bf16x2(v.y)),
                                       max(absmax_bf16x2(v.z), absmax_bf16x2(v.w))));
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const uint32_t a = wave_max_u32(am[m]);
        if (lane == 0) red_u[wave][m] = a;
    }
    __syncthreads();
    if (tid < MT) {
        uint32_t a = 0u;
#pragma unroll
        for (int wv = 0; wv < WAVES; ++wv) a = max(a, red_u[wv][tid]);
        const QuantScale qs = quant_scale(a);
        s_scale[tid] = qs.s;
        s_recip[tid] = qs.r;
        if (sa_out != nullptr && blockIdx.x == 0 && tid < M) sa_out[tid] = f32_to_bf16(qs.s);
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        qsc[m].s = s_scale[m];
        qsc[m].r = s_recip[m];
    }
}

// Quantise x[m][k0 .. k0 + len) of every row into LDS (row stride ldsz bytes),
// 16 elements per thread-iteration, zero-filling words [len/16, words); adds
// this thread's share of sum_k q[m][k] into sq.  len % 64 == 0.
template <int MT, int WAVES>
__device__ __forceinline__ void block_quantize_to_lds(uint8_t* lds_x, int ldsz, const uint16_t* __restrict__ x, int M,
                                                      int K, int k0, int len, int words, const QuantScale (&qsc)[MT],
                                                      int (&sq)[MT]) {
    constexpr int NT = WAVES * 64;
    const int tid = threadIdx.x;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        for (int wd = tid; wd < words; wd += NT) {
            uint4 t = make_uint4(0u, 0u, 0u, 0u);
            if (m < M && wd * 16 < len) {
                const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)m * K + k0 + wd * 16);
                const uint4 lo = src[0];
                const uint4 hi = src[1];
                const uint2 qlo = quantize_bf16x8(lo, qsc[m]);
                const uint2 qhi = quantize_bf16x8(hi, qsc[m]);
                const uint32_t n0 = qlo.x, n1 = qlo.y, n2 = qhi.x, n3 = qhi.y;
                int s = __builtin_amdgcn_sdot4((int)n0, 0x01010101, 0, false);
                s = __builtin_amdgcn_sdot4((int)n1, 0x01010101, s, false);
                s = __builtin_amdgcn_sdot4((int)n2, 0x01010101, s, false);
                s = __builtin_amdgcn_sdot4((int)n3, 0x01010101, s, false);
                sq[m] += s;
                t = transpose4x4(n0, n1, n2, n3);
            }
            *reinterpret_cast<uint4*>(lds_x + m * ldsz + lds_word_offset(wd)) = t;
        }
    }
}

// Block-wide sum of each row's partial sum_k q; result in s_sumq.
template <int MT, int WAVES>
__device__ __forceinline__ void block_sum_q(const int (&sq)[MT], int (*red_i)[MT], int* s_sumq) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int v = wave_sum_i32(sq[m]);
        if (lane == 0) red_i[wave][m] = v;
    }
    __syncthreads();
    if (tid < MT) {
        int s = 0;
#pragma unroll
        for (int wv = 0; wv < WAVES; ++wv) s += red_i[wv][tid];
        s_sumq[tid] = s;
    }
    __syncthreads();
}

// Dot products of one 16-byte piece of packed weights (64 codes, 4 words)
// with the matching 64 quantised activations of every row, read from LDS at
// byte offset `base` of each row (the slot of word j is base + ((j ^ swz) << 4)).
template <int MT>
__device__ __forceinline__ void dot_piece(const uint4& wv, const uint8_t* lds_x, int ldsz, int base, int swz,
                                          int (&a0)[MT], int (&a1)[MT], int (&a2)[MT]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t p = word_of(wv, j);
        const uint32_t c0 = p & 0x03030303u;
        const uint32_t c1 = p & 0x0C0C0C0Cu;
        const uint32_t c2 = p & 0x30303030u;
        const uint32_t c3 = (p >> 6) & 0x03030303u;
        const int off = base + ((j ^ swz) << 4);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4 xq = *reinterpret_cast<const uint4*>(lds_x + m * ldsz + off);
            a0[m] = __builtin_amdgcn_sdot4((int)c0, (int)xq.x, a0[m], false);
            a1[m] = __builtin_amdgcn_sdot4((int)c1, (int)xq.y, a1[m], false);
            a2[m] = __builtin_amdgcn_sdot4((int)c2, (int)xq.z, a2[m], false);
            a0[m] = __builtin_amdgcn_sdot4((int)c3, (int)xq.w, a0[m], false);
        }
    }
}

// ---------------------------------------------------------------- streaming kernel
//
// Workgroup b owns the contiguous 8-row units [b*UPB, (b+1)*UPB); its four
// waves take every fourth unit.  A wave's work is a flat sequence of items
// (unit, 512-weight step); a ring of D 16-byte weight loads runs D items ahead
// of the items being multiplied, across unit boundaries.
//
//  * Every ring load is unconditional, so the in-order load counter lets the
//    compiler wait for exactly the oldest load and keep D-1 in flight.  Loads
//    past the wave's work re-read its last unit and are never used.
//  * A load address is a wave-uniform base (unit row pointer + 128 B per step,
//    scalar registers) plus a per-lane offset (row within the unit, 16-byte
//    piece) that only changes at unit boundaries, so the steady loop spends no
//    vector instructions on addressing.  Rows past N re-read row N-1 and pieces
//    past the row end (K % 512 != 0) re-read the row's last 16 bytes; their x
//    is zero or their result is dropped.
//  * Quantised x sits in LDS in 64-byte segments padded to 80 bytes: the eight
//    lanes of a row then hit eight disjoint 4-bank groups, and a lane's four
//    16-byte reads are one base address with immediate offsets.
//
// Prologue.  All global reads it needs (this thread's XW 16-element words of
// x, and at most one weight scale) are issued before the ring, so waiting for
// them never waits for weights.  x is read once and kept in registers: the
// block absmax (one barrier), then every thread derives the scales itself,
// quantises its words into LDS and publishes its share of sum_k q (second
// barrier).  The weight scales of the workgroup's rows sit in LDS, so the
// per-unit epilogue issues no vector loads.  Needs MT * Kpad <= GV_LDS_BUDGET
// and UPB * 8 <= 256.
constexpr int GV_SEG = 80;  // LDS bytes per 64-element segment of quantised x

// Target of the streaming kernel's loads past a wave's last unit: covers the
// largest step offset (GV_LDS_BUDGET / GV_STEP steps of GV_STEP / 4 bytes) plus
// one 16-byte piece per lane.
constexpr int GV_PAD_BYTES = (GV_LDS_BUDGET / GV_STEP) * (GV_STEP / 4) + 64 * 16;
__device__ __align__(256) uint8_t gv_pad[GV_PAD_BYTES];

template <int MT>
__device__ __forceinline__ void dot_piece_padded(const uint4& wv, const uint8_t* lds_row0, int row_stride,
                                                 int (&a0)[MT], int (&a1)[MT], int (&a2)[MT]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t p = word_of(wv, j);
        const uint32_t c0 = p & 0x03030303u;
        const uint32_t c1 = p & 0x0C0C0C0Cu;
        const uint32_t c2 = p & 0x30303030u;
        const uint32_t c3 = (p >> 6) & 0x03030303u;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4 xq = *reinterpret_cast<const uint4*>(lds_row0 + m * row_stride + j * 16);
            a0[m] = __builtin_amdgcn_sdot4((int)c0, (int)xq.x, a0[m], false);
            a1[m] = __builtin_amdgcn_sdot4((int)c1, (int)xq.y, a1[m], false);
            a2[m] = __builtin_amdgcn_sdot4((int)c2, (int)xq.z, a2[m], false);
            a0[m] = __builtin_amdgcn_sdot4((int)c3, (int)xq.w, a0[m], false);
        }
    }
}

// XF32: x holds f32 activations (quantised as they are, with the f32 absmax),
// else bf16.  BIAS: bias [N] is added to the bf16 outputs.
template <int MT, int D, int XW, bool OUT_I32, bool RMS, int KS, bool XF32, bool BIAS, bool LATE>
__global__ __launch_bounds__(256) void gemv_stream_kernel(uint16_t* __restrict__ out, int32_t* __restrict__ acc_out,
                                                          uint16_t* __restrict__ sa_out,
                                                          const void* __restrict__ x,
                                                          const uint8_t* __restrict__ w,
                                                          const uint16_t* __restrict__ sw, int M, int N, int K,
                                                          int steps, int units, int upb,
                                                          const uint16_t* __restrict__ gain, float eps,
                                                          const uint16_t* __restrict__ bias) {
    static_assert(!(RMS && XF32), "the RMSNorm prologue takes bf16 activations");
    static_assert(!(BIAS && OUT_I32), "the bias applies to the bf16 outputs");
    static_assert(!(LATE && RMS), "the weight ring goes out after the absmax barrier of the plain prologue");
    constexpr int WAVES = 4;
    constexpr int NT = WAVES * 64;
    extern __shared__ __align__(16) uint8_t lds_x[];  // [MT][steps * 8 segments of GV_SEG bytes]
    __shared__ uint32_t red_u[WAVES][MT];
    __shared__ int red_i[WAVES][MT];
    __shared__ uint16_t sw_lds[NT];
    __shared__ uint16_t bias_lds[BIAS ? NT : 1];  // the workgroup's bias values

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps unit bookkeeping scalar
    const int g = lane >> 3;
    const int sl = lane & 7;
    const int KB = K >> 2;
    const int row_stride = steps * 8 * GV_SEG;
    const int wpr = steps * (GV_STEP / 16);  // 16-element words per activation row in LDS

    // With KS > 1 (one activation row), groups of KS waves share each unit,
    // wave kp of a group taking the contiguous steps [s_begin, s_end).
    constexpr int wg_n = WAVES / KS;  // wave groups
    const int wg = wave / KS;
    const int kp = wave - wg * KS;
    const int s_begin = KS == 1 ? 0 : kp * steps / KS;
    const int s_end = KS == 1 ? steps : (kp + 1) * steps / KS;  // the host guarantees steps >= KS
    const int ub0 = blockIdx.x * upb;
    const int ub1 = min(ub0 + upb, units);
    const int my_units = (ub0 + wg < ub1) ? (ub1 - 1 - ub0 - wg) / wg_n + 1 : 0;
    const int items = my_units * (s_end - s_begin);

    // ---- prologue reads, before any weight load: 16 elements a word, as two
    //      (bf16) or four (f32) 16-byte pieces
    constexpr int XV = XF32 ? 4 : 2;
    constexpr int XES = XF32 ? 4 : 2;  // bytes per activation element
    uint4 xr[XW][XV];
    int xm[XW], xw[XW];
#pragma unroll
    for (int i = 0; i < XW; ++i) {
        const int idx = tid + NT * i;
        xm[i] = idx / wpr;
        xw[i] = idx - xm[i] * wpr;
        if (xm[i] < M && xm[i] < MT && xw[i] * 16 < K) {
            const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(x) +
                                                              ((int64_t)xm[i] * K + xw[i] * 16) * XES);
#pragma unroll
            for (int v = 0; v < XV; ++v) xr[i][v] = src[v];
        } else {
#pragma unroll
            for (int v = 0; v < XV; ++v) xr[i][v] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    const int row0 = ub0 * 8;
    const int nrows = min(ub1 * 8, N) - row0;
    const uint16_t sw_mine = (tid < nrows && sw != nullptr) ? sw[row0 + tid] : (uint16_t)0;
    const uint16_t bias_mine = (BIAS && tid < nrows) ? bias[row0 + tid] : (uint16_t)0;

    // ---- the weight ring
    const int last_step = steps - 1;
    const bool ktail = (K % GV_STEP) != 0;  // wave-uniform
    // this lane's 16-byte piece in a step, clamped into the row for the last step
    const uint32_t piece = (uint32_t)(sl * 16);
    const uint32_t piece_last = (uint32_t)min(sl * 16, KB - last_step * (GV_STEP / 4) - 16);
    int lj = 0, lt = s_begin;   // load cursor: unit index (of this wave group) and step
    const uint8_t* unit_ptr;    // row 0 of the unit being loaded (wave-uniform)
    uint32_t voff, voff_last;   // this lane's byte offset from unit_ptr (normal / last step)
    auto set_unit = [&]() {
        // Past this wave's work the ring still issues (never consumed) loads:
        // they read a small pad that stays cached, instead of weight lines the
        // streaming loads have already evicted.  Selects, not branches, so the
        // ring's loads stay in straight-line code.
        const bool live = lj < my_units;  // wave-uniform
        const int u = min(ub0 + wg + wg_n * min(lj, max(my_units - 1, 0)), units - 1);
        const uint32_t lane_row = (uint32_t)((min(u * 8 + g, N - 1) - u * 8) * KB);
        unit_ptr = live ? w + (int64_t)u * 8 * KB : gv_pad;
        voff = live ? lane_row + piece : (uint32_t)(lane * 16);
        voff_last = live ? lane_row + piece_last : (uint32_t)(lane * 16);
    };
    set_unit();
    auto issue = [&](uint4& dst) {
        const uint8_t* b = unit_ptr + lt * (GV_STEP / 4);
        dst = load_stream16(b + ((ktail && lt == last_step) ? voff_last : voff));
        if (++lt == s_end) {
            lt = s_begin;
            ++lj;
            set_unit();
        }
    };
    // The ring goes out now, behind the activation loads, or with LATE once
    // the workgroup holds its activations (after the absmax barrier).
    uint4 buf[D];
    auto issue_ring = [&]() {
#pragma unroll
        for (int i = 0; i < D; ++i) issue(buf[i]);
    };
    if constexpr (!LATE) issue_ring();

    // ---- absmax of every activation row, per wave (of x itself)
    uint32_t am[MT];
    auto wave_absmax = [&]() {
#pragma unroll
        for (int m = 0; m < MT; ++m) am[m] = 0u;
#pragma unroll
        for (int i = 0; i < XW; ++i) {
            uint32_t a = 0u;
#pragma unroll
            for (int h = 0; h < XV; ++h) {
                if constexpr (XF32)
                    a = max(a, absmax_f32x4(xr[i][h]));
                else
                    a = max(a, max(max(absmax_bf16x2(xr[i][h].x), absmax_bf16x2(xr[i][h].y)),
                                   max(absmax_bf16x2(xr[i][h].z), absmax_bf16x2(xr[i][h].w))));
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) am[m] = (xm[i] == m) ? max(am[m], a) : am[m];
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint32_t a = wave_max_u32(am[m]);
            if (lane == 0) red_u[wave][m] = a;
        }
    };

    // ---- RMSNorm of the activation rows, in registers.  Without a gain the
    // normalised absmax is bf16(fp32(max|x| * r)) (both roundings are
    // monotonic and r > 0), so the absmax of x is reduced in the same round as
    // the sum of squares; with a gain the normalised values are scanned again.
    float rr[MT];
    if constexpr (RMS) {
        __shared__ double red_d[WAVES][MT];
        double ss[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) ss[m] = 0.0;
        uint4 gr[XW][2];
#pragma unroll
        for (int i = 0; i < XW; ++i) {
            const double t = sum_sq_bf16x8(xr[i][0]) + sum_sq_bf16x8(xr[i][1]);
#pragma unroll
            for (int m = 0; m < MT; ++m) ss[m] += (xm[i] == m) ? t : 0.0;
            const bool live = gain != nullptr && xm[i] < M && xm[i] < MT && xw[i] * 16 < K;
            if (live) {
                const uint4* src = reinterpret_cast<const uint4*>(gain + xw[i] * 16);
                gr[i][0] = src[0];
                gr[i][1] = src[1];
            } else {
                gr[i][0] = gr[i][1] = make_uint4(BF16X2_ONE, BF16X2_ONE, BF16X2_ONE, BF16X2_ONE);
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const double v = wave_sum_f64(ss[m]);
            if (lane == 0) red_d[wave][m] = v;
        }
        if (gain == nullptr) {  // wave-uniform
            wave_absmax();
            sw_lds[tid] = sw_mine;
            if constexpr (BIAS) bias_lds[tid] = bias_mine;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MT; ++m) rr[m] = rms_inv(((red_d[0][m] + red_d[1][m]) + red_d[2][m]) + red_d[3][m], K, eps);
#pragma unroll
        for (int i = 0; i < XW; ++i) {
            float r = rr[0];
#pragma unroll
            for (int m = 1; m < MT; ++m) r = (xm[i] == m) ? rr[m] : r;
            if (gain == nullptr) {  // wave-uniform; the same bits as a gain of 1
                xr[i][0] = rms_scale_bf16x8(xr[i][0], r);  // zero words stay zero
                xr[i][1] = rms_scale_bf16x8(xr[i][1], r);
            } else {
                xr[i][0] = rms_apply_bf16x8(xr[i][0], gr[i][0], r);
                xr[i][1] = rms_apply_bf16x8(xr[i][1], gr[i][1], r);
            }
        }
    }
    if (!RMS || gain != nullptr) {
        wave_absmax();
        sw_lds[tid] = sw_mine;
        if constexpr (BIAS) bias_lds[tid] = bias_mine;
        __syncthreads();
    }
    if constexpr (LATE) {
        __builtin_amdgcn_sched_barrier(0);  // keep the ring's loads after the barrier
        issue_ring();
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- scales (every thread), quantise own words into LDS, sum_k q
    QuantScale qsc[MT];
    float sa_f[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        uint32_t a = red_u[0][m];
#pragma unroll
        for (int wv = 1; wv < WAVES; ++wv) a = max(a, red_u[wv][m]);
        if (RMS && gain == nullptr) a = (uint32_t)f32_to_bf16(bf16_to_f32(a) * rr[m]) & 0x7FFFu;
        qsc[m] = XF32 ? quant_scale_f32(__builtin_bit_cast(float, a)) : quant_scale(a);
        sa_f[m] = bf16_to_f32(f32_to_bf16(qsc[m].s));
    }
    if (sa_out != nullptr && blockIdx.x == 0 && tid < M && tid < MT) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m == tid) sa_out[m] = f32_to_bf16(qsc[m].s);
    }
    int sq[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) sq[m] = 0;
#pragma unroll
    for (int i = 0; i < XW; ++i) {
        if (xm[i] < MT) {
            QuantScale qs = qsc[0];
#pragma unroll
            for (int m = 1; m < MT; ++m)
                if (xm[i] == m) qs = qsc[m];
            uint32_t n0, n1, n2, n3;
            if constexpr (XF32) {
                n0 = quantize_f32x4(xr[i][0], qs);
                n1 = quantize_f32x4(xr[i][1], qs);
                n2 = quantize_f32x4(xr[i][2], qs);
                n3 = quantize_f32x4(xr[i][3], qs);
            } else {
                const uint2 qlo = quantize_bf16x8(xr[i][0], qs);
                const uint2 qhi = quantize_bf16x8(xr[i][1], qs);
                n0 = qlo.x, n1 = qlo.y, n2 = qhi.x, n3 = qhi.y;
            }
            int t = __builtin_amdgcn_sdot4((int)n0, 0x01010101, 0, false);
            t = __builtin_amdgcn_sdot4((int)n1, 0x01010101, t, false);
            t = __builtin_amdgcn_sdot4((int)n2, 0x01010101, t, false);
            t = __builtin_amdgcn_sdot4((int)n3, 0x01010101, t, false);
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (xm[i] == m) sq[m] += t;
            const int off = xm[i] * row_stride + (xw[i] >> 2) * GV_SEG + (xw[i] & 3) * 16;
            *reinterpret_cast<uint4*>(lds_x + off) = transpose4x4(n0, n1, n2, n3);
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int v = wave_sum_i32(sq[m]);
        if (lane == 0) red_i[wave][m] = v;
    }
    __syncthreads();  // publishes the quantised x and the partial sums
    int sumq2[MT];    // 2 * sum_k q[m][k]
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        int v = red_i[0][m];
#pragma unroll
        for (int wv = 1; wv < WAVES; ++wv) v += red_i[wv][m];
        sumq2[m] = 2 * v;
    }

    // ---- stream
    int a0[MT], a1[MT], a2[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) a0[m] = a1[m] = a2[m] = 0;

    const uint8_t* lds_lane = lds_x + sl * GV_SEG;
    // partial sums of the K parts (exact int32), combined after the stream
    __shared__ int part[KS][KS > 1 ? NT * MT : 1];
    int cj = 0, ct = s_begin;  // consume cursor
    auto consume = [&](const uint4& piece) {
        dot_piece_padded<MT>(piece, lds_lane + ct * (8 * GV_SEG), row_stride, a0, a1, a2);
        if (++ct == s_end) {  // unit complete: reduce its 8 lanes per row and write
            const int ul = wg + wg_n * cj;  // unit index within the workgroup
            const int n = (ub0 + ul) * 8 + g;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                int tot = a0[m] + (a1[m] >> 2) + (a2[m] >> 4);
                tot = group8_sum(tot);
                a0[m] = a1[m] = a2[m] = 0;
                if (KS > 1) {
                    if ((m & 7) == sl) part[kp][(ul * 8 + g) * MT + m] = tot;
                } else if ((m & 7) == sl && n < N && m < M) {
                    tot -= sumq2[m];
                    if (OUT_I32) {
                        acc_out[(int64_t)m * N + n] = tot;
                    } else {
                        uint16_t o = epilogue_bf16(tot, sa_f[m], bf16_to_f32(sw_lds[ul * 8 + g]));
                        if constexpr (BIAS) o = add_bias_bf16(o, bias_lds[ul * 8 + g]);
                        out[(int64_t)m * N + n] = o;
                    }
                }
            }
            ct = s_begin;
            ++cj;
        }
    };

    int base = 0;
    for (; base + D <= items; base += D) {  // steady state: every item issues the load D items ahead
#pragma unroll
        for (int i = 0; i < D; ++i) {
            consume(buf[i]);
            issue(buf[i]);
        }
    }
    const int rem = items - base;  // the last < D items are already in the ring
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (i < rem) consume(buf[i]);

    if constexpr (KS > 1) {  // add the K parts, then the correction and the epilogue
        __syncthreads();
        for (int idx = tid; idx < nrows * MT; idx += NT) {
            const int rr = idx / MT;
            const int m = idx - rr * MT;
            int tot = part[0][idx];
#pragma unroll
            for (int p = 1; p < KS; ++p) tot += part[p][idx];
            tot -= sumq2[m];
            const int n = row0 + rr;
            if (m < M) {
                if (OUT_I32) {
                    acc_out[(int64_t)m * N + n] = tot;
                } else {
                    uint16_t o = epilogue_bf16(tot, sa_f[m], bf16_to_f32(sw_lds[rr]));
                    if constexpr (BIAS) o = add_bias_bf16(o, bias_lds[rr]);
                    out[(int64_t)m * N + n] = o;
                }
            }
        }
    }
}

// ---------------------------------------------------------------- chunked kernel
//
// For activations too large for LDS at once (MT * Kpad > GV_LDS_BUDGET): each
// wave owns 8*RB rows and the K dimension is processed in LDS-sized chunks.
template <int MT, int RB, int WAVES, bool OUT_I32>
__global__ __launch_bounds__(WAVES * 64) void gemv_chunked_kernel(uint16_t* __restrict__ out,
                                                                int32_t* __restrict__ acc_out,
                                                                uint16_t* __restrict__ sa_out,
                                                                const uint16_t* __restrict__ x,
                                                                const uint8_t* __restrict__ w,
                                                                const uint16_t* __restrict__ sw, int M, int N, int K,
                                                                int KC) {
    extern __shared__ __align__(16) uint8_t lds_x[];  // [MT][KC] quantised, transposed, swizzled
    __shared__ uint32_t red_u[WAVES][MT];
    __shared__ int red_i[WAVES][MT];
    __shared__ float s_scale[MT];
    __shared__ float s_recip[MT];
    __shared__ int s_sumq[MT];

    constexpr int NT = WAVES * 64;
    constexpr int ROWS = WAVES * 8 * RB;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 3;   // row of the 8-row group
    const int sl = lane & 7;   // 64-weight piece within a 512-weight step
    const int n_first = blockIdx.x * ROWS + wave * 8 * RB + g;
    const int64_t KB = K >> 2;

    const uint8_t* wrow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int n = min(n_first + rb * 8, N - 1);  // rows past N load a valid row; their results are dropped
        wrow[rb] = w + (int64_t)n * KB;
    }

    const int nchunks = (K + KC - 1) / KC;
    auto steps_in_chunk = [&](int c) {
        const int len = min(KC, K - c * KC);
        return (len + GV_STEP - 1) / GV_STEP;
    };
    auto load_step = [&](int c, int t, uint4 (&dst)[RB]) {
        const int kp = c * KC + t * GV_STEP + sl * 64;  // first weight of this lane's piece
        if (kp < K) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                dst[rb] = load_stream16(wrow[rb] + (kp >> 2));
        } else {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) dst[rb] = make_uint4(0u, 0u, 0u, 0u);
        }
    };

    // First weight loads go out before the prologue.
    uint4 wcur[RB];
    load_step(0, 0, wcur);

    // ---- prologue: row absmax of every activation row (all threads)
    {
        uint32_t am[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) am[m] = 0u;
        const int n8 = K >> 3;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < M) {
                const uint4* xv = reinterpret_cast<const uint4*>(x + (int64_t)m * K);
                for (int i = tid; i < n8; i += NT) {
                    const uint4 v = xv[i];
                    am[m] = max(am[m], max(max(absmax_bf16x2(v.x), absmax_bf16x2(v.y)),
                                           max(absmax_bf16x2(v.z), absmax_bf16x2(v.w))));
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint32_t a = wave_max_u32(am[m]);
            if (lane == 0) red_u[wave][m] = a;
        }
        __syncthreads();
        if (tid < MT) {
            uint32_t a = 0u;
#pragma unroll
            for (int wv = 0; wv < WAVES; ++wv) a = max(a, red_u[wv][tid]);
            const QuantScale qs = quant_scale(a);
            s_scale[tid] = qs.s;
            s_recip[tid] = qs.r;
            if (sa_out != nullptr && blockIdx.x == 0 && tid < M) sa_out[tid] = f32_to_bf16(qs.s);
        }
        __syncthreads();
    }
    QuantScale qsc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        qsc[m].s = s_scale[m];
        qsc[m].r = s_recip[m];
    }

    int a0[RB][MT], a1[RB][MT], a2[RB][MT];
    int sq[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        sq[m] = 0;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) a0[rb][m] = a1[rb][m] = a2[rb][m] = 0;
    }

    for (int c = 0; c < nchunks; ++c) {
        const int k0 = c * KC;
        const int steps = steps_in_chunk(c);
        const int len = min(KC, K - k0);
        const int words = steps * (GV_STEP / 16);

        // ---- quantise this chunk of every row into LDS
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            for (int wd = tid; wd < words; wd += NT) {
                uint4 t = make_uint4(0u, 0u, 0u, 0u);
                if (m < M && wd * 16 < len) {
                    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)m * K + k0 + wd * 16);
                    const uint4 lo = src[0];
                    const uint4 hi = src[1];
                    const uint2 qlo = quantize_bf16x8(lo, qsc[m]);
                    const uint2 qhi = quantize_bf16x8(hi, qsc[m]);
                    const uint32_t n0 = qlo.x, n1 = qlo.y, n2 = qhi.x, n3 = qhi.y;
                    int s = __builtin_amdgcn_sdot4((int)n0, 0x01010101, 0, false);
                    s = __builtin_amdgcn_sdot4((int)n1, 0x01010101, s, false);
                    s = __builtin_amdgcn_sdot4((int)n2, 0x01010101, s, false);
                    s = __builtin_amdgcn_sdot4((int)n3, 0x01010101, s, false);
                    sq[m] += s;
                    t = transpose4x4(n0, n1, n2, n3);
                }
                *reinterpret_cast<uint4*>(lds_x + m * KC + lds_word_offset(wd)) = t;
            }
        }
        __syncthreads();

        // ---- stream the packed weights of this chunk
        for (int t = 0; t < steps; ++t) {
            uint4 wnext[RB];
            const bool more = (t + 1 < steps) || (c + 1 < nchunks);
            if (more) {
                if (t + 1 < steps)
                    load_step(c, t + 1, wnext);
                else
                    load_step(c + 1, 0, wnext);
            }
            const int seg = t * 8 + sl;
            const int swz = (seg >> 1) & 3;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t cd0[RB], cd1[RB], cd2[RB], cd3[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const uint32_t p = word_of(wcur[rb], j);
                    cd0[rb] = p & 0x03030303u;
                    cd1[rb] = p & 0x0C0C0C0Cu;
                    cd2[rb] = p & 0x30303030u;
                    cd3[rb] = (p >> 6) & 0x03030303u;
                }
                const int off = (seg << 6) + ((j ^ swz) << 4);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const uint4 xq = *reinterpret_cast<const uint4*>(lds_x + m * KC + off);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        a0[rb][m] = __builtin_amdgcn_sdot4((int)cd0[rb], (int)xq.x, a0[rb][m], false);
                        a1[rb][m] = __builtin_amdgcn_sdot4((int)cd1[rb], (int)xq.y, a1[rb][m], false);
                        a2[rb][m] = __builtin_amdgcn_sdot4((int)cd2[rb], (int)xq.z, a2[rb][m], false);
                        a0[rb][m] = __builtin_amdgcn_sdot4((int)cd3[rb], (int)xq.w, a0[rb][m], false);
                    }
                }
            }
            if (more) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) wcur[rb] = wnext[rb];
            }
        }
        __syncthreads();  // LDS is rewritten by the next chunk
    }

    // ---- sum_k q[m][k] over the whole block
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int v = wave_sum_i32(sq[m]);
        if (lane == 0) red_i[wave][m] = v;
    }
    __syncthreads();
    if (tid < MT) {
        int s = 0;
#pragma unroll
        for (int wv = 0; wv < WAVES; ++wv) s += red_i[wv][tid];
        s_sumq[tid] = s;
    }
    __syncthreads();

    // ---- reduce the 8 lanes of each row, correct the code offset, write
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int n = n_first + rb * 8;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            int tot = a0[rb][m] + (a1[rb][m] >> 2) + (a2[rb][m] >> 4);
            tot = group8_sum(tot);
            tot -= 2 * s_sumq[m];
            const int idx = rb * MT + m;
            if ((idx & 7) == sl && n < N && m < M) {
                if (OUT_I32)
                    acc_out[(int64_t)m * N + n] = tot;
                else
                    out[(int64_t)m * N + n] = epilogue_bf16(tot, bf16_to_f32(f32_to_bf16(qsc[m].s)), bf16_to_f32(sw[n]));
            }
        }
    }
}

// Plain fused path: one wave per output row, any K % 4 == 0 and any alignment.
template <bool OUT_I32>
__global__ __launch_bounds__(64) void gemv_fused_plain(uint16_t* __restrict__ out, int32_t* __restrict__ acc_out,
                                                       uint16_t* __restrict__ sa_out, const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ w,
                                                       const uint16_t* __restrict__ sw, int M, int N, int K) {
    const int n = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t KB = K >> 2;
    for (int m = 0; m < M; ++m) {
        const uint16_t* xr = x + (int64_t)m * K;
        uint32_t am = 0u;
        for (int k = lane; k < K; k += 64) am = max(am, (uint32_t)xr[k] & 0x7FFFu);
        am = wave_max_u32(am);
        const QuantScale qs = quant_scale(am);
        if (sa_out != nullptr && n == 0 && lane == 0) sa_out[m] = f32_to_bf16(qs.s);
        int acc = 0;
        for (int k = lane; k < K; k += 64) {
            const int code = (w[(int64_t)n * KB + (k >> 2)] >> (2 * (k & 3))) & 3;
            acc += (code - 2) * quantize_one(bf16_to_f32(xr[k]), qs);
        }
        acc = wave_sum_i32(acc);
        if (lane == 0) {
            if (OUT_I32)
                acc_out[(int64_t)m * N + n] = acc;
            else
                out[(int64_t)m * N + n] = epilogue_bf16(acc, bf16_to_f32(f32_to_bf16(qs.s)), bf16_to_f32(sw[n]));
        }
    }
}

// Workgroups of the streaming kernel: enough to fill the GPU several times
// over, never more than there are 4-wave groups of units.
constexpr int GV_STREAM_MAX_BLOCKS = 512;

template <int MT, int D, bool OUT_I32, bool RMS, int KS, bool XF32, bool BIAS, bool LATE = false>
hipError_t launch_stream_xw(int xw, dim3 grid, size_t lds, hipStream_t s, uint16_t* out, int32_t* acc, uint16_t* sa_out,
                            const void* x, const uint8_t* w, const uint16_t* sw, int M, int N, int K, int steps,
                            int units, int upb, const uint16_t* gain, float eps, const uint16_t* bias) {
    if (xw <= 1)
        hipLaunchKernelGGL((gemv_stream_kernel<MT, D, 1, OUT_I32, RMS, KS, XF32, BIAS, LATE>), grid, dim3(256), lds, s, out, acc,
                           sa_out, x, w, sw, M, N, K, steps, units, upb, gain, eps, bias);
    else if (xw <= 2)
        hipLaunchKernelGGL((gemv_stream_kernel<MT, D, 2, OUT_I32, RMS, KS, XF32, BIAS, LATE>), grid, dim3(256), lds, s, out, acc,
                           sa_out, x, w, sw, M, N, K, steps, units, upb, gain, eps, bias);
    else if (xw <= 4)
        hipLaunchKernelGGL((gemv_stream_kernel<MT, D, 4, OUT_I32, RMS, KS, XF32, BIAS, LATE>), grid, dim3(256), lds, s, out, acc,
                           sa_out, x, w, sw, M, N, K, steps, units, upb, gain, eps, bias);
    else
        hipLaunchKernelGGL((gemv_stream_kernel<MT, D, 8, OUT_I32, RMS, KS, XF32, BIAS, LATE>), grid, dim3(256), lds, s, out, acc,
                           sa_out, x, w, sw, M, N, K, steps, units, upb, gain, eps, bias);
    return hipGetLastError();
}

template <int MT, bool OUT_I32, bool RMS = false, bool XF32 = false, bool BIAS = false>
hipError_t launch_stream(uint16_t* out, int32_t* acc, uint16_t* sa_out, const void* x, const uint8_t* w,
                         const uint16_t* sw, int M, int N, int K, hipStream_t s, const uint16_t* gain = nullptr,
                         float eps = 0.0f, const uint16_t* bias = nullptr) {
    const int steps = (K + GV_STEP - 1) / GV_STEP;
    const int units = (N + 7) / 8;
    // Split K inside the workgroup (one or two activation rows) when there are
    // too few units to give every CU several waves of whole rows.
    int ks = 1;
    if (MT == 1)
        while (ks < GV_MAX_KS && units * ks < GV_SPLIT_UNITS && steps >= 8 * ks) ks *= 2;  // >= 4 steps a part
    const int groups = 4 / ks;
    // At most 32 units (256 rows, one weight scale per thread) per workgroup;
    // otherwise as few workgroups as keep the GPU full.
    int blocks = (units + groups - 1) / groups;
    if (blocks > GV_STREAM_MAX_BLOCKS) blocks = GV_STREAM_MAX_BLOCKS;
    if (blocks < (units + 31) / 32) blocks = (units + 31) / 32;
    const int upb = (units + blocks - 1) / blocks;
    blocks = (units + upb - 1) / upb;
    const size_t lds = (size_t)MT * steps * 8 * GV_SEG;
    const int xw = (MT * steps * (GV_STEP / 16) + 255) / 256;  // x words per thread (<= 8 by the budget)
    // Ring depth: 16 loads per lane for long rows, 8 normally, 4 when the MT
    // accumulators already take most of the register file.  With one
    // activation row and a single unit per wave (the smaller decode
    // projections), 4: a deeper ring would only add loads past the wave's few
    // steps, which stall the issue of the prologue behind them (measured on the
    // BitNet-2B-4T gate_up projection: 5.17 -> 4.83 us).  Wherever a wave has
    // a single unit of at most 8 steps, the ring goes out only after the
    // absmax barrier, once the workgroup holds its activations: issued ahead
    // of them, the loads of all workgroups delayed the activations and the
    // prologue (BitNet-2B-4T projections at M = 2..4: 3-10% faster, e.g.
    // gate_up M = 2 6.5 -> 5.9 us; M = 1: between even and 10% faster by box;
    // the LM head, whose ring runs over many units, was 1% slower that way and
    // keeps the early issue).
    constexpr int D_SHORT = MT >= 8 ? 4 : 8;
    constexpr int D_LONG = MT == 1 ? 16 : D_SHORT;
    const dim3 grid(blocks);
    if constexpr (MT == 1) {
        if (ks == 1 && upb <= groups && steps <= 8)
            return launch_stream_xw<MT, 4, OUT_I32, RMS, 1, XF32, BIAS, !RMS>(xw, grid, lds, s, out, acc, sa_out, x, w, sw,
                                                                        M, N, K, steps, units, upb, gain, eps, bias);
        if (ks == 4) {
            if (steps / 4 >= 12)
                return launch_stream_xw<MT, D_LONG, OUT_I32, RMS, 4, XF32, BIAS>(xw, grid, lds, s, out, acc, sa_out, x, w, sw, M, N,
                                                                     K, steps, units, upb, gain, eps, bias);
            return launch_stream_xw<MT, D_SHORT, OUT_I32, RMS, 4, XF32, BIAS>(xw, grid, lds, s, out, acc, sa_out, x, w, sw, M, N, K,
                                                                  steps, units, upb, gain, eps, bias);
        }
        if (ks == 2) {
            if (steps / 2 >= 12)
                return launch_stream_xw<MT, D_LONG, OUT_I32, RMS, 2, XF32, BIAS>(xw, grid, lds, s, out, acc, sa_out, x, w, sw, M, N,
                                                                     K, steps, units, upb, gain, eps, bias);
            return launch_stream_xw<MT, D_SHORT, OUT_I32, RMS, 2, XF32, BIAS>(xw, grid, lds, s, out, acc, sa_out, x, w, sw, M, N, K,
                                                                  steps, units, upb, gain, eps, bias);
        }
    }
    if (steps >= 12)
        return launch_stream_xw<MT, D_LONG, OUT_I32, RMS, 1, XF32, BIAS>(xw, grid, lds, s, out, acc, sa_out, x, w, sw, M, N, K,
                                                             steps, units, upb, gain, eps, bias);
    // One activation row, several units per wave, short rows (the LM head): a
    // ring of 6.  Fewer loads in flight per CU let every workgroup's activation
    // loads through sooner, so the workgroups start streaming together and end
    // closer together (BitNet-2B-4T LM head, 128256 x 2560: 15.2 -> 14.4 us
    // against a ring of 8; 4 and 5 gave 14.4-14.9 us, 3 gave 16.2 us).
    if constexpr (MT == 1)
        return launch_stream_xw<MT, 6, OUT_I32, RMS, 1, XF32, BIAS>(xw, grid, lds, s, out, acc, sa_out, x, w, sw, M, N, K,
                                                                steps, units, upb, gain, eps, bias);
    if (upb <= groups && steps <= 8)
        return launch_stream_xw<MT, D_SHORT, OUT_I32, RMS, 1, XF32, BIAS, !RMS>(xw, grid, lds, s, out, acc, sa_out, x, w, sw, M, N, K,
                                                                steps, units, upb, gain, eps, bias);
    return launch_stream_xw<MT, D_SHORT, OUT_I32, RMS, 1, XF32, BIAS>(xw, grid, lds, s, out, acc, sa_out, x, w, sw, M, N, K,
                                                                steps, units, upb, gain, eps, bias);
}

template <int MT, bool OUT_I32>
hipError_t launch_chunked(uint16_t* out, int32_t* acc, uint16_t* sa_out, const uint16_t* x, const uint8_t* w,
                          const uint16_t* sw, int M, int N, int K, hipStream_t s) {
    constexpr int WAVES = 4;
    constexpr int RB = 1;
    constexpr int ROWS = WAVES * 8 * RB;
    const int kc_max = (GV_LDS_BUDGET / MT) / GV_STEP * GV_STEP;
    const int kpad = (K + GV_STEP - 1) / GV_STEP * GV_STEP;
    const int KC = kpad < kc_max ? kpad : kc_max;
    const size_t lds = (size_t)MT * KC;
    const unsigned blocks = (unsigned)((N + ROWS - 1) / ROWS);
    hipLaunchKernelGGL((gemv_chunked_kernel<MT, RB, WAVES, OUT_I32>), dim3(blocks), dim3(WAVES * 64), lds, s, out,
                       acc, sa_out, x, w, sw, M, N, K, KC);
    return hipGetLastError();
}

template <int MT, bool OUT_I32>
hipError_t dispatch_mt(uint16_t* out, int32_t* acc, uint16_t* sa_out, const uint16_t* x, const uint8_t* w,
                       const uint16_t* sw, int M, int N, int K, hipStream_t s) {
    const int64_t kpad = (K + GV_STEP - 1) / GV_STEP * GV_STEP;
    if (MT * kpad <= GV_LDS_BUDGET) return launch_stream<MT, OUT_I32>(out, acc, sa_out, x, w, sw, M, N, K, s);
    return launch_chunked<MT, OUT_I32>(out, acc, sa_out, x, w, sw, M, N, K, s);
}

template <bool OUT_I32>
hipError_t dispatch(uint16_t* out, int32_t* acc, uint16_t* sa_out, const uint16_t* x, const uint8_t* w,
                    const uint16_t* sw, int M, int N, int K, hipStream_t s) {
    // From five rows the dot4 stream is bound by LDS reads of the activations
    // (one per row and weight word): the matrix-unit kernel takes over.
    if (M >= GV_MFMA_MIN_M && gemv_mfma_fits(M, N, K, x, w))
        return launch_gemv_mfma(out, acc, sa_out, x, w, sw, M, N, K, s);
    const bool fast = (K % 64 == 0) && aligned16(x) && aligned16(w);
    if (!fast) {
        hipLaunchKernelGGL((gemv_fused_plain<OUT_I32>), dim3((unsigned)N), dim3(64), 0, s, out, acc, sa_out, x, w, sw,
                           M, N, K);
        return hipGetLastError();
    }
    if (M == 1) return dispatch_mt<1, OUT_I32>(out, acc, sa_out, x, w, sw, M, N, K, s);
    if (M == 2) return dispatch_mt<2, OUT_I32>(out, acc, sa_out, x, w, sw, M, N, K, s);
    if (M <= 4) return dispatch_mt<4, OUT_I32>(out, acc, sa_out, x, w, sw, M, N, K, s);
    if (M <= 8) return dispatch_mt<8, OUT_I32>(out, acc, sa_out, x, w, sw, M, N, K, s);
    return dispatch_mt<16, OUT_I32>(out, acc, sa_out, x, w, sw, M, N, K, s);
}

}  // namespace

hipError_t launch_gemv_fused(uint16_t* out, int32_t* acc, uint16_t* scale_act_out, const uint16_t* x,
                             const uint8_t* w, const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K,
                             hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (acc != nullptr) return dispatch<true>(nullptr, acc, scale_act_out, x, w, scale_wt, (int)M, (int)N, (int)K, s);
    return dispatch<false>(out, nullptr, scale_act_out, x, w, scale_wt, (int)M, (int)N, (int)K, s);
}

// The streaming kernel with f32 activations or a bias epilogue exists at 1, 2
// and 4 (padded) activation rows whose quantised values fit in LDS.
bool gemv_ex_fusable(int64_t M, int64_t K, const void* x, const void* w) {
    if (M < 1 || M > 4 || K % 64 != 0 || !aligned16(x) || !aligned16(w)) return false;
    const int64_t mt = M == 1 ? 1 : (M == 2 ? 2 : 4);
    const int64_t kpad = (K + GV_STEP - 1) / GV_STEP * GV_STEP;
    return mt * kpad <= GV_LDS_BUDGET;
}

template <bool XF32, bool BIAS>
hipError_t launch_ex_m(uint16_t* out, const void* x, const uint16_t* bias, const uint8_t* w, const uint16_t* scale_wt,
                       int64_t M, int64_t N, int64_t K, hipStream_t s) {
    const int m = (int)M, n = (int)N, k = (int)K;
    if (M == 1)
        return launch_stream<1, false, false, XF32, BIAS>(out, nullptr, nullptr, x, w, scale_wt, m, n, k, s, nullptr,
                                                           0.0f, bias);
    if (M == 2)
        return launch_stream<2, false, false, XF32, BIAS>(out, nullptr, nullptr, x, w, scale_wt, m, n, k, s, nullptr,
                                                           0.0f, bias);
    return launch_stream<4, false, false, XF32, BIAS>(out, nullptr, nullptr, x, w, scale_wt, m, n, k, s, nullptr, 0.0f,
                                                       bias);
}

hipError_t launch_gemv_fused_ex(uint16_t* out, const void* x, bool x_f32, const uint16_t* bias, const uint8_t* w,
                                const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (!gemv_ex_fusable(M, K, x, w)) return hipErrorInvalidValue;
    if (x_f32 && bias != nullptr) return launch_ex_m<true, true>(out, x, bias, w, scale_wt, M, N, K, s);
    if (x_f32) return launch_ex_m<true, false>(out, x, nullptr, w, scale_wt, M, N, K, s);
    if (bias != nullptr) return launch_ex_m<false, true>(out, x, bias, w, scale_wt, M, N, K, s);
    return launch_ex_m<false, false>(out, x, nullptr, w, scale_wt, M, N, K, s);
}

// The fused RMSNorm prologue exists for the streaming kernel at 1, 2 and 4
// (padded) activation rows; other shapes take RMSNorm-quantise + GEMM.
bool gemv_rms_fusable(int64_t M, int64_t K, const void* x, const void* w, const void* gain) {
    if (M < 1 || M > 4 || K % 64 != 0 || !aligned16(x) || !aligned16(w) || (gain != nullptr && !aligned16(gain)))
        return false;
    const int64_t mt = M == 1 ? 1 : (M == 2 ? 2 : 4);
    const int64_t kpad = (K + GV_STEP - 1) / GV_STEP * GV_STEP;
    return mt * kpad <= GV_LDS_BUDGET;
}

hipError_t launch_gemv_fused_rms(uint16_t* out, uint16_t* scale_act_out, const uint16_t* x, const uint16_t* gain,
                                 float eps, const uint8_t* w, const uint16_t* scale_wt, int64_t M, int64_t N,
                                 int64_t K, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (!gemv_rms_fusable(M, K, x, w, gain)) return hipErrorInvalidValue;
    if (M == 1)
        return launch_stream<1, false, true>(out, nullptr, scale_act_out, x, w, scale_wt, (int)M, (int)N, (int)K, s,
                                             gain, eps);
    if (M == 2)
        return launch_stream<2, false, true>(out, nullptr, scale_act_out, x, w, scale_wt, (int)M, (int)N, (int)K, s,
                                             gain, eps);
    return launch_stream<4, false, true>(out, nullptr, scale_act_out, x, w, scale_wt, (int)M, (int)N, (int)K, s, gain,
                                         eps);
}

}  // namespace bitnet
