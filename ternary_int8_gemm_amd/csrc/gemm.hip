// gemm.hip -- batched ternary x int8 GEMM on CDNA4 int8 MFMA (K-GEMM).
//
// Computes bitnet_gemm of "phanerozoic/bitnet-cpu v1,
// torch-ext/bitnet_cpu/__init__.py" for any M:
//   acc[m][n] = sum_k (code[n][k] - 2) * x_int8[m][k]     (exact int32)
//   out[m][n] = epilogue(acc, scale_act[m], scale_wt[n])   (or acc itself)
// The request post of "kernels-community/README discussion #1 (bitnet-tc kernel
// request)" runs this on the matrix units for batched shapes; here that is
// v_mfma_i32_16x16x64_i8 with int32 accumulators.
//
// Data flow of one 128x128 output tile (4 waves, 2 x 2, each 64 x 64 = 4 x 4
// MFMA tiles), per K-tile of KT elements:
//
//  * A (activations, int8, row-major [M][K]) is read with 16-byte loads,
//    4x4-byte transposed in registers and staged in LDS (double-buffered, rows
//    padded by 16 bytes so that the fragment reads of 16 consecutive rows fall
//    in distinct banks).  The same pass sums each row's bytes (v_dot4 with
//    0x01010101), giving sum_k x[m][k] for free.
//  * B (packed weights, [N][K/4]) never goes through LDS: each lane loads the
//    4*S bytes of one column that its MFMA fragments need and expands them in
//    registers, (p >> 2e) & 0x03030303 for e = 0..3, which are exactly the four
//    fragment dwords in the transposed byte order of A.  The fragments carry
//    the codes (1, 2, 3), not the weights.
//  * MFMA: for each of the S = KT/64 steps, one 16-byte A fragment per 16-row
//    tile from LDS, one 16-byte B fragment per 16-column tile from registers,
//    16 MFMAs per wave.  Lane l of a fragment holds row (or column) l % 16 and
//    the k-group l / 16; A and B use the same k order, which is all the
//    contraction needs.
//  * Epilogue: acc = sum(code * x) - 2 * sum_k x[m][k], then the fp32 scale
//    step and bf16 rounding, straight from the accumulator registers.
//
// Tiles are assigned XCD-aware: the hardware deals workgroups round-robin to
// the 8 XCDs, so the block index is remapped to give each XCD a contiguous run
// of tiles that share A row-panels in its own L2.
//
// The fast kernel needs K % 64 == 0 and 16-byte aligned x and w; anything
// else goes to gemm_plain (one wave per output row, same arithmetic).
#include "bitnet_device.h"
#include "launch.h"

namespace bitnet {

namespace {

constexpr int GM_BM = 256;      // block tile rows
constexpr int GM_BN = 128;      // block tile columns
constexpr int GM_KS = 128;      // K per pipeline stage (4 MFMA k-steps of 32)
constexpr int GM_KSTEPS = GM_KS / 32;
constexpr int GM_WAVES = 8;     // 4 along M x 2 along N, each a 64 x 64 wave tile
constexpr int GM_THREADS = GM_WAVES * 64;
constexpr int GM_FRAG = 1024;   // bytes of one 32 x 32 int8 MFMA operand fragment
constexpr int GM_A_STAGE = (GM_BM / 32) * GM_KSTEPS * GM_FRAG;  // 32 KB
constexpr int GM_B_STAGE = (GM_BN / 32) * GM_KSTEPS * GM_FRAG;  // 16 KB
// Depth of the global-load pipeline: the loads of stage k + GM_AHEAD are issued
// while stage k is multiplied (register-staged); LDS is double-buffered.
constexpr int GM_AHEAD = 3;
constexpr size_t GM_LDS_BYTES = 2 * (size_t)(GM_A_STAGE + GM_B_STAGE);

// Signed weights of one packed byte, in natural order: byte e of the result is
// code(e) - 2 for the code in bits 2e..2e+1 of b (b < 256).  The byte is
// spread with two shift-ors (b | b<<6 | b<<12 | b<<18 puts bits 2e..2e+1 of b
// at bits 8e..8e+1), masked to 2 bits per byte, and the codes are mapped by a
// byte permute through the table [0xFE, 0xFF, 0x00, 0x01] (code 0, never
// produced by packing, decodes to -2 like the rest of the library).
__device__ __forceinline__ uint32_t decode_byte(uint32_t b) {
    uint32_t s = b | (b << 6);
    s = s | (s << 12);
    s &= CODE_MASK;
    return __builtin_amdgcn_perm(0u, 0x0100FFFEu, s);
}

__device__ __forceinline__ v4u decode_word(uint32_t p) {
    v4u v;
    v.x = decode_byte(p & 0xFFu);
    v.y = decode_byte((p >> 8) & 0xFFu);
    v.z = decode_byte((p >> 16) & 0xFFu);
    v.w = decode_byte(p >> 24);
    return v;
}

__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int per = total / 8;
    const int rem = total % 8;
    const int xcd = bid % 8;
    const int idx = bid / 8;
    return xcd * per + min(xcd, rem) + idx;
}

// 16-byte slot of fragment lane fl in a fragment of k-step ks: an XOR with an
// even constant below 16, so that lane-contiguous fragment reads stay
// conflict-free and the coalesced staging writes (two rows x eight 16-byte
// chunks per 16 lanes, spread over eight (k-step, k-half) fragments) land in 16
// distinct slots mod 16.
__device__ __forceinline__ int frag_slot(int fl, int ks) { return fl ^ (2 * (fl >> 5) + 4 * ks); }

// Registers of one stage in flight: four 16-byte A pieces and two packed B words.
struct StageRegs {
    v4u a0, a1, a2, a3;
    uint32_t b0, b1;
};

template <bool OUT_I32>
__global__ __launch_bounds__(GM_THREADS) void gemm_mfma_kernel(uint16_t* __restrict__ out,
                                                               int32_t* __restrict__ acc_out,
                                                               const int8_t* __restrict__ x,
                                                               const uint8_t* __restrict__ w,
                                                               const uint16_t* __restrict__ sa,
                                                               const uint16_t* __restrict__ sw, int M, int N, int K,
                                                               int tiles_m, int tiles_n) {
    // LDS: [2 buffers][A: 8 row-tiles x 4 k-steps | B: 4 column-tiles x 4 k-steps]
    // of 1 KB fragments (32 rows or columns x 32 k); fragment lane l (row or
    // column l % 32, 16 bytes of k-half l / 32) sits in slot frag_slot(l, ks).
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int STAGE_BYTES = GM_A_STAGE + GM_B_STAGE;

    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int tm = tile / tiles_n;
    const int tn = tile - tm * tiles_n;
    const int m0 = tm * GM_BM;
    const int n0 = tn * GM_BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1;   // 64-row slab (row-tiles 2wm, 2wm+1)
    const int wn = wave & 1;    // 64-column slab (column tiles 2wn, 2wn+1)
    const int KB = K >> 2;
    const int nk = K / GM_KS;

    // A staging: a load instruction covers 8 rows x 128 contiguous bytes (8
    // lanes per row); wave w stages block rows 32w .. 32w+31 in four pieces.
    const int8_t* a_src;
    int a_off[4];  // LDS byte offsets within a stage
    {
        const int qa = lane & 7;
        const int ks = qa >> 1, kh = qa & 1;
        const int rb = wave * 32 + (lane >> 3);
        a_src = x + (int64_t)min(m0 + rb, M - 1) * K + qa * 16;  // rows past M repeat row M-1
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rb + 8 * i;
            a_off[i] = ((r >> 5) * GM_KSTEPS + ks) * GM_FRAG + frag_slot((r & 31) + 32 * kh, ks) * 16;
        }
    }
    const int64_t a_row8 = (int64_t)8 * K;  // the next piece is 8 rows down
    const bool a_clamp = m0 + GM_BM > M;     // rows past M: recompute each piece's row
    // B staging: thread t loads the two packed words 2h, 2h+1 (h = t % 4) of
    // block column t / 4 (32 weights) and writes them to their fragment slots.
    const uint8_t* b_src;
    int b_off0, b_off1;
    {
        const int h = tid & 3;
        const int cb = tid >> 2;
        b_src = w + (int64_t)min(n0 + cb, N - 1) * KB + h * 8;  // columns past N repeat column N-1
        const int q0 = 2 * h, q1 = 2 * h + 1;
        b_off0 = GM_A_STAGE + ((cb >> 5) * GM_KSTEPS + (q0 >> 1)) * GM_FRAG + frag_slot((cb & 31) + 32 * (q0 & 1), q0 >> 1) * 16;
        b_off1 = GM_A_STAGE + ((cb >> 5) * GM_KSTEPS + (q1 >> 1)) * GM_FRAG + frag_slot((cb & 31) + 32 * (q1 & 1), q1 >> 1) * 16;
    }
    int rd[GM_KSTEPS];  // this lane's fragment slot (bytes) per k-step
#pragma unroll
    for (int ks = 0; ks < GM_KSTEPS; ++ks) rd[ks] = frag_slot(lane, ks) * 16;

    // Loads of stage s (clamped to the last stage, so every step issues the
    // same loads and the waits the compiler derives are exact).
    auto a_ptr = [&](int i, int kb) -> const int8_t* {
        if (a_clamp) {
            const int r = min(m0 + wave * 32 + (lane >> 3) + 8 * i, M - 1);
            return x + (int64_t)r * K + (lane & 7) * 16 + kb;
        }
        return a_src + i * a_row8 + kb;
    };
    auto load_stage = [&](int s, StageRegs& r) {
        const int kb = min(s, nk - 1) * GM_KS;
        r.a0 = *reinterpret_cast<const v4u*>(a_ptr(0, kb));
        r.a1 = *reinterpret_cast<const v4u*>(a_ptr(1, kb));
        r.a2 = *reinterpret_cast<const v4u*>(a_ptr(2, kb));
        r.a3 = *reinterpret_cast<const v4u*>(a_ptr(3, kb));
        const uint2 b = *reinterpret_cast<const uint2*>(b_src + (kb >> 2));
        r.b0 = b.x;
        r.b1 = b.y;
    };
    auto store_stage = [&](int s, const StageRegs& r) {
        uint8_t* S = lds + (s & 1) * STAGE_BYTES;
        *reinterpret_cast<v4u*>(S + a_off[0]) = r.a0;
        *reinterpret_cast<v4u*>(S + a_off[1]) = r.a1;
        *reinterpret_cast<v4u*>(S + a_off[2]) = r.a2;
        *reinterpret_cast<v4u*>(S + a_off[3]) = r.a3;
        *reinterpret_cast<v4u*>(S + b_off0) = decode_word(r.b0);
        *reinterpret_cast<v4u*>(S + b_off1) = decode_word(r.b1);
    };

    v16i acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[mt][c] = v16i{};

    auto compute_stage = [&](int s) {
        const uint8_t* A = lds + (s & 1) * STAGE_BYTES + (wm * 2) * GM_KSTEPS * GM_FRAG;
        const uint8_t* B = lds + (s & 1) * STAGE_BYTES + GM_A_STAGE + (wn * 2) * GM_KSTEPS * GM_FRAG;
#pragma unroll
        for (int ks = 0; ks < GM_KSTEPS; ++ks) {
            v4i af[2], bf[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                af[t] = *reinterpret_cast<const v4i*>(A + (t * GM_KSTEPS + ks) * GM_FRAG + rd[ks]);
                bf[t] = *reinterpret_cast<const v4i*>(B + (t * GM_KSTEPS + ks) * GM_FRAG + rd[ks]);
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    acc[mt][c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[mt], bf[c], acc[mt][c], 0, 0, 0);
        }
    };

    // Stages k+1 .. k+3 sit in three register sets used in a fixed rotation, so
    // every register is named statically (no array indexing, no copies).
    static_assert(GM_AHEAD == 3, "the rotation below is written out for three sets");
    StageRegs r0, r1, r2;
    load_stage(0, r0);
    load_stage(1, r1);
    load_stage(2, r2);
    store_stage(0, r0);
    load_stage(3, r0);

    // Every step issues its loads and LDS stores unconditionally (stage indices
    // past the end are clamped and never multiplied), so the number of loads
    // between any two points is the same on every path and the compiler's
    // waits are exact.
#define BITNET_GEMM_STEP(K_, R_)                                       \
    __syncthreads(); /* stage K_ visible; the other buffer is free */ \
    store_stage((K_) + 1, R_);                                         \
    load_stage((K_) + 1 + GM_AHEAD, R_);                               \
    if ((K_) < nk) compute_stage(K_); /* uniform */
    for (int k = 0; k < nk; k += GM_AHEAD) {
        BITNET_GEMM_STEP(k, r1)
        BITNET_GEMM_STEP(k + 1, r2)
        BITNET_GEMM_STEP(k + 2, r0)
    }
#undef BITNET_GEMM_STEP

    // ---- epilogue straight from the accumulators: register r of lane l of a
    //      32 x 32 tile holds row 8(r/4) + 4(l/32) + r%4, column l%32
    float swf[2];
    int gcol[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        gcol[c] = n0 + (wn * 2 + c) * 32 + (lane & 31);
        swf[c] = (!OUT_I32 && gcol[c] < N) ? bf16_to_f32(sw[gcol[c]]) : 0.0f;
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int gm = m0 + (wm * 2 + mt) * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            if (gm >= M) continue;
            const float fa = OUT_I32 ? 0.0f : bf16_to_f32(sa[gm]);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                if (gcol[c] >= N) continue;
                const int v = acc[mt][c][r];
                if (OUT_I32)
                    acc_out[(int64_t)gm * N + gcol[c]] = v;
                else
                    out[(int64_t)gm * N + gcol[c]] = epilogue_bf16(v, fa, swf[c]);
            }
        }
    }
}

// Plain path: one wave per output row n, any K % 4 == 0 and any alignment.
template <bool OUT_I32>
__global__ __launch_bounds__(64) void gemm_plain(uint16_t* __restrict__ out, int32_t* __restrict__ acc_out,
                                                 const int8_t* __restrict__ x, const uint8_t* __restrict__ w,
                                                 const uint16_t* __restrict__ sa, const uint16_t* __restrict__ sw,
                                                 int M, int N, int K) {
    const int n = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t KB = K >> 2;
    for (int m = 0; m < M; ++m) {
        int acc = 0;
        for (int k = lane; k < K; k += 64) {
            const int code = (w[(int64_t)n * KB + (k >> 2)] >> (2 * (k & 3))) & 3;
            acc += (code - 2) * (int)x[(int64_t)m * K + k];
        }
        acc = wave_sum_i32(acc);
        if (lane == 0) {
            if (OUT_I32)
                acc_out[(int64_t)m * N + n] = acc;
            else
                out[(int64_t)m * N + n] = epilogue_bf16(acc, bf16_to_f32(sa[m]), bf16_to_f32(sw[n]));
        }
    }
}

template <bool OUT_I32>
hipError_t dispatch(uint16_t* out, int32_t* acc, const int8_t* x, const uint8_t* w, const uint16_t* sa,
                    const uint16_t* sw, int M, int N, int K, hipStream_t s) {
    const bool fast = (K % GM_KS == 0) && aligned16(x) && aligned16(w);
    if (!fast) {
        hipLaunchKernelGGL((gemm_plain<OUT_I32>), dim3((unsigned)N), dim3(64), 0, s, out, acc, x, w, sa, sw, M, N, K);
        return hipGetLastError();
    }
    const int tiles_m = (M + GM_BM - 1) / GM_BM;
    const int tiles_n = (N + GM_BN - 1) / GM_BN;
    // more than 64 KB of dynamic LDS: raise the kernel's limit (idempotent)
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_mfma_kernel<OUT_I32>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)GM_LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_mfma_kernel<OUT_I32>), dim3((unsigned)(tiles_m * tiles_n)), dim3(GM_THREADS),
                       GM_LDS_BYTES, s, out, acc, x, w, sa, sw, M, N, K, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(uint16_t* out, int32_t* acc, const int8_t* x, const uint8_t* w, const uint16_t* scale_act,
                       const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (acc != nullptr) return dispatch<true>(nullptr, acc, x, w, nullptr, nullptr, (int)M, (int)N, (int)K, s);
    return dispatch<false>(out, nullptr, x, w, scale_act, scale_wt, (int)M, (int)N, (int)K, s);
}

}  // namespace bitnet
