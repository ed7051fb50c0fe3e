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

constexpr int GM_BM = 128;
constexpr int GM_BN = 128;
constexpr int GM_THREADS = 256;

template <int KT>
struct GemmCfg {
    static constexpr int S = KT / 64;                 // MFMA k-steps per K-tile
    static constexpr int ROWB = KT + 16;              // LDS bytes per A row (padded)
    static constexpr int GROUPS = KT / 16;            // 16-byte A pieces per row per K-tile
    static constexpr int PPT = GM_BM * GROUPS / GM_THREADS;  // A pieces per thread
    static constexpr int LDS_A = GM_BM * ROWB;        // one buffer
    static constexpr size_t LDS_BYTES = 2 * (size_t)LDS_A + GM_BM * sizeof(int);
};

// 4x4 byte transpose (see gemv.hip): t_e byte r = element 4r + e.
__device__ __forceinline__ uint4 transpose16(const uint4& n) {
    const uint32_t u01lo = __builtin_amdgcn_perm(n.y, n.x, 0x05010400u);
    const uint32_t u01hi = __builtin_amdgcn_perm(n.y, n.x, 0x07030602u);
    const uint32_t u23lo = __builtin_amdgcn_perm(n.w, n.z, 0x05010400u);
    const uint32_t u23hi = __builtin_amdgcn_perm(n.w, n.z, 0x07030602u);
    uint4 t;
    t.x = __builtin_amdgcn_perm(u23lo, u01lo, 0x05040100u);
    t.y = __builtin_amdgcn_perm(u23lo, u01lo, 0x07060302u);
    t.z = __builtin_amdgcn_perm(u23hi, u01hi, 0x05040100u);
    t.w = __builtin_amdgcn_perm(u23hi, u01hi, 0x07060302u);
    return t;
}

template <int S>
struct BPack {
    uint32_t d[S];
};

__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int per = total / 8;
    const int rem = total % 8;
    const int xcd = bid % 8;
    const int idx = bid / 8;
    return xcd * per + min(xcd, rem) + idx;
}

template <int KT, bool OUT_I32>
__global__ __launch_bounds__(GM_THREADS) void gemm_mfma_kernel(uint16_t* __restrict__ out,
                                                               int32_t* __restrict__ acc_out,
                                                               const int8_t* __restrict__ x,
                                                               const uint8_t* __restrict__ w,
                                                               const uint16_t* __restrict__ sa,
                                                               const uint16_t* __restrict__ sw, int M, int N, int K,
                                                               int tiles_m, int tiles_n) {
    using C = GemmCfg<KT>;
    constexpr int S = C::S;
    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t* As0 = lds;
    uint8_t* As1 = lds + C::LDS_A;
    int* rowsum_lds = reinterpret_cast<int*>(lds + 2 * C::LDS_A);

    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int tm = tile / tiles_n;
    const int tn = tile - tm * tiles_n;
    const int m0 = tm * GM_BM;
    const int n0 = tn * GM_BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int j16 = lane & 15;
    const int g4 = lane >> 4;
    const int64_t KB = K >> 2;

    // A staging: piece p = tid + 256 i -> row p / GROUPS, 16-byte group p % GROUPS.
    const int8_t* a_src[C::PPT];
    bool a_row_ok[C::PPT];
#pragma unroll
    for (int i = 0; i < C::PPT; ++i) {
        const int p = tid + GM_THREADS * i;
        const int row = p / C::GROUPS;
        const int grp = p % C::GROUPS;
        const int gm = m0 + row;
        a_row_ok[i] = gm < M;
        a_src[i] = x + (int64_t)(a_row_ok[i] ? gm : 0) * K + grp * 16;
    }
    // B: this lane's column in each of the wave's four 16-column tiles.
    const uint8_t* b_src[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int gn = min(n0 + wn * 64 + ct * 16 + j16, N - 1);
        b_src[ct] = w + (int64_t)gn * KB + g4 * 4 * S;
    }

    uint4 a_reg[C::PPT];
    BPack<S> b_cur[4], b_nxt[4];
    int rs[C::PPT];
#pragma unroll
    for (int i = 0; i < C::PPT; ++i) rs[i] = 0;

    auto load_a = [&](int kt) {
        const int kb = kt * KT;
#pragma unroll
        for (int i = 0; i < C::PPT; ++i) {
            const int grp = (tid + GM_THREADS * i) % C::GROUPS;
            if (a_row_ok[i] && kb + grp * 16 < K)
                a_reg[i] = *reinterpret_cast<const uint4*>(a_src[i] + kb);
            else
                a_reg[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto load_b = [&](int kt, BPack<S> (&dst)[4]) {
        const int kb = kt * KT;
        const bool ok = kb + g4 * 16 * S < K;  // K % 64 == 0: a lane's bytes are all in range or all out
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            if (ok) {
                if constexpr (S == 4) {
                    const uint4 v = *reinterpret_cast<const uint4*>(b_src[ct] + (kb >> 2));
                    dst[ct].d[0] = v.x; dst[ct].d[1] = v.y; dst[ct].d[2] = v.z; dst[ct].d[3] = v.w;
                } else if constexpr (S == 2) {
                    const uint2 v = *reinterpret_cast<const uint2*>(b_src[ct] + (kb >> 2));
                    dst[ct].d[0] = v.x; dst[ct].d[1] = v.y;
                } else {
                    dst[ct].d[0] = *reinterpret_cast<const uint32_t*>(b_src[ct] + (kb >> 2));
                }
            } else {
#pragma unroll
                for (int s = 0; s < S; ++s) dst[ct].d[s] = 0u;
            }
        }
    };
    auto store_a = [&](uint8_t* As) {
#pragma unroll
        for (int i = 0; i < C::PPT; ++i) {
            const int p = tid + GM_THREADS * i;
            const int row = p / C::GROUPS;
            const int grp = p % C::GROUPS;
            int s = __builtin_amdgcn_sdot4((int)a_reg[i].x, 0x01010101, rs[i], false);
            s = __builtin_amdgcn_sdot4((int)a_reg[i].y, 0x01010101, s, false);
            s = __builtin_amdgcn_sdot4((int)a_reg[i].z, 0x01010101, s, false);
            rs[i] = __builtin_amdgcn_sdot4((int)a_reg[i].w, 0x01010101, s, false);
            *reinterpret_cast<uint4*>(As + row * C::ROWB + grp * 16) = transpose16(a_reg[i]);
        }
    };

    v4i acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[mt][ct] = v4i{0, 0, 0, 0};

    auto compute = [&](const uint8_t* As, const BPack<S> (&b)[4]) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            v4i af[4], bf[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                af[mt] = *reinterpret_cast<const v4i*>(As + (wm * 64 + mt * 16 + j16) * C::ROWB + (g4 * S + s) * 16);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const uint32_t p = b[ct].d[s];
                bf[ct] = v4i{(int)(p & CODE_MASK), (int)((p >> 2) & CODE_MASK), (int)((p >> 4) & CODE_MASK),
                             (int)((p >> 6) & CODE_MASK)};
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    acc[mt][ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], bf[ct], acc[mt][ct], 0, 0, 0);
        }
    };

    const int nk = (K + KT - 1) / KT;
    load_a(0);
    load_b(0, b_cur);
    store_a(As0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        uint8_t* cur = (kt & 1) ? As1 : As0;
        uint8_t* nxt = (kt & 1) ? As0 : As1;
        const bool more = kt + 1 < nk;
        if (more) {
            load_a(kt + 1);
            load_b(kt + 1, b_nxt);
        }
        compute(cur, b_cur);
        if (more) store_a(nxt);
        __syncthreads();
        if (more) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) b_cur[ct] = b_nxt[ct];
        }
    }

    // Row sums of the A tile: the GROUPS threads of a row are consecutive lanes.
#pragma unroll
    for (int i = 0; i < C::PPT; ++i) {
        int v = rs[i];
        v += dpp_mov<DPP_QUAD_XOR1>(v);
        v += dpp_mov<DPP_QUAD_XOR2>(v);
        v += dpp_mov<DPP_ROW_HALF_MIRROR>(v);
        if constexpr (C::GROUPS == 16) v += dpp_mov<DPP_ROW_MIRROR>(v);
        const int p = tid + GM_THREADS * i;
        if ((p % C::GROUPS) == 0) rowsum_lds[p / C::GROUPS] = v;
    }
    __syncthreads();

#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int lrow = wm * 64 + mt * 16 + g4 * 4 + r;
            const int gm = m0 + lrow;
            if (gm >= M) continue;
            const int corr = 2 * rowsum_lds[lrow];
            const float fa = OUT_I32 ? 0.0f : bf16_to_f32(sa[gm]);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const int gn = n0 + wn * 64 + ct * 16 + j16;
                if (gn >= N) continue;
                const int v = acc[mt][ct][r] - corr;
                if (OUT_I32)
                    acc_out[(int64_t)gm * N + gn] = v;
                else
                    out[(int64_t)gm * N + gn] = epilogue_bf16(v, fa, bf16_to_f32(sw[gn]));
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

constexpr int GEMM_KT = 128;

template <bool OUT_I32>
hipError_t dispatch(uint16_t* out, int32_t* acc, const int8_t* x, const uint8_t* w, const uint16_t* sa,
                    const uint16_t* sw, int M, int N, int K, hipStream_t s) {
    const bool fast = (K % 64 == 0) && aligned16(x) && aligned16(w);
    if (!fast) {
        hipLaunchKernelGGL((gemm_plain<OUT_I32>), dim3((unsigned)N), dim3(64), 0, s, out, acc, x, w, sa, sw, M, N, K);
        return hipGetLastError();
    }
    using C = GemmCfg<GEMM_KT>;
    const int tiles_m = (M + GM_BM - 1) / GM_BM;
    const int tiles_n = (N + GM_BN - 1) / GM_BN;
    hipLaunchKernelGGL((gemm_mfma_kernel<GEMM_KT, OUT_I32>), dim3((unsigned)(tiles_m * tiles_n)), dim3(GM_THREADS),
                       C::LDS_BYTES, s, out, acc, x, w, sa, sw, M, N, K, tiles_m, tiles_n);
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
