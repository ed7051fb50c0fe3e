// gemm.hip -- batched ternary x int8 GEMM on CDNA4 int8 MFMA (K-GEMM).
//
// Computes bitnet_gemm of "phanerozoic/bitnet-cpu v1,
// torch-ext/bitnet_cpu/__init__.py" for any M:
//   acc[m][n] = sum_k (code[n][k] - 2) * x_int8[m][k]     (exact int32)
//   out[m][n] = epilogue(acc, scale_act[m], scale_wt[n])   (or acc itself)
// The request post of "kernels-community/README discussion #1 (bitnet-tc kernel
// request)" runs this on the matrix units for batched shapes; here that is
// v_mfma_i32_32x32x32_i8 (32 x 32 output tile, 32 k per instruction, int32
// accumulators).
//
// Where the time goes on gfx950, and the layout that follows from it.  One CU
// retires about 3840 int8 MACs per clock on the 32x32x32 MFMA, reads LDS at
// about 184 B/clk with conflict-free ds_read_b128 and writes it at about
// 74 B/clk with ds_write_b128.  Staging both operands as int8 bytes in LDS
// costs more LDS time per MAC than the MFMAs take, so:
//
//  * B (packed weights) stays packed in LDS: 2 bits per weight, a quarter of
//    the bytes to write and to read.  A lane's B operand for one MFMA is 16
//    codes, i.e. one packed dword p of its column, expanded in registers as
//    (p >> 2e) & 0x03030303 for e = 0..3: byte r of dword e is the code of
//    element 4r + e.  That is 7 VALU per 16 weights, and the MFMA multiplies
//    the codes (1, 2, 3) themselves; acc = sum(code * x) - 2 * sum_k x[m][k].
//  * A (int8 activations) is staged through registers into LDS, each 16-byte
//    group 4x4-byte transposed on the way so that it has the same element
//    order as the expanded B dwords (dword e byte r = element 4r + e).  The same
//    pass sums the row's bytes (v_dot4 with 0x01010101) for the -2 * sum_k x term.
//  * Within a 128-element K stage, MFMA k-step s of lane half h covers elements
//    64h + 16s .. 64h + 16s + 15: then a lane's four B dwords for the whole
//    stage are 16 contiguous packed bytes (one ds_read_b128), and its A
//    fragment for step s is the 16-byte group 4h + s of its row.
//  * Block tile BM x BN with WAVES_M x WAVES_N waves, each owning a
//    (BM/WAVES_M) x (BN/WAVES_N) tile of 32 x 32 MFMA tiles.  Larger wave tiles
//    mean fewer LDS bytes per MAC; the register file bounds them.
//  * LDS slots are XOR-swizzled so that the staging writes (8 rows x 8 groups
//    per instruction for A; 32 columns x 2 halves for B) and the fragment reads
//    (lane-contiguous) keep every 8 and every 16 consecutive lanes on distinct
//    16-byte bank groups.
//  * Global loads are issued four stages ahead into three register sets; LDS
//    holds three stages, so a stage is stored two steps before it is multiplied
//    and the first fragments of the next stage are read at the end of each step
//    (one barrier per stage).  Every step issues the same loads (stage indices
//    past the end are clamped and never multiplied), so the waits the compiler
//    derives are exact.
//  * With BDMA (every block shape in use) the packed weights skip the registers: LDS
//    DMA loads (16 bytes per lane) put each stage into a ring of NS + 1 weight
//    stages, issued with that stage's activation loads, and each wave counts
//    its own outstanding loads down (vmcnt) before the barrier that publishes
//    the stage.
//
// Tiles are assigned XCD-aware: the hardware deals workgroups round-robin to
// the 8 XCDs, so the block index is remapped to give each XCD a contiguous run
// of tiles that share A row-panels in its own L2.
//
// The fast kernel needs K % 128 == 0 and 16-byte aligned x and w; anything
// else goes to gemm_plain (one wave per output column, same arithmetic).
#include "bitnet_device.h"
#include "launch.h"

namespace bitnet {

namespace {

constexpr int GM_KS = 128;     // K elements per pipeline stage (4 MFMA k-steps of 32)
constexpr int GROUP_M = 8;     // row panels swept per column tile (tile order)
// The same for one round of tiles on a grid of row panels x column tiles (the
// one-round eight-wave blocks): an XCD's 32 concurrent tiles then span 4 row
// panels x 8 column tiles instead of 8 x 4, so each activation panel is read
// by 2 XCDs instead of 4 (LLaMA-7B qkvo at M = 2048: HBM reads 40 -> 32 MB
// by count, 2.3% faster; down 0.4%).
constexpr int GROUP_M_ONE_ROUND = 4;
constexpr int GM_FRAG = 1024;  // bytes of one 32 x 32 int8 A operand fragment (64 lanes x 16 B)
// M * N from which few block tiles beat split-K: measured on the LLaMA-7B shapes,
// split-K still wins at 256 x 4096 (1.05 M outputs), the block tiles at
// 128 x 11008 (1.41 M) and 384 x 4096 (1.57 M).
constexpr int64_t GM_MID_MN = (int64_t)5 << 18;
constexpr int64_t GM_MID_BLOCKS = 160;           // blocks a mid-M block tile should give
// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format;
// stride 0, so bounds are checked against the byte count in word 2).
constexpr int BUFFER_RSRC_WORD3 = 0x00020000;
// Cache policy of the output tile stores: sc0 | sc1 (system coherence), i.e.
// written through the L2.
constexpr int STORE_WT = 17;

template <int BM, int BN, int WAVES_M, int WAVES_N, bool BDMA, int NS>
struct GemmShape {
    static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
    static constexpr int MT = BM / WAVES_M / 32;  // MFMA row tiles per wave
    static constexpr int NT = BN / WAVES_N / 32;  // MFMA column tiles per wave
    static constexpr int A_STAGE = BM * GM_KS;     // int8, [row tile][k-step] fragments
    static constexpr int B_STAGE = BN * GM_KS / 4; // packed, [column tile] of 32 x 32 B
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int A_CH = BM * (GM_KS / 16) / THREADS;  // 16-byte A groups per thread per stage
    static constexpr int B_CH = BN * 2 / THREADS;             // 16-byte B halves per thread per stage
    // LDS: three A (or A and B) stage buffers; with BDMA a separate ring of
    // NB = NS + 1 B stages after them; then row sums and scales.
    static constexpr int NB = NS + 1;
    static constexpr int A_BUF = BDMA ? A_STAGE : STAGE;
    static constexpr int B_RING = 3 * A_BUF;
    static constexpr int DATA = BDMA ? 3 * A_STAGE + NB * B_STAGE : 3 * STAGE;
    static constexpr int B_DMA = BN / 32 / (WAVES_M * WAVES_N);  // 1 KB B tiles each wave loads per stage
    static constexpr size_t LDS = (size_t)DATA + 8 * BM + 4 * BN;
    static_assert(!BDMA || B_DMA * 32 * WAVES_M * WAVES_N == BN, "whole B tiles per wave");
    static_assert(THREADS >= BM && THREADS >= BN, "one thread per block row / column fetches its scale");
    static_assert(BM % (32 * WAVES_M) == 0 && BN % (32 * WAVES_N) == 0, "wave tiles are whole MFMA tiles");
    static_assert(A_CH * THREADS == BM * 8 && B_CH * THREADS == BN * 2, "staging splits evenly");
};

__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int per = total / 8;
    const int rem = total % 8;
    const int xcd = bid % 8;
    const int idx = bid / 8;
    return xcd * per + min(xcd, rem) + idx;
}

// Byte offset, within a 1 KB A fragment of k-step s, of the 16-byte slot of
// fragment lane l (row l % 32, lane half h = l / 32).  Staging writes: eight
// consecutive lanes are one row's eight (h, s) groups, which the XOR with
// 2s + 9h sends to eight distinct slots mod 8, and sixteen consecutive lanes
// (two rows) to sixteen distinct slots mod 16; fragment reads: 16 consecutive
// lanes share h and s, so the XOR keeps them distinct.  (The counters read no
// LDS bank conflicts with it; an XOR with 2s + 8h left 1.2 conflict cycles per
// LDS instruction, at the same speed.)
__device__ __forceinline__ int a_slot(int l, int s) { return (l ^ (2 * s + 9 * (l >> 5))) * 16; }

// Byte offset, within the 1 KB packed B tile of 32 columns, of half h of
// column n (n < 32): 16 consecutive columns of one half fall on 16 distinct
// slots mod 16, as do eight columns x both halves.
__device__ __forceinline__ int b_slot(int n, int h) { return (2 * n + (h ^ ((n >> 3) & 1))) * 16; }

template <int A_CH, int B_CH>
struct StageRegs {
    v4u a[A_CH];
    v4u b[B_CH];
};
template <int A_CH>
struct StageRegs<A_CH, 0> {  // weights loaded straight into LDS: no B registers
    v4u a[A_CH];
};

// s_waitcnt on the vector-memory counter alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt and lgkmcnt at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16 bytes per lane from a buffer straight into LDS: lane l writes
// lds_dst + 16 l (lds_dst wave-uniform).  A device-only function: a lambda in
// a kernel is also compiled for the host, where this builtin does not exist.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_dst, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, soff, 0, 0);
}

// Workgroup barrier for LDS written by this wave's ds_write and by LDS DMA
// loads that have been waited for explicitly.  __syncthreads() would wait for
// every LDS DMA in flight (its release fence covers them), including those of
// stages far ahead; here each wave waits for its own LDS writes (lgkmcnt 0), the
// s_barrier joins the waves, and the wavefront-scope fences only keep the
// compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Epilogue of one wave's (32 MT) x (32 NT) accumulator tile, straight from
// the accumulators: register r of lane l of a 32 x 32 tile holds row
// 8(r/4) + 4(l/32) + r%4, column l%32.  (gm0, gn0) is the tile's first output
// element, (lr0, lc0) the same position within the block, whose row sums,
// row scales and column scales are in LDS.  whole: the block tile lies inside
// the output, so no bounds checks are needed.
template <int MT, int NT, bool OUT_I32>
__device__ __forceinline__ void store_tile(const v16i (&acc)[MT][NT], uint16_t* __restrict__ out,
                                           int32_t* __restrict__ acc_out, int M, int N, int gm0, int gn0, bool whole,
                                           int lr0, int lc0, int lane, const int* rowsum, const float* rowscale,
                                           const float* colscale) {
    if (whole) {
        // Branch-free buffer stores whose per-register row offset is a scalar,
        // two rows per bf16 conversion.  The stores write through the L2
        // (system-coherence bits): the tile is not read again by this kernel,
        // and lines left dirty in the L2s would be written back when the
        // kernel ends, after the last tile (measured: 1-3 % faster).
        constexpr int ES = OUT_I32 ? 4 : 2;
        void* dst = OUT_I32 ? static_cast<void*>(acc_out) : static_cast<void*>(out);
        const __amdgpu_buffer_rsrc_t o_rsrc =
            __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, M * N * ES, BUFFER_RSRC_WORD3);
        const int lrow0 = lr0 + (lane >> 5) * 4;  // block row of (t = 0, r = 0)
        const int lcol0 = lc0 + (lane & 31);
        float swf[NT];
#pragma unroll
        for (int u = 0; u < NT; ++u) swf[u] = colscale[lcol0 + u * 32];
        const int voff = ((gm0 + (lane >> 5) * 4) * N + gn0 + (lane & 31)) * ES;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int dr = t * 32 + (r >> 2) * 8 + (r & 3);  // row offset, lane-independent
                const int lr = lrow0 + dr;
                const int c0 = 2 * rowsum[lr], c1 = 2 * rowsum[lr + 1];
                const float a0 = rowscale[lr], a1 = rowscale[lr + 1];
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    const int soff = (dr * N + u * 32) * ES;
                    const int v0 = acc[t][u][r] - c0;
                    const int v1 = acc[t][u][r + 1] - c1;
                    if (OUT_I32) {
                        __builtin_amdgcn_raw_buffer_store_b32(v0, o_rsrc, voff, soff, STORE_WT);
                        __builtin_amdgcn_raw_buffer_store_b32(v1, o_rsrc, voff, soff + N * ES, STORE_WT);
                    } else {
                        const uint32_t pk = epilogue_bf16x2(v0, a0, v1, a1, swf[u]);
                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)pk, o_rsrc, voff, soff, STORE_WT);
                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pk >> 16), o_rsrc, voff, soff + N * ES, STORE_WT);
                    }
                }
            }
        }
        return;
    }
    float swf[NT];
    int gcol[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int lc = lc0 + u * 32 + (lane & 31);
        gcol[u] = gn0 + u * 32 + (lane & 31);
        swf[u] = colscale[lc];
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int dr = t * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            const int lr = lr0 + dr;
            const int gm = gm0 + dr;
            if (gm >= M) continue;
            const int corr = 2 * rowsum[lr];
            const float fa = rowscale[lr];
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                if (gcol[u] >= N) continue;
                const int v = acc[t][u][r] - corr;
                if (OUT_I32)
                    acc_out[(int64_t)gm * N + gcol[u]] = v;
                else
                    out[(int64_t)gm * N + gcol[u]] = epilogue_bf16(v, fa, swf[u]);
            }
        }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int WAVES_PER_EU, int NS, bool BDMA, bool OUT_I32>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) __attribute__((amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void gemm_mfma_kernel(uint16_t* __restrict__ out, int32_t* __restrict__ acc_out, const int8_t* __restrict__ x,
                      const uint8_t* __restrict__ w, const uint16_t* __restrict__ sa,
                      const uint16_t* __restrict__ sw, int M, int N, int K, int tiles_m, int tiles_n,
                      int group_m) {
    using S = GemmShape<BM, BN, WAVES_M, WAVES_N, BDMA, NS>;
    constexpr int MT = S::MT, NT = S::NT, A_CH = S::A_CH, B_CH = S::B_CH;
    constexpr int B_REG = BDMA ? 0 : B_CH;  // B halves staged through registers
    using Regs = StageRegs<A_CH, B_REG>;
    // k-steps by which A fragment reads run ahead of their MFMAs: two for
    // 64-row wave tiles (measured: 0.3-1.5% at M = 2048 on two boxes), one for 128-row tiles,
    // whose register budget the extra fragments would exceed
    constexpr int A_AHEAD = MT <= 2 ? 2 : 1;
    extern __shared__ __align__(16) uint8_t lds[];
    int* rowsum = reinterpret_cast<int*>(lds + S::DATA);
    float* rowscale = reinterpret_cast<float*>(lds + S::DATA + 4 * BM);
    float* colscale = reinterpret_cast<float*>(lds + S::DATA + 8 * BM);

    // Block -> tile: consecutive logical tiles land on one XCD (xcd_remap) and
    // sweep group_m row panels per column tile, so an XCD's concurrent tiles
    // share a few activation panels and a few weight panels in its L2.
    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int per_group = group_m * tiles_n;
    const int group = tile / per_group;
    const int first_m = group * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const int in_group = tile - group * per_group;
    const int tm = first_m + in_group % gsize;
    const int tn = in_group / gsize;
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N;
    const int wn = wave - wm * WAVES_N;
    const int KB = K >> 2;
    const int nk = K / GM_KS;

    // Staging loads are buffer loads: one SGPR resource per operand, a 32-bit
    // per-lane offset and the stage's K offset in an SGPR.  Rows past M and
    // columns past N lie past the end of their buffer and read as zero, which
    // contributes nothing (and they are never written out).
    const __amdgpu_buffer_rsrc_t x_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(x), (short)0, M * K, BUFFER_RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t w_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w), (short)0, N * KB, BUFFER_RSRC_WORD3);

    // A staging: group g = tid + THREADS * i covers row g / 8, 16-byte group
    // c = g % 8 (= tid % 8) of the stage's 128 bytes, i.e. lane half h = c / 4
    // and k-step s = c % 4.
    const int ac = tid & 7;
    int a_voff[A_CH], a_off[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int r = (tid >> 3) + (S::THREADS / 8) * i;
        a_voff[i] = (m0 + r) * K + ac * 16;
        a_off[i] = ((r >> 5) * 4 + (ac & 3)) * GM_FRAG + a_slot((r & 31) + 32 * (ac >> 2), ac & 3);
    }
    // B staging through registers: half g % 2 (= tid % 2) of column g / 2.
    const int bh = tid & 1;
    int b_voff[B_CH], b_off[B_CH];
#pragma unroll
    for (int j = 0; j < B_CH; ++j) {
        const int n = (tid >> 1) + (S::THREADS / 2) * j;
        b_voff[j] = (n0 + n) * KB + bh * 16;
        b_off[j] = S::A_STAGE + (n >> 5) * GM_FRAG + b_slot(n & 31, bh);
    }
    // B straight into LDS (BDMA): the d-th load of wave w fills 32-column tile
    // w + WAVES * d, lane l writing slot l, i.e. column l / 2, half
    // (l % 2) ^ bit 3 of the column (the inverse of b_slot).
    int bd_voff[S::B_DMA];
#pragma unroll
    for (int d = 0; d < S::B_DMA; ++d) {
        const int n = (wave + WAVES_M * WAVES_N * d) * 32 + (lane >> 1);
        bd_voff[d] = (n0 + n) * KB + ((lane & 1) ^ ((lane >> 4) & 1)) * 16;
    }
    // Scales for the epilogue, fetched now so that their latency hides under
    // the K loop, and parked in LDS after it.  The loads are unconditional
    // (clamped indices) and the values are converted only after the loop: a
    // load inside a branch, or a use of its value, would make the compiler
    // wait for it before the operand loads go out.
    uint16_t sa_bits = 0, sw_bits = 0;
    if constexpr (!OUT_I32) {
        sa_bits = sa[min(m0 + tid, M - 1)];
        sw_bits = sw[min(n0 + tid, N - 1)];
    }

    int rs[A_CH];  // this thread's share of sum_k x over its A rows
#pragma unroll
    for (int i = 0; i < A_CH; ++i) rs[i] = 0;

    // Global loads of stage st (clamped to the last stage past the end).  With
    // BDMA the B part goes straight into ring slot st % NB.
    auto load_stage = [&](int st, Regs& R) {
        const int kb = min(st, nk - 1) * GM_KS;  // wave-uniform
        if constexpr (BDMA) {
            uint8_t* ring = lds + S::B_RING + (st % S::NB) * S::B_STAGE;
#pragma unroll
            for (int d = 0; d < S::B_DMA; ++d)
                buffer_load_lds16(w_rsrc, ring + (wave + WAVES_M * WAVES_N * d) * GM_FRAG, bd_voff[d], kb >> 2);
        }
#pragma unroll
        for (int i = 0; i < A_CH; ++i) R.a[i] = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, a_voff[i], kb, 0);
        if constexpr (!BDMA) {
#pragma unroll
            for (int j = 0; j < B_CH; ++j) R.b[j] = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, b_voff[j], kb >> 2, 0);
        }
    };
    // The B tiles of stage k + 1 are issued with the loads of stage k + 1 (in
    // whatever order the compiler picks within that group); each of the NS - 1
    // later groups up to the barrier of step k issues B_DMA + A_CH more loads,
    // and vector-memory loads complete in issue order, so at most B_WAIT loads
    // may still be in flight when they have landed.  (The A loads of stage k + 1
    // have to complete a step earlier anyway, for their LDS store.)  The groups
    // stay apart: the loop steps are separated by barriers, the prologue's
    // groups by scheduling barriers.
    constexpr int B_WAIT = (NS - 1) * (S::B_DMA + A_CH);
    v16i acc[MT][NT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u) acc[t][u] = v16i{};

    int a_rd[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a_rd[s] = a_slot(lane, s);
    const int b_rd = b_slot(lane & 31, lane >> 5);

    // Staging of one 16-byte A group into LDS: transpose, store, and add its
    // bytes to the row sum (clamped repeats of the last stage are not summed).
    auto store_a = [&](uint8_t* base, int i, const v4u& v, int live) {
        const uint4 t = transpose4x4(v.x, v.y, v.z, v.w);
        *reinterpret_cast<v4u*>(base + a_off[i]) = v4u{t.x, t.y, t.z, t.w};
        int sum = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, 0, false);
        sum = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, sum, false);
        sum = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, sum, false);
        sum = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, sum, false);
        rs[i] += live * sum;
    };

    // Fragment reads: the packed B dwords of a whole stage, and the A
    // fragments of k-step s.  A reads run A_AHEAD k-steps ahead of their
    // MFMAs; the previous step reads the B dwords and the first A_AHEAD
    // k-steps' A fragments of the next stage.
    auto read_b = [&](const uint8_t* bbase, v4u (&pb)[NT]) {
        const uint8_t* B = bbase + (wn * NT) * GM_FRAG;
#pragma unroll
        for (int u = 0; u < NT; ++u) pb[u] = *reinterpret_cast<const v4u*>(B + u * GM_FRAG + b_rd);
    };
    auto read_a = [&](const uint8_t* base, int s, v4i (&af)[MT]) {
        const uint8_t* A = base + (wm * MT) * 4 * GM_FRAG;
#pragma unroll
        for (int t = 0; t < MT; ++t) af[t] = *reinterpret_cast<const v4i*>(A + (t * 4 + s) * GM_FRAG + a_rd[s]);
    };

    // One pipeline step k, between two barriers, with LDS buffer bi = k % 3:
    // issue the global loads of stage k+NS+1 into the register set that held
    // stage k+1, multiply stage k, move stage k+2 from its register set into
    // buffer (k+2) % 3, and read the first fragments of stage k+1 (written
    // during step k-1, visible since this step's barrier).  The program order
    // is chosen for overlap, because the compiler keeps LDS reads and writes in
    // program order (it cannot tell the buffers apart): each k-step's fragment
    // reads are issued before the MFMAs of the previous k-step, and the stores
    // of stage k+2 are spread over the k-steps.
    v4u pb[NT];
    v4i afn[A_AHEAD][MT];  // the next stage's first A_AHEAD k-steps
    auto b_of = [&](const uint8_t* abuf, int st) -> const uint8_t* {  // B tiles of stage st
        if constexpr (BDMA) return lds + S::B_RING + (st % S::NB) * S::B_STAGE;
        return abuf + S::A_STAGE;
    };
    auto step = [&](const int bi, int k, const Regs& SS, Regs& SL) {
        // stage k+1 visible; buffer (k+2) % 3 no longer read
        if constexpr (BDMA) {
            wait_vmcnt<B_WAIT>();  // this wave's B tiles of stage k+1 have landed
            lds_barrier();
        } else {
            __syncthreads();
        }
        // The global loads go out at raised wave priority, so that a wave leaving
        // the barrier issues them ahead of the MFMA and LDS work of the other
        // wave on its SIMD (measured: about one point of MFMA utilisation at M = 2048).
        __builtin_amdgcn_s_setprio(1);
        load_stage(k + NS + 1, SL);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads at the top
        __builtin_amdgcn_s_setprio(0);
        const uint8_t* cur = lds + bi * S::A_BUF;
        uint8_t* later = lds + ((bi + 2) % 3) * S::A_BUF;
        const uint8_t* next = lds + ((bi + 1) % 3) * S::A_BUF;
        const int live = (k + 2 < nk) ? 1 : 0;
        constexpr int R = A_AHEAD + 1;  // A fragment sets in flight
        v4i af[R][MT];
#pragma unroll
        for (int j = 0; j < A_AHEAD; ++j)
#pragma unroll
            for (int t = 0; t < MT; ++t) af[j][t] = afn[j][t];
        v4u pbc[NT];
#pragma unroll
        for (int u = 0; u < NT; ++u) pbc[u] = pb[u];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s + A_AHEAD < 4) {
                read_a(cur, s + A_AHEAD, af[(s + A_AHEAD) % R]);
            } else {  // k-step sn of the next stage (written during step k - 1)
                const int sn = s + A_AHEAD - 4;
                if (sn == 0) read_b(b_of(next, k + 1), pb);
                read_a(next, sn, afn[sn]);
            }
#pragma unroll
            for (int i = 0; i < A_CH; ++i)
                if (i % 4 == s) store_a(later, i, SS.a[i], live);
            if constexpr (!BDMA) {
                if (s == 1) {
#pragma unroll
                    for (int j = 0; j < B_CH; ++j) *reinterpret_cast<v4u*>(later + b_off[j]) = SS.b[j];
                }
            }
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                const uint32_t p = pbc[u][s];
                const v4i bf = {(int)(p & CODE_MASK), (int)((p >> 2) & CODE_MASK), (int)((p >> 4) & CODE_MASK),
                                (int)((p >> 6) & CODE_MASK)};
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[t][u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s % R][t], bf, acc[t][u], 0, 0, 0);
            }
        }
    };

    // Stage j lives in register set j % NS from its load (step j - NS - 1)
    // until its LDS store (step j - 2), and in LDS buffer j % 3 from its store
    // until it is multiplied.
    // With BDMA, stage j's B tiles are written into ring slot j % NB at step
    // j - NS - 1, after that step's barrier: the slot's previous stage, j - NB,
    // was last read during step j - NB - 1, which is why NB = NS + 1.
    constexpr int LEAD = NS + 1;
    Regs sets[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        load_stage(i, sets[i]);
        if constexpr (BDMA) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < A_CH; ++i) store_a(lds, i, sets[0].a[i], 1);
    if constexpr (!BDMA) {
#pragma unroll
        for (int j = 0; j < B_CH; ++j) *reinterpret_cast<v4u*>(lds + b_off[j]) = sets[0].b[j];
    }
#pragma unroll
    for (int i = 0; i < A_CH; ++i) store_a(lds + S::A_BUF, i, sets[1].a[i], nk > 1 ? 1 : 0);
    if constexpr (!BDMA) {
#pragma unroll
        for (int j = 0; j < B_CH; ++j) *reinterpret_cast<v4u*>(lds + S::STAGE + b_off[j]) = sets[1].b[j];
    }
    load_stage(NS, sets[0]);
    if constexpr (BDMA) {
        wait_vmcnt<B_WAIT>();  // B tiles of stages 0 and 1 have landed
        lds_barrier();
    } else {
        __syncthreads();
    }
    read_b(b_of(lds, 0), pb);
#pragma unroll
    for (int j = 0; j < A_AHEAD; ++j) read_a(lds, j, afn[j]);
    // stage k + i sits in LDS buffer (k + i) % 3; k advances by NS, so with
    // NS a multiple of 3 that is the constant i % 3
    int k = 0;
    for (; k + NS <= nk; k += NS) {
#pragma unroll
        for (int i = 0; i < NS; ++i)
            step(NS % 3 == 0 ? i % 3 : (k + i) % 3, k + i, sets[(i + 2) % NS], sets[(i + LEAD) % NS]);
    }
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
        if (k + i < nk) step(NS % 3 == 0 ? i % 3 : (k + i) % 3, k + i, sets[(i + 2) % NS], sets[(i + LEAD) % NS]);

    // The B tiles of the clamped stages past the end must land before the
    // workgroup ends and its LDS is reused.
    if constexpr (BDMA) wait_vmcnt<0>();
    // ---- row sums (the 8 threads of a row are aligned lanes) and row scales to LDS
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int v = group8_sum(rs[i]);
        if (ac == 0) rowsum[(tid >> 3) + (S::THREADS / 8) * i] = v;
    }
    if (tid < BM) rowscale[tid] = (!OUT_I32 && m0 + tid < M) ? bf16_to_f32(sa_bits) : 0.0f;
    if (tid < BN) colscale[tid] = (!OUT_I32 && n0 + tid < N) ? bf16_to_f32(sw_bits) : 0.0f;
    __syncthreads();

    store_tile<MT, NT, OUT_I32>(acc, out, acc_out, M, N, m0 + wm * MT * 32, n0 + wn * NT * 32,
                                m0 + BM <= M && n0 + BN <= N, wm * MT * 32, wn * NT * 32, lane, rowsum, rowscale,
                                colscale);
}

// Skinny path: few rows (M up to a few hundred), where the block tiles above
// would leave most CUs idle and each block would walk the whole K loop alone.
// A block owns a BM x BN output tile (BM = 32 * MT, BN = 32 * NT) and its KW
// waves split K: wave w takes the 128-element chunks w, w + KW, ...  Operands
// go straight from global memory into MFMA registers (no LDS staging, no
// barriers in the K loop): lane (r, h) loads, for each k-step s of a chunk,
// the 16 activation bytes 64h + 16s .. 64h + 16s + 15 of row r and transposes
// them, and the 16 packed bytes 16h .. 16h + 15 of the chunk of column r,
// which hold its B operand dwords for the four k-steps (the k order of the
// tiled kernel).  A ring of D chunks keeps loads in flight.  At the end the
// waves add their partial accumulators (and partial row sums) into an int32
// LDS tile with ds_add and the block writes the epilogue row by row.
template <int MT, int NT, int KW, int D, bool OUT_I32>
__global__ __launch_bounds__(64 * KW) void gemm_skinny_kernel(uint16_t* __restrict__ out,
                                                              int32_t* __restrict__ acc_out,
                                                              const int8_t* __restrict__ x,
                                                              const uint8_t* __restrict__ w,
                                                              const uint16_t* __restrict__ sa,
                                                              const uint16_t* __restrict__ sw, int M, int N, int K,
                                                              int tiles_n) {
    constexpr int BM = 32 * MT, BN = 32 * NT;
    constexpr int LDN = BN + 8;  // padded row: the two lane halves of an MFMA row group hit different banks
    constexpr int THREADS = 64 * KW;
    __shared__ int red[BM * LDN];
    __shared__ int rsum[BM];
    __shared__ float rscale[BM];
    __shared__ float cscale[BN];

    const int tm = blockIdx.x / tiles_n;
    const int tn = blockIdx.x - tm * tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int KB = K >> 2;
    const int nc = K / GM_KS;
    const int r = lane & 31, h = lane >> 5;

    for (int i = tid; i < BM * LDN; i += THREADS) red[i] = 0;
    for (int i = tid; i < BM; i += THREADS) rsum[i] = 0;
    // This thread's row and column scale (THREADS >= BM, BN): loaded now,
    // unconditionally from clamped indices, and converted and parked in LDS
    // only after the K loop, so that no wait for them precedes the operand loads.
    static_assert(THREADS >= BM && THREADS >= BN, "one thread per block row / column fetches its scale");
    uint16_t sa_bits = 0, sw_bits = 0;
    if constexpr (!OUT_I32) {
        sa_bits = sa[min(m0 + tid, M - 1)];
        sw_bits = sw[min(n0 + tid, N - 1)];
    }

    const __amdgpu_buffer_rsrc_t x_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(x), (short)0, M * K, BUFFER_RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t w_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w), (short)0, N * KB, BUFFER_RSRC_WORD3);
    int a_voff[MT], b_voff[NT];
#pragma unroll
    for (int t = 0; t < MT; ++t) a_voff[t] = (m0 + 32 * t + r) * K + 64 * h;  // rows past M read zeros
#pragma unroll
    for (int u = 0; u < NT; ++u) b_voff[u] = (n0 + 32 * u + r) * KB + 16 * h;  // columns past N read zeros

    struct Chunk {
        v4u a[MT][4];
        v4u b[NT];
    };
    auto load = [&](int j, Chunk& C) {
        const int c = wave + KW * j;  // only chunks of this wave (j < nj)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                C.a[t][s] = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, a_voff[t], c * GM_KS + 16 * s, 0);
#pragma unroll
        for (int u = 0; u < NT; ++u) C.b[u] = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, b_voff[u], c * (GM_KS / 4), 0);
    };

    v16i acc[MT][NT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u) acc[t][u] = v16i{};
    int rs[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) rs[t] = 0;

    auto compute = [&](const Chunk& C) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            v4i af[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const v4u v = C.a[t][s];
                const uint4 tt = transpose4x4(v.x, v.y, v.z, v.w);
                af[t] = v4i{(int)tt.x, (int)tt.y, (int)tt.z, (int)tt.w};
                int sum = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, rs[t], false);
                sum = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, sum, false);
                sum = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, sum, false);
                rs[t] = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, sum, false);
            }
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                const uint32_t p = C.b[u][s];
                const v4i bf = {(int)(p & CODE_MASK), (int)((p >> 2) & CODE_MASK), (int)((p >> 4) & CODE_MASK),
                                (int)((p >> 6) & CODE_MASK)};
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[t][u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[t], bf, acc[t][u], 0, 0, 0);
            }
        }
    };

    // The ring: each iteration issues the load D chunks ahead, except past the
    // wave's last chunk (such loads would only delay the split-K barrier); the
    // last < D chunks are already in.
    const int nj = (nc - 1 - wave) / KW + 1;  // chunks of this wave (the host guarantees nc >= KW)
    Chunk ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (i < nj) load(i, ring[i]);
    int j = 0;
    for (; j + D <= nj; j += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            compute(ring[i]);
            if (j + D + i < nj) load(j + D + i, ring[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (j + i < nj) compute(ring[i]);

    // ---- split-K reduction in LDS, then the epilogue
    if (tid < BM) rscale[tid] = (!OUT_I32 && m0 + tid < M) ? bf16_to_f32(sa_bits) : 0.0f;
    if (tid < BN) cscale[tid] = (!OUT_I32 && n0 + tid < N) ? bf16_to_f32(sw_bits) : 0.0f;
    __syncthreads();  // the tile is zeroed
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int u = 0; u < NT; ++u)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = 32 * t + 8 * (q >> 2) + 4 * h + (q & 3);
                atomicAdd(&red[row * LDN + 32 * u + r], acc[t][u][q]);
            }
        atomicAdd(&rsum[32 * t + r], rs[t]);
    }
    __syncthreads();
    for (int e = tid; e < BM * BN; e += THREADS) {
        const int row = e / BN, col = e - row * BN;
        const int gm = m0 + row, gn = n0 + col;
        if (gm < M && gn < N) {
            const int v = red[row * LDN + col] - 2 * rsum[row];
            if (OUT_I32)
                acc_out[(int64_t)gm * N + gn] = v;
            else
                out[(int64_t)gm * N + gn] = epilogue_bf16(v, rscale[row], cscale[col]);
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

template <int BM, int BN, int WAVES_M, int WAVES_N, int WAVES_PER_EU, int NS, bool BDMA, bool OUT_I32>
hipError_t launch_mfma(uint16_t* out, int32_t* acc, const int8_t* x, const uint8_t* w, const uint16_t* sa,
                       const uint16_t* sw, int M, int N, int K, hipStream_t s, int group_m = GROUP_M) {
    using S = GemmShape<BM, BN, WAVES_M, WAVES_N, BDMA, NS>;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    auto kern = gemm_mfma_kernel<BM, BN, WAVES_M, WAVES_N, WAVES_PER_EU, NS, BDMA, OUT_I32>;
    if (S::LDS > 65536) {
        const hipError_t e = raise_lds_limit(kern, S::LDS);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(tiles_m * tiles_n)), dim3(S::THREADS), S::LDS, s, out, acc, x, w, sa,
                       sw, M, N, K, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

// ---------------------------------------------------------------- skinny kernel, LDS-staged operands
//
// The same split-K tiling as gemm_skinny_kernel, but each wave stages its
// 256-element chunk of both operands through its own LDS region, so that the
// global loads read whole row segments: the weights as 16 rows x 64 bytes and
// the activations as 4 rows x 256 bytes per wave instruction, instead of the
// 32 rows x 32 bytes that loading MFMA fragments directly touches.  The
// fragments are then read from LDS (rows padded so that the reads hit distinct
// banks) in the same k order as the direct kernel: lane (r, h), k-step s, holds
// elements 128h + 16s .. 128h + 16s + 15 of the chunk.  The region is private
// to the wave (LDS operations of one wave complete in order), so no barrier is
// needed until the split-K reduction; the next chunk's global loads are in
// flight while the current one is multiplied.
constexpr int GS_KS = 256;            // K elements per chunk
constexpr int GS_XROW = GS_KS + 16;   // bytes per staged activation row (padded)
constexpr int GS_WROW = GS_KS / 4 + 16;  // bytes per staged weight row (padded)

// XR: activation rows staged per chunk (a multiple of 4, at most 32 * MT).
// With XR < 32 * MT (few rows: M <= XR within the block's single row tile)
// only those rows are loaded and stored; the wave zeroes the others once.
template <int MT, int NT, int KW, int D, bool OUT_I32, int XR>
__global__ __launch_bounds__(64 * KW) void gemm_skinny_lds_kernel(uint16_t* __restrict__ out,
                                                                  int32_t* __restrict__ acc_out,
                                                                  const int8_t* __restrict__ x,
                                                                  const uint8_t* __restrict__ w,
                                                                  const uint16_t* __restrict__ sa,
                                                                  const uint16_t* __restrict__ sw, int M, int N, int K,
                                                                  int tiles_n) {
    constexpr int BM = 32 * MT, BN = 32 * NT;
    constexpr int LDN = BN + 8;
    constexpr int THREADS = 64 * KW;
    constexpr int XB = BM * GS_XROW;  // staged activation bytes per wave
    constexpr int WB = BN * GS_WROW;  // staged weight bytes per wave
    __shared__ __align__(16) uint8_t stage[KW][XB + WB];
    __shared__ int red[BM * LDN];
    __shared__ int rsum[BM];
    __shared__ float rscale[BM];
    __shared__ float cscale[BN];

    const int tm = blockIdx.x / tiles_n;
    const int tn = blockIdx.x - tm * tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int KB = K >> 2;
    const int nc = K / GS_KS;
    const int r = lane & 31, h = lane >> 5;

    for (int i = tid; i < BM * LDN; i += THREADS) red[i] = 0;
    for (int i = tid; i < BM; i += THREADS) rsum[i] = 0;
    // This thread's row and column scale (THREADS >= BM, BN): loaded now,
    // unconditionally from clamped indices, and converted and parked in LDS
    // only after the K loop, so that no wait for them precedes the operand loads.
    static_assert(THREADS >= BM && THREADS >= BN, "one thread per block row / column fetches its scale");
    uint16_t sa_bits = 0, sw_bits = 0;
    if constexpr (!OUT_I32) {
        sa_bits = sa[min(m0 + tid, M - 1)];
        sw_bits = sw[min(n0 + tid, N - 1)];
    }

    const __amdgpu_buffer_rsrc_t x_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(x), (short)0, M * K, BUFFER_RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t w_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w), (short)0, N * KB, BUFFER_RSRC_WORD3);
    // global pieces of this lane: activation rows 4i + lane/16 (16 bytes at
    // lane%16), weight rows 16i + lane/4 (16 bytes at lane%4); rows past M or N
    // read zeros
    const int xr_l = lane >> 4, xp_l = lane & 15;
    const int wr_l = lane >> 2, wp_l = lane & 3;
    uint8_t* const xs = stage[wave];
    uint8_t* const ws = stage[wave] + XB;

    static_assert(XR % 4 == 0 && XR <= BM && (XR == BM || MT == 1), "staged rows: whole load instructions of one tile");
    constexpr int XI = XR / 4;   // activation load instructions per chunk
    constexpr int WI = BN / 16;  // weight load instructions per chunk
    if constexpr (XR < BM) {     // rows XR .. BM-1 of this wave's activation stage stay zero
        constexpr int ZW = (BM - XR) * GS_XROW / 16;  // 16-byte words to clear
        for (int i = lane; i < ZW; i += 64)
            *reinterpret_cast<v4u*>(xs + XR * GS_XROW + 16 * i) = v4u{0u, 0u, 0u, 0u};
    }
    struct ChunkRegs {
        v4u xg[XI], wg[WI];
    };
    ChunkRegs sets[D];  // the loads of D chunks in flight
    auto load = [&](int c, ChunkRegs& G) {
#pragma unroll
        for (int i = 0; i < XI; ++i)
            G.xg[i] = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, (m0 + 4 * i + xr_l) * K + 16 * xp_l, c * GS_KS, 0);
#pragma unroll
        for (int i = 0; i < WI; ++i)
            G.wg[i] = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, (n0 + 16 * i + wr_l) * KB + 16 * wp_l,
                                                            c * (GS_KS / 4), 0);
    };
    auto store = [&](const ChunkRegs& G) {
#pragma unroll
        for (int i = 0; i < XI; ++i)
            *reinterpret_cast<v4u*>(xs + (4 * i + xr_l) * GS_XROW + 16 * xp_l) = G.xg[i];
#pragma unroll
        for (int i = 0; i < WI; ++i)
            *reinterpret_cast<v4u*>(ws + (16 * i + wr_l) * GS_WROW + 16 * wp_l) = G.wg[i];
    };

    v16i acc[MT][NT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u) acc[t][u] = v16i{};
    int rs[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) rs[t] = 0;

    auto compute = [&]() {
        v4u bw[NT][2];  // this lane's 32 weight bytes of each column tile (8 k-steps)
#pragma unroll
        for (int u = 0; u < NT; ++u)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                bw[u][i] = *reinterpret_cast<const v4u*>(ws + (32 * u + r) * GS_WROW + 32 * h + 16 * i);
#pragma unroll
        for (int s = 0; s < GS_KS / 32; ++s) {
            v4i af[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const v4u v = *reinterpret_cast<const v4u*>(xs + (32 * t + r) * GS_XROW + 128 * h + 16 * s);
                const uint4 tt = transpose4x4(v.x, v.y, v.z, v.w);
                af[t] = v4i{(int)tt.x, (int)tt.y, (int)tt.z, (int)tt.w};
                int sum = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, rs[t], false);
                sum = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, sum, false);
                sum = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, sum, false);
                rs[t] = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, sum, false);
            }
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                const uint32_t p = bw[u][s >> 2][s & 3];
                const v4i bf = {(int)(p & CODE_MASK), (int)((p >> 2) & CODE_MASK), (int)((p >> 4) & CODE_MASK),
                                (int)((p >> 6) & CODE_MASK)};
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[t][u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[t], bf, acc[t][u], 0, 0, 0);
            }
        }
    };

    // chunks wave, wave + KW, ...: the loads of the D chunks after the current
    // one are in flight while it is multiplied.  Nothing is loaded past the
    // wave's last chunk: a load issued there would only delay the split-K
    // barrier below, which waits for every load in flight (measured 3-9%
    // faster at M = 32..128 than issuing clamped repeats of the last chunk).
    const int nj = (nc - 1 - wave) / KW + 1;  // the host guarantees nc >= KW
    auto chunk = [&](int j) { return wave + KW * j; };
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d < nj) load(chunk(d), sets[d]);
    int j = 0;
    for (; j + D <= nj; j += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            store(sets[d]);  // after the previous chunk's fragment reads (same wave: in order)
            if (j + d + D < nj) load(chunk(j + d + D), sets[d]);
            compute();
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        if (j + d < nj) {
            store(sets[d]);
            compute();
        }
    }

    // ---- split-K reduction in LDS, then the epilogue
    if (tid < BM) rscale[tid] = (!OUT_I32 && m0 + tid < M) ? bf16_to_f32(sa_bits) : 0.0f;
    if (tid < BN) cscale[tid] = (!OUT_I32 && n0 + tid < N) ? bf16_to_f32(sw_bits) : 0.0f;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int u = 0; u < NT; ++u)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = 32 * t + 8 * (q >> 2) + 4 * h + (q & 3);
                atomicAdd(&red[row * LDN + 32 * u + r], acc[t][u][q]);
            }
        atomicAdd(&rsum[32 * t + r], rs[t]);
    }
    __syncthreads();
    for (int e = tid; e < BM * BN; e += THREADS) {
        const int row = e / BN, col = e - row * BN;
        const int gm = m0 + row, gn = n0 + col;
        if (gm < M && gn < N) {
            const int v = red[row * LDN + col] - 2 * rsum[row];
            if (OUT_I32)
                acc_out[(int64_t)gm * N + gn] = v;
            else
                out[(int64_t)gm * N + gn] = epilogue_bf16(v, rscale[row], cscale[col]);
        }
    }
}

template <int MT, int NT, int KW, bool OUT_I32>
hipError_t launch_skinny_lds(uint16_t* out, int32_t* acc, const int8_t* x, const uint8_t* w, const uint16_t* sa,
                             const uint16_t* sw, int M, int N, int K, hipStream_t s) {
    const int tiles_m = (M + 32 * MT - 1) / (32 * MT);
    const int tiles_n = (N + 32 * NT - 1) / (32 * NT);
    constexpr int D = 1;  // chunks in flight per wave besides the one being multiplied
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(64 * KW);
    // Few rows: stage only the activation rows that exist, rounded up to 4, 8
    // or (one column tile) 16; measured on the LLaMA-7B and BitNet-2B-4T shapes
    // at M = 1 ... 16: 7-14% faster at M <= 4, 4-10% at M = 8, up to 5% at 16
    // rows with one column tile, 1-3% slower at 12-16 rows with two.
    if constexpr (MT == 1) {
        if (M <= 4) {
            hipLaunchKernelGGL((gemm_skinny_lds_kernel<MT, NT, KW, D, OUT_I32, 4>), grid, block, 0, s, out, acc, x, w,
                               sa, sw, M, N, K, tiles_n);
            return hipGetLastError();
        }
        if (M <= 8) {
            hipLaunchKernelGGL((gemm_skinny_lds_kernel<MT, NT, KW, D, OUT_I32, 8>), grid, block, 0, s, out, acc, x, w,
                               sa, sw, M, N, K, tiles_n);
            return hipGetLastError();
        }
        if (NT == 1 && M <= 16) {
            hipLaunchKernelGGL((gemm_skinny_lds_kernel<MT, NT, KW, D, OUT_I32, 16>), grid, block, 0, s, out, acc, x, w,
                               sa, sw, M, N, K, tiles_n);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_skinny_lds_kernel<MT, NT, KW, D, OUT_I32, 32 * MT>), grid, block, 0, s, out, acc, x, w,
                       sa, sw, M, N, K, tiles_n);
    return hipGetLastError();
}

template <int MT, int NT, int KW, int D, bool OUT_I32>
hipError_t launch_skinny(uint16_t* out, int32_t* acc, const int8_t* x, const uint8_t* w, const uint16_t* sa,
                         const uint16_t* sw, int M, int N, int K, hipStream_t s) {
    const int tiles_m = (M + 32 * MT - 1) / (32 * MT);
    const int tiles_n = (N + 32 * NT - 1) / (32 * NT);
    hipLaunchKernelGGL((gemm_skinny_kernel<MT, NT, KW, D, OUT_I32>), dim3((unsigned)(tiles_m * tiles_n)),
                       dim3(64 * KW), 0, s, out, acc, x, w, sa, sw, M, N, K, tiles_n);
    return hipGetLastError();
}

template <bool OUT_I32>
hipError_t launch_tiles(uint16_t* out, int32_t* acc, const int8_t* x, const uint8_t* w, const uint16_t* sa,
                        const uint16_t* sw, int M, int N, int K, hipStream_t s) {
    // Tile choice, by the number of 128 x 256 block tiles.  At least one per
    // CU: the block-tiled kernel (the large-M choice at the end).  Fewer, and
    // fewer than GM_MID_MN outputs (else the mid-M blocks below): a split-K
    // skinny kernel (each wave needs at least one chunk of K): the LDS-staged
    // one when K % 256 == 0, else the direct one.  Configurations measured on
    // the LLaMA-7B layer shapes: short rings and more resident waves beat deep
    // per-wave prefetch here.
    const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + 255) / 256);
    const int nc = K / GM_KS;
    if (M <= 64 && tiles >= 256) {
        // Few rows but very many columns (an LM head): 128-row blocks would
        // spend most of their MFMAs on padding rows, so the block is cut to 32
        // or 64 rows (four waves, 32 x 64 or 64 x 64 each).  Measured on the
        // 128256 x 2560 head: 1.5-1.6x faster than 128-row blocks at M = 8 ... 64.
        if (M <= 32) return launch_mfma<32, 256, 1, 4, 2, 3, true, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
        return launch_mfma<64, 256, 1, 4, 2, 3, true, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
    }
    if (tiles < 256 && (int64_t)M * N >= GM_MID_MN) {
        // Mid-sized M: the split-K kernels re-read the activations once per 64
        // output columns, which costs more than leaving CUs idle in a block-tiled
        // kernel.  Take the largest block tile that still gives GM_MID_BLOCKS
        // blocks (measured on the LLaMA-7B shapes at M = 128 ... 1024); the
        // smallest, 64 x 128, has four 32 x 64 wave tiles, so that even a few
        // blocks put one wave on every SIMD they occupy.
        if (tiles >= GM_MID_BLOCKS) return launch_mfma<128, 256, 2, 4, 2, 3, true, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
        if ((int64_t)((M + 127) / 128) * ((N + 127) / 128) >= GM_MID_BLOCKS)
            return launch_mfma<128, 128, 2, 2, 2, 3, true, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
        return launch_mfma<64, 128, 2, 2, 2, 3, true, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
    }
    if (tiles < 256 && K % GS_KS == 0 && K / GS_KS >= 4) {
        // LDS-staged skinny kernel (configurations measured on the LLaMA-7B
        // layer shapes at M = 8 ... 256; wide layers take two column tiles)
        const int ncs = K / GS_KS;
        const bool wide = N >= 8192;
        if (ncs >= 8) {
            if (M <= 32) {
                if (wide) return launch_skinny_lds<1, 2, 8, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
                return launch_skinny_lds<1, 1, 8, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
            }
            if (M <= 64) {
                if (wide) return launch_skinny_lds<1, 2, 4, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
                return launch_skinny_lds<1, 1, 8, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
            }
            if (M <= 128) {
                if (wide) return launch_skinny_lds<1, 2, 4, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
                return launch_skinny_lds<1, 2, 8, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
            }
            return launch_skinny_lds<2, 2, 4, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
        }
        if (M <= 64) return launch_skinny_lds<1, 1, 4, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
        if (M <= 128) return launch_skinny_lds<1, 2, 4, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
        return launch_skinny_lds<2, 2, 4, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
    }
    if (tiles < 256 && nc >= 4) {  // K % 256 != 0: the direct kernel
        // wide layers: two column tiles per block halve the activation re-reads
        if (M <= 64 && N >= 8192 && nc >= 8) return launch_skinny<1, 2, 8, 1, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
        if (M <= 16 && nc >= 8) return launch_skinny<1, 1, 8, 1, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
        if (M <= 64) return launch_skinny<1, 1, 4, 1, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
        if (M <= 128) return launch_skinny<1, 2, 4, 1, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
        return launch_skinny<2, 2, 4, 1, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
    }
    // Large M.  128 x 512 blocks (eight 128 x 64 wave tiles, two waves per
    // SIMD) spend the least VALU per MFMA; they are taken when their rounds of
    // 256 blocks come out at least 85 % full.  Otherwise, with more than 256
    // blocks of 128 x 256, four-wave 128 x 256 blocks (128 x 64 wave tiles),
    // two resident per CU, so that a last partial round still keeps two waves
    // on the SIMDs it occupies; with at most 256, one eight-wave block per CU
    // (64 x 64 wave tiles).  Measured on the LLaMA-7B shapes at M = 2048 and
    // 4096 (e.g. gate_up, M = 2048: 688 blocks, four-wave blocks 6 % faster;
    // qkvo, M = 4096: 256 wide blocks, 15 % faster than 128 x 256).
    const int64_t wide_tiles = (int64_t)((M + 127) / 128) * ((N + 511) / 512);
    const int64_t wide_rounds = (wide_tiles + 255) / 256;
    if (wide_tiles >= 256 && wide_tiles * 100 >= wide_rounds * 256 * 85)
        return launch_mfma<128, 512, 1, 8, 2, 3, true, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
    if (tiles > 256) return launch_mfma<128, 256, 1, 4, 2, 2, true, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s);
    return launch_mfma<128, 256, 2, 4, 2, 3, true, OUT_I32>(out, acc, x, w, sa, sw, M, N, K, s, GROUP_M_ONE_ROUND);
}

template <bool OUT_I32>
hipError_t dispatch(uint16_t* out, int32_t* acc, const int8_t* x, const uint8_t* w, const uint16_t* sa,
                    const uint16_t* sw, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    // The MFMA kernel addresses x, w and the output with 32-bit byte offsets
    // (buffer loads and stores).  Rows are processed in chunks that keep every
    // offset below 2^31, including those of the tile rows past the end of a
    // chunk; weights whose padded size reaches 2^31 bytes take the plain path.
    constexpr int64_t LIMIT = (int64_t)1 << 31;
    const int64_t KB = K / 4;
    const int64_t row_bytes = K > 4 * N ? K : 4 * N;
    const int64_t chunk = ((LIMIT - 1) / row_bytes - 128) / 128 * 128;
    const bool fast = (K % GM_KS == 0) && aligned16(x) && aligned16(w) && (N + 511) * KB < LIMIT && chunk >= 128;
    if (!fast) {
        hipLaunchKernelGGL((gemm_plain<OUT_I32>), dim3((unsigned)N), dim3(64), 0, s, out, acc, x, w, sa, sw, (int)M,
                           (int)N, (int)K);
        return hipGetLastError();
    }
    for (int64_t r0 = 0; r0 < M; r0 += chunk) {
        const int64_t rows = M - r0 < chunk ? M - r0 : chunk;
        const hipError_t e = launch_tiles<OUT_I32>(OUT_I32 ? nullptr : out + r0 * N, OUT_I32 ? acc + r0 * N : nullptr,
                                                   x + r0 * K, w, OUT_I32 ? nullptr : sa + r0, sw, (int)rows, (int)N,
                                                   (int)K, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemm(uint16_t* out, int32_t* acc, const int8_t* x, const uint8_t* w, const uint16_t* scale_act,
                       const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (acc != nullptr) return dispatch<true>(nullptr, acc, x, w, nullptr, nullptr, M, N, K, s);
    return dispatch<false>(out, nullptr, x, w, scale_act, scale_wt, M, N, K, s);
}

}  // namespace bitnet
