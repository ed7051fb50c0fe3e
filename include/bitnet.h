/*
 * bitnet.h -- C ABI of the MI355X (gfx950) W1.58A8 linear layer.
 *
 * The layer is BitNet b1.58's ternary-weight x INT8-activation matmul as
 * described in "phanerozoic/bitnet-cpu v1, torch-ext/bitnet_cpu/__init__.py"
 * (module docstring and the functions pack_weights, quantize_activation,
 * bitnet_gemm, bitnet_gemv_fused and bitnet_linear) and in
 * "kernels-community/README discussion #1 (bitnet-tc kernel request)"
 * (request post: 2-bit packing, per-token INT8 activations, a batched matrix
 * unit path and a fused decode path; numbers post: int32 accumulation).
 *
 * Conventions for every call:
 *   - All matrices are row-major and dense (leading stride = row length).
 *   - bf16 values travel as their uint16_t bit patterns.
 *   - Shapes: x / x_int8 are [M][K]; packed weights are [N][K/4]; outputs are
 *     [M][N]; scale_act is [M]; scale_wt is [N].
 *   - Buffers are owned by the caller.  The library never allocates, frees or
 *     synchronises device memory.  Its only state is per device and set once:
 *     a cached architecture check, a flag per GEMM kernel instance recording
 *     that its dynamic LDS limit has been raised (hipFuncSetAttribute), and
 *     the device's static arrays (two small always-cached pads that the
 *     surplus ring loads of the decode GEMV kernels read, and the scratch of
 *     bitnet_linear_noalloc with its device address, looked up on that call's
 *     first use of the device).
 *   - Except bitnet_pack_weights (host memory), every pointer is device memory
 *     and every call is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns without waiting.  Faults during execution surface at
 *     the caller's next synchronisation, as for any stream-ordered work.
 *   - M == 0 or N == 0 is a successful no-op.  Otherwise K must satisfy
 *     0 < K <= BITNET_MAX_K and K % 4 == 0 (BITNET_ERR_SHAPE if not).  The
 *     bound keeps |acc| <= 127 * K below 2^24 so the epilogue's int -> fp32
 *     conversion is exact.
 *   - Any shape in range is correct.  The fast kernels additionally want
 *     K % 64 == 0 and 16-byte aligned base pointers; other shapes take
 *     slower, plain kernels with the same results.
 *   - Calls on distinct output buffers are independent and may overlap on
 *     different streams.
 */
#ifndef BITNET_H
#define BITNET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITNET_MAX_K 131072
/* bitnet_gemv_fused takes M in [0, BITNET_FUSED_MAX_M]; bitnet_linear sends
 * M <= BITNET_FUSED_MAX_M to the fused path and larger M to quantise + GEMM. */
#define BITNET_FUSED_MAX_M 15

typedef enum bitnet_status {
    BITNET_OK = 0,
    BITNET_ERR_NULL = 1,      /* a required pointer is NULL                        */
    BITNET_ERR_SHAPE = 2,     /* negative size, K <= 0, K % 4 != 0, K > MAX_K,
                                 or M > BITNET_FUSED_MAX_M for the fused call       */
    BITNET_ERR_VALUE = 3,     /* a weight outside {-1, 0, +1} given to the packer   */
    BITNET_ERR_WORKSPACE = 4, /* workspace smaller than bitnet_linear_workspace_bytes */
    BITNET_ERR_DEVICE = 5,    /* current device is not gfx950, or no device         */
    BITNET_ERR_LAUNCH = 6,    /* the HIP runtime rejected a kernel launch           */
    BITNET_ERR_TOO_LARGE = 7  /* bitnet_linear_noalloc: the workspace this call needs
                                 exceeds BITNET_NOALLOC_SCRATCH_BYTES               */
} bitnet_status;

/* A hipStream_t, kept opaque so that this header needs no HIP headers. */
typedef void* bitnet_stream_t;

/*
 * Pack ternary weights, 2 bits each, 4 per byte (pack_weights of bitnet-cpu):
 * code = w + 2 (-1 -> 1, 0 -> 2, +1 -> 3) and
 *   w_packed[n][j] = code(w[n][4j]) | code(w[n][4j+1]) << 2
 *                  | code(w[n][4j+2]) << 4 | code(w[n][4j+3]) << 6.
 * HOST memory: w is int8 [N][K], w_packed is uint8 [N][K/4] (written).
 * Errors: NULL pointers (if N*K > 0), N < 0, K < 0, K % 4 != 0 -> SHAPE;
 * a value outside {-1,0,1} -> VALUE (w_packed contents are then unspecified).
 * Runs on the calling thread; no device is touched.
 */
bitnet_status bitnet_pack_weights(uint8_t* w_packed, const int8_t* w, int64_t N, int64_t K);

/*
 * Per-token absmax INT8 quantisation (quantize_activation of bitnet-cpu), in
 * fp32 on the widened bf16 input, for each row m:
 *   a = max(max_k |x[m][k]|, 1e-5f);   s = a / 127.0f  (IEEE fp32 division)
 *   x_int8[m][k] = clamp(round_half_even(x[m][k] / s), -127, 127)
 *   scale_act[m] = bf16_round_nearest_even(s)
 * x: bf16 [M][K] (read); x_int8: int8 [M][K] (written); scale_act: bf16 [M]
 * (written).  Device pointers, enqueued on stream.
 */
bitnet_status bitnet_quantize_act(int8_t* x_int8, uint16_t* scale_act, const uint16_t* x, int64_t M, int64_t K,
                                  bitnet_stream_t stream);

/*
 * Ternary x int8 matmul with the scale epilogue (bitnet_gemm of bitnet-cpu):
 *   acc[m][n] = sum_k w[n][k] * x_int8[m][k]            (exact, int32)
 *   out[m][n] = bf16_rne( fp32( (float)acc * fp32( (float)scale_act[m] * (float)scale_wt[n] ) ) )
 * where w[n][k] = code - 2 decoded from w_packed.  out: bf16 [M][N] (written);
 * x_int8: int8 [M][K]; w_packed: uint8 [N][K/4]; scale_act: bf16 [M];
 * scale_wt: bf16 [N].  Device pointers, enqueued on stream.  Any M >= 0.
 */
bitnet_status bitnet_gemm(uint16_t* out, const int8_t* x_int8, const uint8_t* w_packed, const uint16_t* scale_act,
                          const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K, bitnet_stream_t stream);

/*
 * Fused quantise + ternary GEMV for the decode case (bitnet_gemv_fused of
 * bitnet-cpu; the fused decode path of the bitnet-tc request).  Computes, for
 * 0 <= M <= BITNET_FUSED_MAX_M, exactly the composition
 *   bitnet_quantize_act(x) followed by bitnet_gemm,
 * bit for bit, without writing the int8 activations anywhere (every workgroup
 * quantises the rows it needs: a streaming dot4 kernel for M <= 4, int8 MFMA
 * from M = 5 when K % 128 == 0 and x, w are 16-byte aligned).
 * out: bf16 [M][N] (written); x: bf16 [M][K]; w_packed: uint8 [N][K/4];
 * scale_wt: bf16 [N].  Device pointers, enqueued on stream.
 * Errors: M > BITNET_FUSED_MAX_M -> SHAPE.
 */
bitnet_status bitnet_gemv_fused(uint16_t* out, const uint16_t* x, const uint8_t* w_packed, const uint16_t* scale_wt,
                                int64_t M, int64_t N, int64_t K, bitnet_stream_t stream);

/*
 * Device workspace (bytes) that bitnet_linear needs for an [M][K] input:
 * 0 when it takes the fused GEMV (M <= 2, or M <= 4 with K <= 8192), else
 * room for x_int8 [M][K] and scale_act [M] (each rounded up to 256 bytes).
 * Returns 0 for invalid sizes.
 */
size_t bitnet_linear_workspace_bytes(int64_t M, int64_t K);

/*
 * One-shot BitLinear forward (bitnet_linear of bitnet-cpu): dispatches on M.
 * bitnet-cpu sends M < 16 to its fused GEMV; here both paths give identical
 * bits, so the choice is made for speed: bitnet_gemv_fused for M <= 2 (and for
 * M <= 4 when K <= 8192), its matrix-unit kernel for 5 <= M <= 8 when
 * M * K <= 20480 and N <= 65536 (16-byte aligned x and w, K % 128 == 0; the
 * workspace is then required but unused), otherwise bitnet_quantize_act into
 * the workspace, then bitnet_gemm (one quantisation pass is cheaper than the
 * fused kernels' per-workgroup quantisation once there are more rows).
 * out: bf16 [M][N]; x: bf16 [M][K]; w_packed: uint8 [N][K/4];
 * scale_wt: bf16 [N]; workspace: device memory of workspace_bytes bytes, 256-byte
 * aligned, used as scratch (may be NULL when bitnet_linear_workspace_bytes is 0).
 * Errors: workspace_bytes too small -> WORKSPACE.
 */
bitnet_status bitnet_linear(uint16_t* out, const uint16_t* x, const uint8_t* w_packed, const uint16_t* scale_wt,
                            int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                            bitnet_stream_t stream);

/* Size of the per-device static scratch of bitnet_linear_noalloc (32 MiB). */
#define BITNET_NOALLOC_SCRATCH_BYTES (32 << 20)

/*
 * bitnet_linear for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, dispatch and bits as bitnet_linear, with the
 * workspace (x_int8 [M][K] and scale_act [M]) held in a static array of
 * BITNET_NOALLOC_SCRATCH_BYTES bytes that the library keeps on each device
 * until the process ends, instead of a caller buffer.  No call allocates or
 * frees memory (no hipMalloc, hipFree or allocating library routine); the
 * device address of the array is looked up on the first call on each device.
 * out: bf16 [M][N] (written); x: bf16 [M][K]; w_packed: uint8 [N][K/4];
 * scale_wt: bf16 [N].  Device pointers, enqueued on stream.
 * Every call on one device shares that device's array and leaves its contents
 * behind; the quantiser writes every byte the GEMM reads before it reads it, so
 * no clearing is needed, but calls that overlap on one device (other streams,
 * other threads) race and must be serialised by the caller.
 * Errors: bitnet_linear_workspace_bytes(M, K) > BITNET_NOALLOC_SCRATCH_BYTES
 * -> TOO_LARGE (e.g. M * K above about 33.5 million); others as bitnet_linear.
 */
bitnet_status bitnet_linear_noalloc(uint16_t* out, const uint16_t* x, const uint8_t* w_packed,
                                    const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K,
                                    bitnet_stream_t stream);

/* Activation element types accepted by bitnet_linear_ex. */
#define BITNET_DTYPE_BF16 0
#define BITNET_DTYPE_F32 1

/*
 * Per-token absmax INT8 quantisation of f32 activations (quantize_activation
 * of bitnet-cpu takes x in bf16 or f32): the formula of bitnet_quantize_act
 * applied to the f32 values themselves, with no rounding to bf16 first:
 *   a = max(max_k |x[m][k]|, 1e-5f);   s = a / 127.0f  (IEEE fp32 division)
 *   x_int8[m][k] = clamp(round_half_even(x[m][k] / s), -127, 127)
 *   scale_act[m] = bf16_round_nearest_even(s)
 * x: f32 [M][K]; x_int8: int8 [M][K] (written); scale_act: bf16 [M] (written).
 * Device pointers, enqueued on stream.  NaN/Inf inputs are outside the contract.
 */
bitnet_status bitnet_quantize_act_f32(int8_t* x_int8, uint16_t* scale_act, const float* x, int64_t M, int64_t K,
                                      bitnet_stream_t stream);

/*
 * Device workspace (bytes) that bitnet_linear_ex needs: for bf16 activations
 * the same as bitnet_linear_workspace_bytes; for f32 activations room for
 * x_int8 [M][K] and scale_act [M] at every M (required even when the call
 * takes the one-launch path below and leaves it untouched).  Returns 0 for
 * invalid sizes or dtypes.
 */
size_t bitnet_linear_ex_workspace_bytes(int64_t M, int64_t K, int x_dtype);

/*
 * BitLinear forward with the two options of bitnet-cpu's API: f32 or bf16
 * activations (bitnet_linear and quantize_activation accept both) and an
 * optional bias (class BitLinear adds its bf16 bias to the bf16 result).
 *   y = bitnet_linear(x)   (for f32 x: bitnet_quantize_act_f32, then bitnet_gemm)
 *   out[m][n] = bias ? bf16_rne( fp32(y[m][n]) + fp32(bias[n]) ) : y[m][n]
 * Where bitnet_linear takes the fused GEMV (small M) and x and w_packed are
 * 16-byte aligned with K % 64 == 0 and M <= 4, the whole call is one kernel:
 * either activation type quantised in the GEMV's prologue, the bias added in
 * its epilogue, with the same bits as the separate steps.
 * out: bf16 [M][N] (written); x: [M][K] of x_dtype (BITNET_DTYPE_BF16 or
 * BITNET_DTYPE_F32); w_packed: uint8 [N][K/4]; scale_wt: bf16 [N]; bias: bf16
 * [N] or NULL; workspace: bitnet_linear_ex_workspace_bytes(M, K, x_dtype)
 * bytes of device memory (256-byte aligned).  Device pointers, enqueued on stream.
 * Errors: unknown x_dtype -> VALUE; workspace too small -> WORKSPACE.
 */
bitnet_status bitnet_linear_ex(uint16_t* out, const void* x, int x_dtype, const uint8_t* w_packed,
                               const uint16_t* scale_wt, const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                               void* workspace, size_t workspace_bytes, bitnet_stream_t stream);

/*
 * RMSNorm, then the per-token quantisation of the normalised rows
 * (activation_norm_quant of "kyegomez/BitNet issue #77": F.rms_norm over the
 * last dimension before the int8 quantisation, which that page notes can be
 * one fused kernel; bitnet-cpu's BitLinearKernel likewise runs its rms_norm
 * module before bitnet_linear).  Per row m, in fp32 as torch's rms_norm
 * computes on bf16 input:
 *   mean = fp32( sum_k x[m][k]^2 / K )      (exact squares summed in double)
 *   r    = fp32( 1 / fp32( sqrt( fp32(mean + eps) ) ) )   (IEEE sqrt, division)
 *   xn[m][k] = bf16_round_nearest_even( fp32( fp32(x[m][k] * r) * gain[k] ) )
 * (no gain multiply when gain is NULL), then bitnet_quantize_act on xn.
 * The double sum's order is the library's; a different order could move the
 * fp32 mean by one step only where the double mean lies within about
 * K * 2^-52 (relative) of an fp32 rounding boundary.
 * x: bf16 [M][K]; gain: bf16 [K] or NULL; eps: finite, >= 0 (torch's default is
 * the fp32 epsilon 2^-23); x_int8: int8 [M][K] (written); scale_act: bf16 [M]
 * (written); x_norm: bf16 [M][K] (written when not NULL).  Device pointers,
 * enqueued on stream.  Errors: eps negative or not finite -> VALUE.
 */
bitnet_status bitnet_rmsnorm_quantize(int8_t* x_int8, uint16_t* scale_act, uint16_t* x_norm, const uint16_t* x,
                                      const uint16_t* gain, float eps, int64_t M, int64_t K, bitnet_stream_t stream);

/*
 * Device workspace (bytes) that bitnet_linear_rms needs: room for x_int8
 * [M][K] and scale_act [M] (each rounded up to 256 bytes) at every M.
 * Returns 0 for invalid sizes.
 */
size_t bitnet_linear_rms_workspace_bytes(int64_t M, int64_t K);

/*
 * BitLinear forward preceded by RMSNorm (the rms_norm step of bitnet-cpu's
 * BitLinearKernel, fused as "kyegomez/BitNet issue #77" suggests):
 *   out = bitnet_linear( rms_norm(x) )  with rms_norm as in
 *   bitnet_rmsnorm_quantize.
 * For 1 <= M <= 4 (K % 64 == 0, 16-byte aligned x, w_packed and gain) the
 * normalisation runs in the prologue of the fused decode GEMV and the
 * workspace is not touched; otherwise bitnet_rmsnorm_quantize into the
 * workspace, then bitnet_gemm.  The two paths add the squares in different
 * orders; they give the same bits except in the rare rows whose fp32 mean is
 * ambiguous in the sense of bitnet_rmsnorm_quantize.
 * out: bf16 [M][N]; x: bf16 [M][K]; gain: bf16 [K] or NULL; w_packed: uint8
 * [N][K/4]; scale_wt: bf16 [N]; workspace: device memory of at least
 * bitnet_linear_rms_workspace_bytes(M, K) bytes, 256-byte aligned (always
 * required).  Errors: workspace too small -> WORKSPACE; eps negative or not
 * finite -> VALUE.
 */
bitnet_status bitnet_linear_rms(uint16_t* out, const uint16_t* x, const uint16_t* gain, float eps,
                                const uint8_t* w_packed, const uint16_t* scale_wt, int64_t M, int64_t N, int64_t K,
                                void* workspace, size_t workspace_bytes, bitnet_stream_t stream);

/* Largest activation row count bitnet_w8a16_gemv takes (decode batches). */
#define BITNET_W8A16_MAX_M 64

/*
 * INT8 weight-only decode matmul (int8_matmul of "CoolDip00/tiny-llm,
 * src/tinyllm/kernels/int8_gemv.py"): each int8 weight is read once, converted
 * exactly to bf16 in registers, multiplied with bf16 activations and summed in
 * fp32; the per-row scale is applied to the fp32 sum:
 *   y[m][n] = scale[n] * sum_k x[m][k] * q[n][k].
 * y: fp32 [M][N] (written); x: bf16 [M][K]; q: int8 [N][K]; scale: fp32 [N].
 * 0 <= M <= BITNET_W8A16_MAX_M, 0 < K <= BITNET_MAX_K (any K; K % 64 == 0 and
 * 16-byte aligned x and q take the fast kernel).  The fp32 summation order is
 * the library's own (fixed for a given shape, so results are deterministic);
 * it differs from an exact sum by at most K * 2^-24 * sum_k |x * q| * |scale|
 * plus the final rounding.  Device pointers, enqueued on stream.
 * Errors: M > BITNET_W8A16_MAX_M, K <= 0 or K > BITNET_MAX_K -> SHAPE.
 */
bitnet_status bitnet_w8a16_gemv(float* y, const uint16_t* x, const int8_t* q, const float* scale, int64_t M,
                                int64_t N, int64_t K, bitnet_stream_t stream);

/*
 * Debug: the raw int32 accumulators of the batched path,
 *   acc[m][n] = sum_k w[n][k] * x_int8[m][k],
 * computed by the same matrix-core kernel as bitnet_gemm (its int32 output
 * variant).  acc: int32 [M][N] (written).  Device pointers, enqueued on stream.
 */
bitnet_status bitnet_gemm_i32(int32_t* acc, const int8_t* x_int8, const uint8_t* w_packed, int64_t M, int64_t N,
                              int64_t K, bitnet_stream_t stream);

/*
 * Debug: the fused decode path's intermediate results, computed by the same
 * fused kernel as bitnet_gemv_fused (its int32 output variant):
 * acc: int32 [M][N], the exact sum_k w[n][k] * q[m][k] of the in-kernel
 * quantised rows q; scale_act: bf16 [M], the in-kernel scales.
 * 0 <= M <= BITNET_FUSED_MAX_M.  Device pointers, enqueued on stream.
 */
bitnet_status bitnet_gemv_fused_i32(int32_t* acc, uint16_t* scale_act, const uint16_t* x, const uint8_t* w_packed,
                                    int64_t M, int64_t N, int64_t K, bitnet_stream_t stream);

/*
 * Debug: the scale epilogue on its own,
 *   out[m][n] = bf16_rne( fp32( (float)acc[m][n] * fp32( (float)scale_act[m] * (float)scale_wt[n] ) ) ).
 * out: bf16 [M][N] (written); acc: int32 [M][N]; scale_act: bf16 [M];
 * scale_wt: bf16 [N].  Device pointers, enqueued on stream.  No K involved.
 */
bitnet_status bitnet_scale_epilogue(uint16_t* out, const int32_t* acc, const uint16_t* scale_act,
                                    const uint16_t* scale_wt, int64_t M, int64_t N, bitnet_stream_t stream);

/* A static, human-readable name for a status code. */
const char* bitnet_status_string(bitnet_status status);

/* Library version: major * 10000 + minor * 100 + patch. */
int bitnet_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_H */
