"""Parity of the HIP path (through the C ABI) with the CPU oracle, element by element.

Bar: int8 activations, bf16 scales and int32 accumulators bit-exact; bf16
outputs within 1 bf16 ulp (ordered-integer distance, +0 == -0), and in fact
expected bit-exact because both sides fix the same fp32 operation order.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_int8_gemm_amd as tg

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


# ----------------------------------------------------------------------------- helpers

def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bf16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def ulp_distance(a, b):
    a = a.astype(np.int32)
    b = b.astype(np.int32)
    oa = np.where(a & 0x8000, -(a & 0x7FFF), a & 0x7FFF)
    ob = np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(oa - ob)


def assert_bf16_parity(got, want, what):
    d = ulp_distance(got, want)
    assert d.max(initial=0) <= 1, f"{what}: max ulp {d.max()} at {np.unravel_index(np.argmax(d), d.shape)}"
    assert np.array_equal(got, want), f"{what}: {int((got != want).sum())} outputs differ by 1 ulp"


def misaligned(t):
    """A contiguous copy of t whose data pointer is 2 bytes past a 16-byte boundary."""
    flat = t.reshape(-1)
    esz = flat.element_size()
    pad = max(1, 2 // esz)
    buf = torch.empty(flat.numel() + 16, dtype=t.dtype, device=t.device)
    view = buf[pad:pad + flat.numel()]
    view.copy_(flat)
    assert view.data_ptr() % 16 != 0
    return view.view(t.shape)


def lib_pack(W):
    """Pack with the library's host packer (the chain the kernels see in use) and
    require the oracle's bytes: the kernels then run on library-packed weights."""
    P = tg.pack_weights(torch.from_numpy(np.ascontiguousarray(W))).numpy()
    assert np.array_equal(P, oracle.pack(W)), "bitnet_pack_weights differs from the oracle's pack"
    return P


def problem(M, N, K, seed, outliers=0.0, row_scales=False):
    x = synth.activations_bf16(M, K, seed, outlier_frac=outliers)
    W = synth.ternary_weights(N, K, seed + 1)
    P = lib_pack(W)
    sw = synth.row_scales_bf16(N, seed + 2) if row_scales else synth.weight_scale_bf16(N, K, seed + 2)
    return x, W, P, sw


# ----------------------------------------------------------------------------- quantisation

QUANT_SHAPES = [(4, 256), (1, 4), (3, 12), (7, 100), (16, 2560), (33, 4096), (5, 6912), (2, 131072), (130, 64),
                # many rows (one workgroup each)
                (2049, 4096), (2051, 6912), (2053, 520),
                # each register depth of the workgroup-per-row kernel, full and ragged last chunks, and the
                # first lengths past it (two-pass and plain kernels)
                (1, 2048), (1, 2056), (3, 8192), (9, 12000), (3, 16384), (5, 16400), (2, 16392)]


@pytest.mark.parametrize("M,K", QUANT_SHAPES)
def test_quantize_parity(M, K):
    x = synth.activations_bf16(M, K, seed=1000 + M + K, outlier_frac=0.01 if K >= 100 else 0.0)
    if M > 2:
        x[1, :] = 0                          # all-zero row: eps floor
        x[2, : K // 2] = 0x3000              # a run of tiny values (2^-31)
    q_ref, s_ref = oracle.quantize(x)
    q, s = tg.quantize_activation(dev_bf16(x))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(host_bf16(s), s_ref)


def test_quantize_golden_vectors_on_gpu():
    from conftest import read_golden
    for r in read_golden("quantize_vectors.txt"):
        vals = [float(t) for t in r["x"]]
        K = (len(vals) + 3) // 4 * 4                 # pad with zeros: changes neither absmax nor q
        xb = torch.tensor(vals + [0.0] * (K - len(vals)), dtype=torch.float32).to(torch.bfloat16)
        q, s = tg.quantize_activation(xb.view(1, K).to(DEV))
        assert q.cpu().numpy()[0, :len(vals)].tolist() == [int(t) for t in r["q"]]
        assert int(host_bf16(s)[0]) == int(r["scale_bf16"][0], 16)


def exhaustive_bf16_rows(seed=1234, rows=45):
    """Rows whose absmax is A and which hold every bf16 value v with A/512 <= |v| <= A (both
    signs): every bf16 input the quantiser can see at that scale outside the band that
    rounds to 0.  A runs over powers of two, 127, values near the 1e-5 floor and random
    bf16 values from 2^-20 to 2^100; rows are zero-padded to one length (K % 64 == 0)."""
    g = synth.rng(seed)
    special = [0x3F80, 0x42FE, 0x3727, 0x3728, 0x3729, 0x3000, 0x7F7F, 0x0080]    # 1, 127, ~1e-5, 2^-31, max, min normal
    randoms = [int(b) for b in g.integers(0x3580, 0x71FF, size=rows - len(special))]
    out = []
    allv = np.arange(0x0080, 0x7F80, dtype=np.uint32)                 # positive normal bf16 bit patterns
    vals = (allv << 16).view(np.float32)
    for A_bits in special + randoms:
        A = float(np.array([A_bits << 16], dtype=np.uint32).view(np.float32)[0])
        keep = allv[(vals <= A) & (vals >= A / 512)]
        row = np.concatenate([np.array([A_bits], dtype=np.uint32), keep, keep | 0x8000]).astype(np.uint16)
        g.shuffle(row)
        out.append(row)
    K = max(len(r) for r in out)
    K = (K + 63) // 64 * 64
    x = np.zeros((len(out), K), dtype=np.uint16)
    for i, r in enumerate(out):
        x[i, :len(r)] = r
    return x


def test_quantize_exhaustive_bf16():
    """Every bf16 value at many scales through the standalone quantiser (the
    workgroup-per-row kernel), bit-exact against the oracle."""
    x = exhaustive_bf16_rows()
    q_ref, s_ref = oracle.quantize(x)
    q, s = tg.quantize_activation(dev_bf16(x))
    assert np.array_equal(host_bf16(s), s_ref)
    bad = np.argwhere(q.cpu().numpy() != q_ref)
    assert bad.size == 0, f"{len(bad)} int8 values differ, first at {tuple(bad[0])}"


def test_gemv_prologue_exhaustive_bf16():
    """The same rows quantised in the fused decode GEMV's prologue: with one-hot
    weights (w[n][k] = 1 iff k == n) the int32 outputs are the int8 activations."""
    x = exhaustive_bf16_rows(seed=4321, rows=30)
    M, K = x.shape
    q_ref, s_ref = oracle.quantize(x)
    W = np.zeros((K, K), dtype=np.int8)
    np.fill_diagonal(W, 1)
    Pd = dev(lib_pack(W))
    # 1, 2 and 4 rows take the streaming kernel; 8 and 15 rows of this length (K % 128 != 0) its
    # K-chunked variant
    assert K % 128 != 0
    for m0, m1 in ((0, 1), (1, 3), (3, 7), (7, 15), (15, 30)):
        xs = x[m0:m1]
        acc, sa = tg.bitnet_gemv_fused_i32(dev_bf16(xs), Pd)
        assert np.array_equal(host_bf16(sa), s_ref[m0:m1])
        assert np.array_equal(acc.cpu().numpy(), q_ref[m0:m1].astype(np.int32)), f"rows {m0}..{m1}"
    # zero-padded to K % 128 == 0, 5 to 15 rows take the matrix-unit kernel
    K2 = (K + 127) // 128 * 128
    x2 = np.zeros((M, K2), dtype=np.uint16)
    x2[:, :K] = x
    W2 = np.zeros((K2, K2), dtype=np.int8)
    np.fill_diagonal(W2, 1)
    Pd2 = dev(lib_pack(W2))
    for m0, m1 in ((0, 5), (5, 13), (13, 28), (28, 30)):
        acc, sa = tg.bitnet_gemv_fused_i32(dev_bf16(x2[m0:m1]), Pd2)
        assert np.array_equal(host_bf16(sa), s_ref[m0:m1])
        assert np.array_equal(acc.cpu().numpy()[:, :K], q_ref[m0:m1].astype(np.int32)), f"rows {m0}..{m1}"
        assert not acc.cpu().numpy()[:, K:].any()


def test_quantize_f32_near_ties():
    """f32 activations placed on and next to the values whose quotient by s is a
    half-integer (where a wrong last bit of x / s flips the rounded int8)."""
    g = synth.rng(99)
    M, K = 40, 1024
    x = np.zeros((M, K), dtype=np.float32)
    for m in range(M):
        A = np.float32(10.0 ** g.uniform(-4, 4))
        s = np.float32(A / np.float32(127.0))
        k = g.integers(0, 127, size=K - 1)
        base = ((k + 0.5) * np.float64(s)).astype(np.float32) * np.where(g.random(K - 1) < 0.5, 1, -1).astype(np.float32)
        d = g.integers(-2, 3, size=K - 1).astype(np.int32)
        x[m, 1:] = (base.view(np.int32) + d).view(np.float32)
        x[m, 0] = A
        x[m] = np.clip(x[m], -A, A)
    q_ref, s_ref = oracle.quantize_f32(x)
    q, s = tg.quantize_activation(dev_f32(x))
    assert np.array_equal(host_bf16(s), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_quantize_misaligned_plain_path():
    x = synth.activations_bf16(6, 96, seed=7)
    q_ref, s_ref = oracle.quantize(x)
    xd = misaligned(dev_bf16(x))
    q = misaligned(torch.zeros((6, 96), dtype=torch.int8, device=DEV))
    s = torch.empty((6,), dtype=torch.bfloat16, device=DEV)
    tg.quantize_activation(xd, out=q, scale=s)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(host_bf16(s), s_ref)


# ----------------------------------------------------------------------------- int32 GEMM

GEMM_SHAPES = [
    (1, 1, 64), (4, 128, 256), (17, 33, 64), (128, 128, 128), (129, 130, 192), (300, 257, 320),
    (16, 4096, 4096), (64, 512, 2560), (255, 129, 6912), (8, 64, 68), (5, 7, 100), (3, 3, 4),
    # split-K path for few rows: every configuration, ragged N, K of 4..9 chunks of 128
    (9, 100, 1152), (20, 777, 1024), (100, 1000, 640), (130, 70, 512), (1, 33, 4096), (64, 31, 512),
    # LDS-staged split-K kernel (K % 256 == 0): every configuration, wide and ragged N, ragged M
    (32, 8200, 2048), (33, 300, 2048), (64, 9000, 1024), (100, 8192, 2048), (128, 500, 2048),
    (200, 9001, 2048), (250, 300, 1024), (5, 4096, 768), (77, 2000, 1280),
    # the same kernel staging only 4, 8 or 16 activation rows (few rows), one and two column tiles
    (3, 9000, 2048), (7, 9001, 2048), (2, 300, 1024), (6, 333, 2048), (13, 300, 2048), (16, 1000, 1024),
    # mid-sized M (M * N >= 5 * 2^18 with few 128 x 256 tiles): 128 x 256, 128 x 128 and 64 x 128
    # blocks (the LDS-staged shape (200, 9001, 2048) above takes 64 x 128 blocks too); (200, 4000, 2048)
    # keeps the split-K kernel for M > 128 and K >= 2048 covered
    (513, 10000, 256), (300, 13000, 384), (1000, 2200, 512), (200, 4000, 2048),
    # weights straight into the LDS ring, ragged M and N: 128 x 128 blocks over 10 stages (the ring
    # wraps); four-wave 128 x 256 blocks (more than 256 of them, too few 128 x 512 blocks to fill their
    # rounds) over 5 stages and over a single stage; 128 x 512 blocks with a single stage
    (700, 4000, 1280), (1100, 8200, 640), (1030, 32770, 128), (1030, 65000, 128),
    # few rows, very many columns: 32- and 64-row blocks
    (5, 66000, 1024), (32, 65600, 512), (40, 70000, 512), (64, 65537, 256),
    # the eight-wave 128 x 256 block (one round of at most 256 blocks): 2, 3, 5 and 9 stages on
    # ragged M and N
    (300, 500, 256), (250, 300, 384), (2000, 3900, 640), (1930, 3850, 1152),
    # the same block on exactly 256 tiles with ragged edges: 6, 8 and 10 stages
    (1000, 8000, 768), (2000, 3900, 1024), (1930, 3850, 1280),
]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_i32_parity(M, N, K):
    q = synth.random_int8((M, K), seed=2000 + M + N + K)
    W = synth.ternary_weights(N, K, seed=2100 + M + N + K)
    P = lib_pack(W)
    acc_ref = oracle.gemm_i32(q, P)
    acc = tg.bitnet_gemm_i32(dev(q), dev(P))
    assert np.array_equal(acc.cpu().numpy(), acc_ref)


def test_gemm_i32_random_bytes_include_code_zero():
    M, N, K = 70, 96, 512
    q = synth.random_int8((M, K), seed=31)
    P = synth.random_bytes(N * K // 4, seed=32).reshape(N, K // 4)   # code 0 decodes to -2
    assert np.array_equal(tg.bitnet_gemm_i32(dev(q), dev(P)).cpu().numpy(), oracle.gemm_i32(q, P))


def test_gemm_i32_extremes():
    M, N, K = 32, 64, 4096
    q = np.full((M, K), 127, dtype=np.int8)
    q[1::2] = -127
    W = np.ones((N, K), dtype=np.int8)
    W[::3] = -1
    P = lib_pack(W)
    assert np.array_equal(tg.bitnet_gemm_i32(dev(q), dev(P)).cpu().numpy(), oracle.gemm_i32(q, P))


def test_gemm_i32_misaligned_plain_path():
    M, N, K = 9, 20, 128
    q = synth.random_int8((M, K), seed=41)
    W = synth.ternary_weights(N, K, seed=42)
    P = lib_pack(W)
    acc = tg.bitnet_gemm_i32(misaligned(dev(q)), dev(P))
    assert np.array_equal(acc.cpu().numpy(), oracle.gemm_i32(q, P))


# ----------------------------------------------------------------------------- bf16 GEMM

@pytest.mark.parametrize("M,N,K", [(4, 128, 256), (16, 4096, 4096), (200, 300, 1024), (33, 65, 68),
                                   (513, 10000, 256), (300, 13000, 384), (1000, 2200, 512), (700, 4000, 1280),
                                   (1100, 8200, 640), (16, 128256, 512), (40, 70000, 512),
                                   # ragged M and N: four-wave 128 x 256 blocks over one stage, the 128 x 512
                                   # block tile (its rounds of 256 blocks at least 85 % full) over two stages;
                                   # the same two block shapes over four and six stages, more blocks than
                                   # are resident at once, edge tiles in M and N
                                   (1030, 32770, 128), (600, 70000, 256), (1500, 11000, 512), (390, 55700, 768),
                                   # the eight-wave 128 x 256 block: 2 and 9 stages, ragged M and N
                                   (300, 500, 256), (1930, 3850, 1152),
                                   # exactly 256 tiles with ragged edges: 6 and 10 stages
                                   (1000, 8000, 768), (1930, 3850, 1280)])
def test_gemm_bf16_parity(M, N, K):
    x, W, P, _ = problem(M, N, K, seed=3000 + M)
    sw = synth.row_scales_bf16(N, seed=3100 + M)
    q, sa = oracle.quantize(x)
    out_ref = oracle.epilogue(oracle.gemm_i32(q, P), sa, sw)
    out = tg.bitnet_gemm(dev(q), dev(P), dev_bf16(sa), dev_bf16(sw))
    assert_bf16_parity(host_bf16(out), out_ref, f"gemm {M}x{N}x{K}")


# ----------------------------------------------------------------------------- fused GEMV

GEMV_SHAPES = [
    (1, 1, 64), (1, 7, 256), (4, 128, 256), (2, 1000, 512), (3, 129, 576), (5, 64, 2560), (8, 3840, 2560),
    (9, 100, 6912), (15, 256, 4096), (1, 2560, 6912), (16 - 1, 33, 40960), (1, 300, 68), (7, 50, 100),
    # K split across the waves of a workgroup (one row, few units, long rows): 4 parts, 4 parts
    # with a partial last step, 2 parts with a partial last step; two rows are never split
    (1, 1000, 16384), (1, 300, 8256), (1, 520, 7232), (2, 520, 7232),
]


@pytest.mark.parametrize("M,N,K", GEMV_SHAPES)
def test_gemv_fused_parity(M, N, K):
    x, W, P, sw = problem(M, N, K, seed=4000 + M * 7 + N + K, row_scales=True)
    ref = oracle.linear(x, P, sw)
    xd, Pd = dev_bf16(x), dev(P)
    out = tg.bitnet_gemv_fused(xd, Pd, dev_bf16(sw))
    acc, sa = tg.bitnet_gemv_fused_i32(xd, Pd)
    assert np.array_equal(host_bf16(sa), ref["scale_act"])
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    assert_bf16_parity(host_bf16(out), ref["out"], f"gemv {M}x{N}x{K}")


# The matrix-unit fused kernel (five rows and more, K % 128 == 0): every number of K parts
# per column tile (1, 2, 4, 8, 16 by the launch rule), K in one chunk, two chunks, ten chunks
# and a last chunk of a single stage (K parts with no stage in it), ragged N, and M = 5 ... 15.
GEMV_MFMA_SHAPES = [
    (13, 66001, 256),    # 1 part (2063 tiles)
    (6, 40001, 512),     # 2 parts
    (6, 20001, 512),     # 4 parts
    (14, 13824, 2560),   # 8 parts
    (16 - 1, 3000, 2048),  # 16 parts, one chunk
    (9, 100, 11008),     # 16 parts, two chunks
    (7, 200, 8320),      # 16 parts, a last chunk of one stage
    (12, 40, 40960),     # five chunks
    (8, 3840, 2560), (5, 2560, 6912), (11, 10000, 1024),
]


@pytest.mark.parametrize("M,N,K", GEMV_MFMA_SHAPES)
def test_gemv_fused_mfma_parity(M, N, K):
    x, W, P, sw = problem(M, N, K, seed=4400 + M * 3 + N + K, outliers=0.01, row_scales=True)
    x[M // 2] = 0  # an all-zero row: the 1e-5 absmax floor
    ref = oracle.linear(x, P, sw)
    xd, Pd = dev_bf16(x), dev(P)
    out = tg.bitnet_gemv_fused(xd, Pd, dev_bf16(sw))
    acc, sa = tg.bitnet_gemv_fused_i32(xd, Pd)
    assert np.array_equal(host_bf16(sa), ref["scale_act"])
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    assert_bf16_parity(host_bf16(out), ref["out"], f"gemv mfma {M}x{N}x{K}")
    q, sa2 = tg.quantize_activation(xd)   # same bits as the split path
    assert np.array_equal(host_bf16(tg.bitnet_gemm(q, Pd, sa2, dev_bf16(sw))), host_bf16(out))


def test_gemv_fused_misaligned_plain_path():
    M, N, K = 3, 40, 256
    x, W, P, sw = problem(M, N, K, seed=51)
    ref = oracle.linear(x, P, sw)
    out = tg.bitnet_gemv_fused(misaligned(dev_bf16(x)), dev(P), dev_bf16(sw))
    assert_bf16_parity(host_bf16(out), ref["out"], "gemv misaligned")


# ----------------------------------------------------------------------------- dispatch

@pytest.mark.parametrize("M", list(range(1, 18)) + [64])
def test_linear_dispatch_neutral(M):
    N, K = 192, 1024
    x, W, P, sw = problem(M, N, K, seed=5000 + M, outliers=0.01, row_scales=True)
    ref = oracle.linear(x, P, sw)
    out = tg.bitnet_linear(dev_bf16(x), dev(P), dev_bf16(sw))
    assert_bf16_parity(host_bf16(out), ref["out"], f"linear M={M}")
    if M <= tg.FUSED_MAX_M:   # the fused GEMV and the split path give the same bits too
        fused = tg.bitnet_gemv_fused(dev_bf16(x), dev(P), dev_bf16(sw))
        assert np.array_equal(host_bf16(fused), host_bf16(out))
        q, sa = tg.quantize_activation(dev_bf16(x))
        out2 = tg.bitnet_gemm(q, dev(P), sa, dev_bf16(sw))
        assert np.array_equal(host_bf16(out2), host_bf16(out))


# bitnet_linear where the GEMM is the LDS-staged split-K kernel: every configuration of that kernel
# (rows 32 / 64 / 128 / more, one or two column tiles, 4 or >= 8 chunks of 256), ragged M and N, an
# all-zero row (eps floor) and outliers; the result must equal the oracle, and the separately called
# quantise and GEMM entry points, bit for bit.
LINEAR_XQ_SHAPES = [(5, 300, 1024), (16, 2560, 2560), (16, 3840, 2560), (16, 13824, 2560), (16, 2560, 6912),
                    (40, 1000, 2048), (64, 9000, 1024), (100, 3000, 2048), (100, 8192, 2048), (100, 500, 1024),
                    (200, 4000, 2048), (250, 300, 1024), (33, 70, 4096)]


@pytest.mark.parametrize("M,N,K", LINEAR_XQ_SHAPES)
def test_linear_split_k_shapes(M, N, K):
    x, W, P, sw = problem(M, N, K, seed=7000 + M + N, outliers=0.01)
    x[M // 2, :] = 0
    ref = oracle.linear(x, P, sw)
    xd, Pd, swd = dev_bf16(x), dev(P), dev_bf16(sw)
    out = tg.bitnet_linear(xd, Pd, swd)
    assert_bf16_parity(host_bf16(out), ref["out"], f"linear {M}x{N}x{K}")
    q, sa = tg.quantize_activation(xd)
    out2 = tg.bitnet_gemm(q, Pd, sa, swd)
    assert np.array_equal(host_bf16(out2), host_bf16(out))


def test_linear_split_k_misaligned_activations():
    M, N, K = 8, 300, 1024   # a split-K shape, with activations 2 bytes off a 16-byte boundary
    x, W, P, sw = problem(M, N, K, seed=71)
    ref = oracle.linear(x, P, sw)
    out = tg.bitnet_linear(misaligned(dev_bf16(x)), dev(P), dev_bf16(sw))
    assert_bf16_parity(host_bf16(out), ref["out"], "linear misaligned")


def test_linear_leading_dims():
    x, W, P, sw = problem(6, 64, 256, seed=61)
    ref = oracle.linear(x, P, sw)
    out = tg.bitnet_linear(dev_bf16(x).view(2, 3, 256), dev(P), dev_bf16(sw))
    assert out.shape == (2, 3, 64)
    assert np.array_equal(host_bf16(out).reshape(6, 64), ref["out"])


# bitnet_linear captured in a graph (the benchmark's launch mode) on each dispatch path, replayed three
# times with eager work and a synchronisation in between: every replay must rewrite every output with the
# oracle's bits.
GRAPH_LINEAR_SHAPES = [(3, 1000, 1024),     # one-launch fused GEMV (M <= 4)
                       (8, 3840, 2560),     # fused quantise + matrix-unit product
                       (16, 2560, 2560),    # quantise + LDS-staged split-K GEMM
                       (1024, 1536, 1024)]  # quantise + mid-M block tiles


@pytest.mark.parametrize("M,N,K", GRAPH_LINEAR_SHAPES)
def test_linear_graph_replays(M, N, K):
    x, W, P, sw = problem(M, N, K, seed=7700 + M, outliers=0.01)
    ref = oracle.linear(x, P, sw)["out"]
    xd, Pd, swd = dev_bf16(x), dev(P), dev_bf16(sw)
    od = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((max(1, tg.linear_workspace_bytes(M, K)),), dtype=torch.uint8, device=DEV)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        tg.bitnet_linear(xd, Pd, swd, out=od, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(od), ref), f"eager linear {M}x{N}x{K}"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        tg.bitnet_linear(xd, Pd, swd, out=od, workspace=ws)
    for rep in range(3):
        od.fill_(1.0)                                   # a replay must rewrite every output
        ws.fill_(0xA5)                                  # and must not depend on the workspace's old contents
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16(od), ref), f"replay {rep} of linear {M}x{N}x{K}"


# ----------------------------------------------------------------------------- epilogue

@pytest.mark.parametrize("M,N", [(3, 8), (5, 7), (64, 1000)])
def test_scale_epilogue_parity(M, N):
    g = synth.rng(70 + N)
    acc = g.integers(-(1 << 23), 1 << 23, size=(M, N)).astype(np.int32)
    sa = synth.row_scales_bf16(M, seed=71, lo=1e-3, hi=0.1)
    sw = synth.row_scales_bf16(N, seed=72)
    ref = oracle.epilogue(acc, sa, sw)
    out = tg.bitnet_scale_epilogue(dev(acc), dev_bf16(sa), dev_bf16(sw))
    assert_bf16_parity(host_bf16(out), ref, "epilogue")


def test_scale_epilogue_golden_ties():
    from conftest import read_golden
    rows = read_golden("epilogue_cases.txt")
    acc = np.array([[int(r["acc"][0]) for r in rows]], dtype=np.int32)
    for i, r in enumerate(rows):
        sa = np.array([int(r["sa"][0], 16)], dtype=np.uint16)
        sw = np.array([int(r["sw"][0], 16)], dtype=np.uint16)
        out = tg.bitnet_scale_epilogue(dev(acc[:, i:i + 1]), dev_bf16(sa), dev_bf16(sw))
        assert int(host_bf16(out)[0, 0]) == int(r["out"][0], 16), r


# ----------------------------------------------------------------------------- degenerate cases

def test_zero_sizes_are_noops():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    P = torch.zeros((8, 16), dtype=torch.uint8, device=DEV)
    sw = torch.ones((8,), dtype=torch.bfloat16, device=DEV)
    assert tg.bitnet_linear(x, P, sw).shape == (0, 8)
    out = tg.bitnet_linear(torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV),
                           torch.zeros((0, 16), dtype=torch.uint8, device=DEV),
                           torch.ones((0,), dtype=torch.bfloat16, device=DEV))
    assert out.shape == (4, 0)


def test_zero_activation_row_and_constant_weights():
    M, N, K = 4, 48, 512
    x = synth.activations_bf16(M, K, seed=81)
    x[0] = 0
    W = np.ones((N, K), dtype=np.int8)
    W[N // 2:] = -1
    W[N - 1] = 0
    P = lib_pack(W)
    sw = np.full((N,), 0x3F80, dtype=np.uint16)
    ref = oracle.linear(x, P, sw)
    for fn in (lambda: tg.bitnet_gemv_fused(dev_bf16(x), dev(P), dev_bf16(sw)),):
        out = host_bf16(fn())
        assert_bf16_parity(out, ref["out"], "constant W")
        assert np.all(out[0] == 0)                       # zero row -> +0.0 everywhere
    q, sa = tg.quantize_activation(dev_bf16(x))
    assert int(host_bf16(sa)[0]) == 0x33A9


def test_max_k():
    K = tg.MAX_K
    for M in (1, 16):
        x, W, P, sw = problem(M, 24, K, seed=90 + M)
        ref = oracle.linear(x, P, sw)
        out = tg.bitnet_linear(dev_bf16(x), dev(P), dev_bf16(sw))
        assert_bf16_parity(host_bf16(out), ref["out"], f"max K M={M}")


def test_device_errors_raise():
    x = torch.zeros((16, 64), dtype=torch.bfloat16, device=DEV)
    P = torch.zeros((8, 16), dtype=torch.uint8, device=DEV)
    sw = torch.ones((8,), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tg.BitnetError):
        tg.bitnet_gemv_fused(x, P, sw)                   # M = 16 > 15
    with pytest.raises(ValueError):                       # the binding checks the workspace first
        tg.bitnet_linear(x, P, sw, workspace=torch.empty((8,), dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):                       # and the size of a given output
        tg.bitnet_linear(x, P, sw, out=torch.empty((16, 7), dtype=torch.bfloat16, device=DEV))


# ----------------------------------------------------------------------------- f32 activations and bias

def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


F32_QUANT_SHAPES = [(4, 256), (1, 4), (3, 12), (7, 100), (16, 2560), (33, 4096), (5, 6912), (2, 131072), (130, 64),
                    (1, 1024), (1, 1028), (3, 16384), (2, 16388), (2049, 4096),
                    (3, 8192), (2, 8196)]


@pytest.mark.parametrize("M,K", F32_QUANT_SHAPES)
def test_quantize_f32_parity(M, K):
    g = synth.rng(6000 + M + K)
    x = (g.standard_normal((M, K)) * 3.0).astype(np.float32)
    if M > 2:
        x[1, :] = 0.0                          # all-zero row: eps floor
        x[2, : K // 2] = np.float32(2.0 ** -31)
    q_ref, s_ref = oracle.quantize_f32(x)
    q, s = tg.quantize_activation(dev_f32(x))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(host_bf16(s), s_ref)


def test_quantize_f32_golden_vectors_on_gpu():
    from conftest import read_golden
    for r in read_golden("quantize_f32_vectors.txt"):
        x = np.array([int(t, 16) for t in r["x"]], dtype=np.uint32).view(np.float32)
        K = (len(x) + 3) // 4 * 4
        xp = np.zeros((1, K), dtype=np.float32)
        xp[0, :len(x)] = x
        q, s = tg.quantize_activation(dev_f32(xp))
        assert q.cpu().numpy()[0, :len(x)].tolist() == [int(t) for t in r["q"]]
        assert int(host_bf16(s)[0]) == int(r["scale_bf16"][0], 16)


def test_quantize_f32_misaligned_plain_path():
    g = synth.rng(61)
    x = g.standard_normal((5, 96)).astype(np.float32)
    q_ref, s_ref = oracle.quantize_f32(x)
    q = torch.zeros((5, 96), dtype=torch.int8, device=DEV)
    s = torch.empty((5,), dtype=torch.bfloat16, device=DEV)
    tg.quantize_activation(misaligned(dev_f32(x)), out=q, scale=s)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(host_bf16(s), s_ref)


@pytest.mark.parametrize("M,N,K", [(1, 3840, 2560), (5, 300, 1024), (16, 4096, 4096), (64, 1000, 640),
                                   (300, 257, 320), (7, 33, 100),
                                   # M <= 4: f32 quantised in the GEMV's prologue (one to three K parts,
                                   # one step, the LDS limit at 1, 2 and 4 rows, ragged N)
                                   (2, 1000, 4096), (4, 257, 8192), (1, 20000, 2560), (3, 64, 64), (2, 5, 16384),
                                   (1, 700, 32768), (1, 2560, 6912)])
def test_linear_f32_parity(M, N, K):
    g = synth.rng(6100 + M + N + K)
    x = g.standard_normal((M, K)).astype(np.float32)
    W = synth.ternary_weights(N, K, seed=6200 + M)
    P = lib_pack(W)
    sw = synth.row_scales_bf16(N, seed=6300 + M)
    ref = oracle.linear_f32(x, P, sw)
    out = tg.bitnet_linear(dev_f32(x), dev(P), dev_bf16(sw))
    assert_bf16_parity(host_bf16(out), ref["out"], f"linear f32 {M}x{N}x{K}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(1, 3840, 2560), (3, 130, 256), (40, 1000, 1024), (17, 33, 68), (2048, 64, 512),
                                   (2, 1000, 6912), (4, 37, 8192)])
def test_linear_bias_parity(dtype, M, N, K):
    g = synth.rng(6400 + M + N + K)
    W = synth.ternary_weights(N, K, seed=6500 + M)
    P = lib_pack(W)
    sw = synth.row_scales_bf16(N, seed=6600 + M)
    bias = synth.row_scales_bf16(N, seed=6700 + M, lo=-4.0, hi=4.0)
    if dtype == "bf16":
        x = synth.activations_bf16(M, K, seed=6800 + M)
        ref = oracle.linear(x, P, sw)["out"]
        xd = dev_bf16(x)
    else:
        x = g.standard_normal((M, K)).astype(np.float32)
        ref = oracle.linear_f32(x, P, sw)["out"]
        xd = dev_f32(x)
    want = oracle.add_bias(ref, bias)
    out = tg.bitnet_linear(xd, dev(P), dev_bf16(sw), bias=dev_bf16(bias))
    assert_bf16_parity(host_bf16(out), want, f"linear+bias {dtype} {M}x{N}x{K}")


def test_linear_f32_fused_special_rows():
    """The GEMV prologue's f32 absmax and rounding on the rows that stress them:
    all zeros (the eps floor), values far below the floor, and one outlier."""
    M, N, K = 4, 300, 1024
    g = synth.rng(6900)
    x = g.standard_normal((M, K)).astype(np.float32)
    x[1, :] = 0.0
    x[2, :] = np.float32(2.0 ** -31)
    x[3, 17] = np.float32(3.0e4)
    W = synth.ternary_weights(N, K, seed=6901)
    P = lib_pack(W)
    sw = synth.row_scales_bf16(N, seed=6902)
    ref = oracle.linear_f32(x, P, sw)
    out = tg.bitnet_linear(dev_f32(x), dev(P), dev_bf16(sw))
    assert_bf16_parity(host_bf16(out), ref["out"], "linear f32 special rows")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(1, 3840, 2560), (2, 1000, 4096), (4, 300, 512)])
def test_linear_ex_fused_equals_split(dtype, M, N, K):
    """The one-launch path (quantise in the GEMV prologue, bias in its epilogue)
    and the quantise + GEMM + bias path give the same bits: a misaligned x
    sends the same call down the second."""
    W = synth.ternary_weights(N, K, seed=7000 + M)
    P = dev(lib_pack(W))
    sw = dev_bf16(synth.row_scales_bf16(N, seed=7001 + M))
    bias = dev_bf16(synth.row_scales_bf16(N, seed=7002 + M, lo=-4.0, hi=4.0))
    if dtype == "bf16":
        xd = dev_bf16(synth.activations_bf16(M, K, seed=7003 + M))
    else:
        xd = dev_f32(synth.rng(7004 + M).standard_normal((M, K)).astype(np.float32))
    for b in (None, bias):
        fused = tg.bitnet_linear(xd, P, sw, bias=b)
        split = tg.bitnet_linear(misaligned(xd), P, sw, bias=b)
        assert torch.equal(fused.view(torch.int16), split.view(torch.int16)), f"{dtype} {M}x{N}x{K} bias={b is not None}"
    if dtype == "bf16":  # bitnet_linear_ex itself with bf16 and no bias (the binding calls bitnet_linear there)
        lib = tg.load_library()
        o = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        st = lib.bitnet_linear_ex(o.data_ptr(), xd.data_ptr(), tg.DTYPE_BF16, P.data_ptr(), sw.data_ptr(), None,
                                  M, N, K, None, 0, torch.cuda.current_stream().cuda_stream)
        assert st == 0
        assert torch.equal(o.view(torch.int16), tg.bitnet_linear(xd, P, sw).view(torch.int16))


# ----------------------------------------------------------------------------- INT8 weight-only (W8A16)

def w8a16_problem(M, N, K, seed, int_x=False):
    g = synth.rng(seed)
    if int_x:
        # integer activations in [-8, 8]: every product and partial sum is an
        # integer below 2^24, so any fp32 summation order gives the exact sum
        x = synth._to_bf16_bits(g.integers(-8, 9, size=(M, K)).astype(np.float32))
    else:
        x = synth.activations_bf16(M, K, seed=seed + 1)
    q = synth.random_int8((N, K), seed=seed + 2)
    scale = (g.uniform(0.5, 2.0, size=N) * np.where(g.random(N) < 0.5, -1.0, 1.0) / 127.0).astype(np.float32)
    return x, q, scale


def assert_w8a16_close(got, y, bound, K, what):
    # fp32 summation of K exact products (bf16 x int8 fits 24 bits): each partial
    # sum rounds once, so |error| <= (K - 1) * 2^-24 * sum|x*q| * |scale| (to first
    # order; 1% slack covers the higher-order terms), plus one rounding of the
    # final product with the scale, 2^-24 * |y| (doubled for the fp32 input to it)
    tol = bound * (K * 2.0 ** -24) * 1.01 + np.abs(y) * 2.0 ** -23 + 1e-30
    err = np.abs(got.astype(np.float64) - y)
    worst = np.unravel_index(np.argmax(err / tol), err.shape)
    assert np.all(err <= tol), f"{what}: |err| {err[worst]:.3e} > tol {tol[worst]:.3e} at {worst}"


W8A16_EXACT_SHAPES = [(1, 64, 256), (5, 100, 4096), (32, 33, 1024), (33, 4096, 4096), (64, 96, 2560),
                      (3, 7, 200), (2, 4, 64),
                      # M <= 4 streaming kernel: partial last step, tiny K, the LDS limit, ragged N
                      (1, 13, 2576), (2, 130, 1040), (3, 257, 4096), (4, 9, 4096), (1, 8, 16), (1, 5, 16384),
                      (2, 3, 8192), (4, 1000, 2560),
                      # two column tiles per workgroup on wide layers: ragged N, one and two row tiles
                      (8, 16400, 512), (40, 16385, 1024), (17, 20000, 384), (3, 16392, 256), (20, 11000, 640),
                      # one column tile staging only 4, 8 or 16 activation rows: ragged N
                      (3, 1001, 1024), (7, 5000, 1280), (12, 300, 1024), (16, 4097, 512)]


@pytest.mark.parametrize("M,N,K", W8A16_EXACT_SHAPES)
def test_w8a16_exact_integer_activations(M, N, K):
    """Exact sums make the output bit-checkable: this pins the MFMA operand and
    result layouts (a swapped row, column or k index changes some output)."""
    x, q, scale = w8a16_problem(M, N, K, seed=7000 + M + N + K, int_x=True)
    y, _ = oracle.w8a16(x, q, scale)
    got = tg.w8a16_gemv(dev_bf16(x), dev(q), dev(scale)).cpu().numpy()
    assert np.array_equal(got, y.astype(np.float32)), f"w8a16 exact {M}x{N}x{K}"


W8A16_SHAPES = [(1, 4096, 4096), (1, 1, 256), (1, 32000, 4096), (3, 100, 256), (16, 4096, 4096), (16, 31, 11008),
                (33, 1000, 1024), (64, 257, 11008), (7, 300, 11072), (2, 64, 131072), (5, 300, 200), (4, 3, 68),
                (1, 128256, 2560), (2, 3840, 2560), (4, 13824, 2560), (1, 4096, 11008), (3, 2560, 6912),
                (16, 32000, 4096), (64, 16448, 2560), (32, 13824, 2560), (5, 128256, 2560)]


@pytest.mark.parametrize("M,N,K", W8A16_SHAPES)
def test_w8a16_parity(M, N, K):
    x, q, scale = w8a16_problem(M, N, K, seed=7100 + M + N + K)
    y, bound = oracle.w8a16(x, q, scale)
    got = tg.w8a16_gemv(dev_bf16(x), dev(q), dev(scale)).cpu().numpy()
    assert_w8a16_close(got, y, bound, K, f"w8a16 {M}x{N}x{K}")


def test_w8a16_misaligned_plain_path_and_determinism():
    M, N, K = 6, 130, 1024
    x, q, scale = w8a16_problem(M, N, K, seed=7200)
    y, bound = oracle.w8a16(x, q, scale)
    xd, qd, sd = dev_bf16(x), dev(q), dev(scale)
    fast = tg.w8a16_gemv(xd, qd, sd)
    assert torch.equal(fast, tg.w8a16_gemv(xd, qd, sd)), "fast path: repeated calls differ"
    plain = tg.w8a16_gemv(misaligned(xd), qd, sd)
    assert_w8a16_close(plain.cpu().numpy(), y, bound, K, "w8a16 misaligned x")
    assert_w8a16_close(fast.cpu().numpy(), y, bound, K, "w8a16 fast")


def test_w8a16_shape_errors():
    x = torch.zeros((65, 64), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((8, 64), dtype=torch.int8, device=DEV)
    s = torch.ones((8,), dtype=torch.float32, device=DEV)
    with pytest.raises(RuntimeError):
        tg.w8a16_gemv(x, q, s)                      # M > 64
    assert tg.w8a16_gemv(x[:0], q, s).shape == (0, 8)


# ----------------------------------------------------------------------------- RMSNorm + quantise

def rms_references(x, gain, eps):
    """The oracle's result and, for rows whose fp32 mean a different double
    summation order could round the other way, the result with that other mean."""
    ref = oracle.rmsnorm_quantize(x, gain, eps)
    alt = ref
    if ref["ambiguous"].any():
        alt = oracle.rmsnorm_quantize(x, gain, eps, means=ref["mean_alt"])
    return ref, alt


def rows_match(got, ref, alt, amb):
    """Per row: equal to the oracle's row, or (ambiguous rows only) to the alternative."""
    got = got.reshape(got.shape[0], -1)
    ok = np.all(got == ref.reshape(got.shape), axis=1)
    ok_alt = np.all(got == alt.reshape(got.shape), axis=1) & amb
    return ok | ok_alt


def check_rms_quantize(x, gain, eps, q, sa, xn, what):
    ref, alt = rms_references(x, gain, eps)
    amb = ref["ambiguous"]
    for name, got in (("x_norm", host_bf16(xn)), ("q", q.cpu().numpy()), ("scale_act", host_bf16(sa)[:, None])):
        want = ref["xn"] if name == "x_norm" else (ref["q"] if name == "q" else ref["scale_act"][:, None])
        want_alt = alt["xn"] if name == "x_norm" else (alt["q"] if name == "q" else alt["scale_act"][:, None])
        ok = rows_match(got, want, want_alt, amb)
        assert ok.all(), f"{what} {name}: rows {np.nonzero(~ok)[0][:8].tolist()} differ (ambiguous rows: {int(amb.sum())})"


RMS_QUANT_SHAPES = [(1, 2560), (4, 6912), (16, 4096), (33, 11008), (5, 100), (3, 20000), (2049, 2560), (7, 8),
                    (2, 2048), (3, 16384), (65, 640)]


@pytest.mark.parametrize("with_gain", [False, True])
@pytest.mark.parametrize("M,K", RMS_QUANT_SHAPES)
def test_rmsnorm_quantize_parity(M, K, with_gain):
    x = synth.activations_bf16(M, K, seed=8000 + M + K, outlier_frac=0.01)
    if M > 2:
        x[1, :] = 0                                          # zero row: eps alone
        x[2, :] = synth.activations_bf16(1, K, seed=8001)[0] & np.uint16(0x83FF)   # tiny magnitudes
    gain = synth.row_scales_bf16(K, seed=8002 + K, lo=0.25, hi=2.0) if with_gain else None
    eps = 1e-5 if with_gain else oracle.FP32_EPS
    xn = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    q, sa = tg.rmsnorm_quantize(dev_bf16(x), None if gain is None else dev_bf16(gain), eps, x_norm=xn)
    check_rms_quantize(x, gain, eps, q, sa, xn, f"rmsnorm_quantize {M}x{K} gain={with_gain}")


def test_rmsnorm_quantize_misaligned_plain_path():
    M, K = 5, 1024
    x = synth.activations_bf16(M, K, seed=8100)
    gain = synth.row_scales_bf16(K, seed=8101, lo=0.5, hi=1.5)
    xn = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    q, sa = tg.rmsnorm_quantize(misaligned(dev_bf16(x)), misaligned(dev_bf16(gain)), 1e-6, x_norm=xn)
    check_rms_quantize(x, gain, 1e-6, q, sa, xn, "rmsnorm_quantize misaligned")


@pytest.mark.parametrize("with_gain", [False, True])
@pytest.mark.parametrize("M,N,K", [(1, 3840, 2560), (2, 2560, 6912), (3, 130, 4096), (4, 13824, 2560), (1, 100, 1024),
                                   (1, 2560, 6912), (1, 4096, 11008),
                                   (5, 300, 2560), (16, 4096, 4096), (64, 1000, 1024), (300, 257, 512), (2, 33, 68)])
def test_linear_rms_parity(M, N, K, with_gain):
    x = synth.activations_bf16(M, K, seed=8200 + M + N + K)
    W = synth.ternary_weights(N, K, seed=8300 + M)
    P = lib_pack(W)
    sw = synth.row_scales_bf16(N, seed=8400 + M)
    gain = synth.row_scales_bf16(K, seed=8500 + K, lo=0.5, hi=1.5) if with_gain else None
    eps = oracle.FP32_EPS
    ref = oracle.linear_rms(x, P, sw, gain, eps)
    alt = oracle.linear_rms(x, P, sw, gain, eps, means=ref["mean_alt"]) if ref["ambiguous"].any() else ref
    out = tg.bitnet_linear_rms(dev_bf16(x), dev(P), dev_bf16(sw), None if gain is None else dev_bf16(gain), eps)
    ok = rows_match(host_bf16(out), ref["out"], alt["out"], ref["ambiguous"])
    assert ok.all(), f"linear_rms {M}x{N}x{K}: rows {np.nonzero(~ok)[0][:8].tolist()} differ"


def test_linear_rms_fused_equals_split_on_unambiguous_rows():
    M, N, K = 4, 4096, 2560
    x = synth.activations_bf16(M, K, seed=8600)
    W = synth.ternary_weights(N, K, seed=8601)
    Pd, swd = dev(lib_pack(W)), dev_bf16(synth.row_scales_bf16(N, seed=8602))
    xd = dev_bf16(x)
    fused = tg.bitnet_linear_rms(xd, Pd, swd)                 # fused decode GEMV with the prologue
    q, sa = tg.rmsnorm_quantize(xd)
    split = tg.bitnet_gemm(q, Pd, sa, swd)
    amb = oracle.rmsnorm_quantize(x)["ambiguous"]
    same = np.all(host_bf16(fused) == host_bf16(split), axis=1)
    assert np.all(same | amb)


@pytest.mark.parametrize("M", [1, 8])
@pytest.mark.parametrize("kind", ["denormal", "tiny_normal", "mixed"])
def test_w8a16_denormal_activations(M, kind):
    """bf16 subnormal and smallest-normal activations: both the vector (M = 1)
    and the matrix-unit (M = 8) paths keep them (no flush to zero)."""
    K, N = 1024, 96
    g = synth.rng(7300 + M)
    if kind == "denormal":
        bits = g.integers(1, 0x80, size=(M, K)).astype(np.uint16)
    elif kind == "tiny_normal":
        bits = g.integers(0x0080, 0x0100, size=(M, K)).astype(np.uint16)
    else:
        bits = synth.activations_bf16(M, K, seed=7301)
        bits[:, ::2] = g.integers(1, 0x80, size=(M, K // 2)).astype(np.uint16)
    bits |= g.integers(0, 2, size=(M, K)).astype(np.uint16) << 15
    q = synth.random_int8((N, K), seed=7302)
    scale = np.ones(N, dtype=np.float32)
    y, bound = oracle.w8a16(bits, q, scale)
    got = tg.w8a16_gemv(dev_bf16(bits), dev(q), dev(scale)).cpu().numpy()
    assert_w8a16_close(got, y, bound, K, f"w8a16 {kind} M={M}")
    assert np.all((got != 0) | (y == 0)), "an output was flushed to zero"
