"""CPU-side checks of the C ABI: the library loads, exports what include/bitnet.h
declares, packs on the host bit-exactly like the oracle, and rejects bad
arguments before touching any device.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_int8_gemm_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitnet.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bitnet_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["bitnet_pack_weights", "bitnet_quantize_act", "bitnet_gemm", "bitnet_gemv_fused",
                     "bitnet_linear", "bitnet_gemm_i32", "bitnet_gemv_fused_i32", "bitnet_scale_epilogue",
                     "bitnet_linear_workspace_bytes", "bitnet_status_string", "bitnet_version",
                     "bitnet_quantize_act_f32", "bitnet_linear_ex", "bitnet_linear_ex_workspace_bytes",
                     "bitnet_w8a16_gemv", "bitnet_rmsnorm_quantize", "bitnet_linear_rms",
                     "bitnet_linear_rms_workspace_bytes", "bitnet_linear_noalloc"]:
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = tg.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_exports_nothing_else():
    # the .so's dynamic symbol table: only the C ABI is visible
    out = os.popen(f"nm -D --defined-only {tg.library_path()}").read()
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert exported == set(declared_functions()), exported ^ set(declared_functions())


def test_library_links_no_oracle():
    deps = os.popen(f"ldd {tg.library_path()} 2>/dev/null").read()
    assert "oracle" not in deps
    syms = os.popen(f"nm -D {tg.library_path()}").read()
    assert "oracle_" not in syms


def test_host_pack_matches_oracle():
    for (N, K, seed) in ((1, 4, 1), (7, 12, 2), (33, 256, 3), (128, 2560, 4)):
        W = synth.ternary_weights(N, K, seed)
        got = tg.pack_weights(torch.from_numpy(W)).numpy()
        assert np.array_equal(got, oracle.pack(W))


def test_host_pack_errors():
    lib = tg.load_library()
    w = np.zeros((2, 8), dtype=np.int8)
    p = np.zeros((2, 2), dtype=np.uint8)
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    assert lib.bitnet_pack_weights(vp(p), vp(w), 2, 6) == 2          # K % 4
    assert lib.bitnet_pack_weights(vp(p), vp(w), -1, 8) == 2         # N < 0
    assert lib.bitnet_pack_weights(None, vp(w), 2, 8) == 1           # NULL
    assert lib.bitnet_pack_weights(vp(p), vp(w), 0, 8) == 0          # empty is fine
    w[1, 3] = 2
    assert lib.bitnet_pack_weights(vp(p), vp(w), 2, 8) == 3          # value outside {-1,0,1}
    w[1, 3] = -2
    assert lib.bitnet_pack_weights(vp(p), vp(w), 2, 8) == 3
    with pytest.raises(tg.BitnetError):
        tg.pack_weights(torch.full((1, 4), 5, dtype=torch.int8))


def test_shape_errors_precede_device_use():
    # These all fail argument validation and return before any HIP call.
    lib = tg.load_library()
    d = ctypes.c_void_p(16)  # never dereferenced
    assert lib.bitnet_gemm(d, d, d, d, d, 4, 8, 6, None) == 2                 # K % 4
    assert lib.bitnet_gemm(d, d, d, d, d, 4, 8, 0, None) == 2                 # K == 0
    assert lib.bitnet_gemm(d, d, d, d, d, 4, 8, 131072 + 4, None) == 2       # K > MAX_K
    assert lib.bitnet_gemm(d, d, d, d, d, -1, 8, 64, None) == 2               # M < 0
    assert lib.bitnet_gemm(d, d, d, d, d, 0, 8, 64, None) == 0                # M == 0: no-op
    assert lib.bitnet_gemm(d, d, d, d, d, 4, 0, 64, None) == 0                # N == 0: no-op
    assert lib.bitnet_gemm(None, d, d, d, d, 4, 8, 64, None) == 1             # NULL out
    assert lib.bitnet_gemv_fused(d, d, d, d, 16, 8, 64, None) == 2            # M > 15
    assert lib.bitnet_gemv_fused_i32(d, d, d, d, 16, 8, 64, None) == 2
    assert lib.bitnet_quantize_act(d, d, d, 4, 10, None) == 2
    assert lib.bitnet_quantize_act(None, d, d, 4, 64, None) == 1
    assert lib.bitnet_gemm_i32(d, d, d, 4, 8, 63, None) == 2
    assert lib.bitnet_linear(d, d, d, d, 32, 8, 64, None, 0, None) == 4       # workspace missing
    assert lib.bitnet_linear(d, d, d, d, 32, 8, 64, d, 100, None) == 4        # workspace too small
    assert lib.bitnet_scale_epilogue(None, d, d, d, 2, 2, None) == 1
    assert lib.bitnet_quantize_act_f32(d, d, d, 4, 10, None) == 2             # K % 4
    assert lib.bitnet_quantize_act_f32(d, None, d, 4, 64, None) == 1
    assert lib.bitnet_linear_ex(d, d, 7, d, d, None, 4, 8, 64, d, 1 << 20, None) == 3   # unknown dtype
    assert lib.bitnet_linear_ex(d, d, 1, d, d, None, 1, 8, 64, None, 0, None) == 4      # f32 always needs it
    assert lib.bitnet_linear_ex(d, d, 1, d, d, None, 4, 8, 62, d, 1 << 20, None) == 2   # K % 4
    assert lib.bitnet_linear_ex(None, d, 0, d, d, None, 4, 8, 64, d, 1 << 20, None) == 1
    assert lib.bitnet_w8a16_gemv(d, d, d, d, 65, 8, 64, None) == 2           # M > 64
    assert lib.bitnet_w8a16_gemv(d, d, d, d, 4, 8, 0, None) == 2             # K == 0
    assert lib.bitnet_w8a16_gemv(d, d, d, d, 4, 8, 131072 + 1, None) == 2   # K > MAX_K
    assert lib.bitnet_w8a16_gemv(d, d, d, d, 0, 8, 64, None) == 0            # M == 0: no-op
    assert lib.bitnet_w8a16_gemv(d, None, d, d, 4, 8, 64, None) == 1
    nan, inf = float("nan"), float("inf")
    assert lib.bitnet_rmsnorm_quantize(d, d, None, d, None, -1e-6, 4, 64, None) == 3     # eps < 0
    assert lib.bitnet_rmsnorm_quantize(d, d, None, d, None, nan, 4, 64, None) == 3       # eps NaN
    assert lib.bitnet_rmsnorm_quantize(d, d, None, d, None, inf, 4, 64, None) == 3       # eps inf
    assert lib.bitnet_rmsnorm_quantize(d, d, None, d, None, 1e-5, 4, 62, None) == 2      # K % 4
    assert lib.bitnet_rmsnorm_quantize(d, None, None, d, None, 1e-5, 4, 64, None) == 1
    assert lib.bitnet_rmsnorm_quantize(d, d, None, d, None, 1e-5, 0, 64, None) == 0      # M == 0: no-op
    assert lib.bitnet_linear_rms(d, d, None, 1e-5, d, d, 1, 8, 64, None, 0, None) == 4   # always needs it
    assert lib.bitnet_linear_rms(d, d, None, 1e-5, d, d, 1, 8, 64, d, 100, None) == 4    # too small
    assert lib.bitnet_linear_rms(d, d, None, -1.0, d, d, 1, 8, 64, d, 1 << 20, None) == 3
    assert lib.bitnet_linear_rms(None, d, None, 1e-5, d, d, 1, 8, 64, d, 1 << 20, None) == 1
    assert lib.bitnet_linear_rms(d, d, None, 1e-5, d, d, 1, 0, 64, None, 0, None) == 0   # N == 0: no-op
    assert lib.bitnet_linear_noalloc(d, d, d, d, 4, 8, 62, None) == 2                   # K % 4
    assert lib.bitnet_linear_noalloc(None, d, d, d, 4, 8, 64, None) == 1
    assert lib.bitnet_linear_noalloc(d, d, d, d, 8193, 8, 4096, None) == 7             # beyond the scratch
    assert lib.bitnet_linear_noalloc(d, d, d, d, 0, 8, 64, None) == 0                  # M == 0: no-op


def test_workspace_size():
    assert tg.linear_workspace_bytes(1, 2560) == 0
    assert tg.linear_workspace_bytes(2, 131072) == 0          # one or two rows: always the fused GEMV
    assert tg.linear_workspace_bytes(4, 8192) == 0            # up to four rows while K <= 8192
    assert tg.linear_workspace_bytes(4, 8196) == 33024 + 256
    assert tg.linear_workspace_bytes(5, 2560) == 12800 + 256  # from five rows: quantise + GEMM
    assert tg.linear_workspace_bytes(15, 2560) == 38400 + 256
    assert tg.linear_workspace_bytes(16, 4096) == 16 * 4096 + 256
    assert tg.linear_workspace_bytes(17, 100) == 1792 + 256
    assert tg.linear_workspace_bytes(17, 6) == 0   # invalid K
    # f32 activations always go through quantise + GEMM, so they need it at every M
    assert tg.linear_ex_workspace_bytes(1, 2560, torch.float32) == 2560 + 256
    assert tg.linear_ex_workspace_bytes(16, 4096, torch.float32) == 16 * 4096 + 256
    assert tg.linear_ex_workspace_bytes(3, 2560, torch.bfloat16) == 0
    assert tg.load_library().bitnet_linear_ex_workspace_bytes(4, 64, 9) == 0


def test_rms_workspace_size():
    lib = tg.load_library()
    assert lib.bitnet_linear_rms_workspace_bytes(1, 2560) == 2560 + 256
    assert lib.bitnet_linear_rms_workspace_bytes(3, 100) == 512 + 256
    assert lib.bitnet_linear_rms_workspace_bytes(16, 4096) == 16 * 4096 + 256
    assert lib.bitnet_linear_rms_workspace_bytes(4, 62) == 0


def test_status_strings():
    lib = tg.load_library()
    for code in range(8):
        assert lib.bitnet_status_string(code).decode() not in ("", "unknown status")
    assert lib.bitnet_version() >= 100


# ----------------------------------------------------------------------------- binding argument checks

def test_binding_rejects_bad_outputs():
    """Caller-supplied outputs are checked before any call: dtype, device,
    density and element count (the kernels write prod(shape) elements)."""
    like = torch.empty((2, 8), dtype=torch.bfloat16)
    ok = torch.empty((4, 6), dtype=torch.bfloat16)
    assert tg._need_out(ok, torch.bfloat16, (4, 6), "out", like) is ok
    assert tg._need_out(ok.view(24), torch.bfloat16, (4, 6), "out", like).numel() == 24   # any view of them
    with pytest.raises(TypeError):
        tg._need_out(torch.empty((4, 6), dtype=torch.float32), torch.bfloat16, (4, 6), "out", like)
    with pytest.raises(ValueError):
        tg._need_out(torch.empty((4, 5), dtype=torch.bfloat16), torch.bfloat16, (4, 6), "out", like)   # too small
    with pytest.raises(ValueError):
        tg._need_out(torch.empty((4, 7), dtype=torch.bfloat16), torch.bfloat16, (4, 6), "out", like)   # too large
    with pytest.raises(ValueError):
        tg._need_out(torch.empty((6, 4), dtype=torch.bfloat16).t(), torch.bfloat16, (4, 6), "out", like)  # strided
    with pytest.raises(ValueError):
        tg._need_out(torch.empty((4, 6), dtype=torch.bfloat16, device="meta"), torch.bfloat16, (4, 6), "out", like)
    assert tg._out_or_new(None, torch.int8, (3, 5), "out", like).shape == (3, 5)


def test_binding_rejects_bad_workspace():
    like = torch.empty((2, 8), dtype=torch.bfloat16)
    assert tg._workspace(None, 0, like) == (None, 0)
    ws, n = tg._workspace(None, 100, like)
    assert n == 100 and ws.dtype == torch.uint8
    ws = torch.empty((300,), dtype=torch.uint8)
    assert tg._workspace(ws, 256, like)[1] == 300
    with pytest.raises(ValueError):
        tg._workspace(ws, 301, like)                                       # too small
    with pytest.raises(TypeError):
        tg._workspace(torch.empty((300,), dtype=torch.int32), 256, like)   # bytes are uint8
    with pytest.raises(ValueError):
        tg._workspace(torch.empty((300, 2), dtype=torch.uint8)[:, 0], 256, like)   # strided
    with pytest.raises(ValueError):
        tg._workspace(torch.empty((300,), dtype=torch.uint8, device="meta"), 256, like)
