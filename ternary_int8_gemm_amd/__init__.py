"""Python binding of the gfx950 W1.58A8 linear-layer library (include/bitnet.h).

Argument marshalling only: every function checks dtypes/shapes/devices of the
torch tensors it is given, allocates outputs with torch (device memory is the
only thing torch is used for, plus the current HIP stream), and calls the C ABI
in libbitnet_hip.so through ctypes.  All arithmetic runs in the HIP kernels.

The names follow the API of "phanerozoic/bitnet-cpu v1,
torch-ext/bitnet_cpu/__init__.py": pack_weights, quantize_activation,
bitnet_gemm, bitnet_gemv_fused, bitnet_linear; plus the int32 debug entry
points bitnet_gemm_i32 / bitnet_gemv_fused_i32 and bitnet_scale_epilogue.

There is no fallback: if the library is not built, or the device is not an
MI355X (gfx950), calls raise.
"""
import ctypes
import os

import torch

__all__ = [
    "BitnetError", "load_library", "library_path", "pack_weights", "quantize_activation", "bitnet_gemm",
    "bitnet_gemv_fused", "bitnet_linear", "bitnet_gemm_i32", "bitnet_gemv_fused_i32", "bitnet_scale_epilogue",
    "linear_workspace_bytes", "FUSED_MAX_M", "MAX_K", "STATUS",
]

FUSED_MAX_M = 15
MAX_K = 131072

STATUS = {
    0: "BITNET_OK", 1: "BITNET_ERR_NULL", 2: "BITNET_ERR_SHAPE", 3: "BITNET_ERR_VALUE",
    4: "BITNET_ERR_WORKSPACE", 5: "BITNET_ERR_DEVICE", 6: "BITNET_ERR_LAUNCH", 7: "BITNET_ERR_TOO_LARGE",
}
NOALLOC_SCRATCH_BYTES = 32 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbitnet_hip.so")
_LIB = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_st = ctypes.c_int


class BitnetError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_status_string(status)})")


def library_path():
    return _LIB_PATH


def load_library():
    """Load libbitnet_hip.so; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with ternary_int8_gemm_amd/build.py (or __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "bitnet_pack_weights": [_p, _p, _i64, _i64],
        "bitnet_quantize_act": [_p, _p, _p, _i64, _i64, _p],
        "bitnet_gemm": [_p, _p, _p, _p, _p, _i64, _i64, _i64, _p],
        "bitnet_gemv_fused": [_p, _p, _p, _p, _i64, _i64, _i64, _p],
        "bitnet_linear": [_p, _p, _p, _p, _i64, _i64, _i64, _p, _sz, _p],
        "bitnet_linear_noalloc": [_p, _p, _p, _p, _i64, _i64, _i64, _p],
        "bitnet_gemm_i32": [_p, _p, _p, _i64, _i64, _i64, _p],
        "bitnet_gemv_fused_i32": [_p, _p, _p, _p, _i64, _i64, _i64, _p],
        "bitnet_scale_epilogue": [_p, _p, _p, _p, _i64, _i64, _p],
        "bitnet_quantize_act_f32": [_p, _p, _p, _i64, _i64, _p],
        "bitnet_linear_ex": [_p, _p, _st, _p, _p, _p, _i64, _i64, _i64, _p, _sz, _p],
        "bitnet_w8a16_gemv": [_p, _p, _p, _p, _i64, _i64, _i64, _p],
        "bitnet_rmsnorm_quantize": [_p, _p, _p, _p, _p, ctypes.c_float, _i64, _i64, _p],
        "bitnet_linear_rms": [_p, _p, _p, ctypes.c_float, _p, _p, _i64, _i64, _i64, _p, _sz, _p],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _st
    lib.bitnet_linear_workspace_bytes.argtypes = [_i64, _i64]
    lib.bitnet_linear_workspace_bytes.restype = _sz
    lib.bitnet_linear_ex_workspace_bytes.argtypes = [_i64, _i64, _st]
    lib.bitnet_linear_ex_workspace_bytes.restype = _sz
    lib.bitnet_linear_rms_workspace_bytes.argtypes = [_i64, _i64]
    lib.bitnet_linear_rms_workspace_bytes.restype = _sz
    lib.bitnet_status_string.argtypes = [_st]
    lib.bitnet_status_string.restype = ctypes.c_char_p
    lib.bitnet_version.argtypes = []
    lib.bitnet_version.restype = ctypes.c_int
    _LIB = lib
    return lib


def _status_string(status):
    try:
        return load_library().bitnet_status_string(int(status)).decode()
    except Exception:  # noqa: BLE001 - only used to format an error
        return "?"


def _check(status, what):
    if status != 0:
        raise BitnetError(status, what)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, dtype, name, device=True):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device and t.device.type != "cuda":
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_out(t, dtype, shape, name, like):
    """A caller-supplied output: `dtype`, dense, on the device of `like`, and
    holding exactly prod(shape) elements (its own shape may be any view of
    them); the kernels write that many elements from its first one."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != like.device:
        raise ValueError(f"{name} must be on {like.device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    n = 1
    for d in shape:
        n *= int(d)
    if t.numel() != n:
        raise ValueError(f"{name} must hold {tuple(shape)} = {n} elements, got {tuple(t.shape)}")
    return t


def _out_or_new(out, dtype, shape, name, like):
    if out is None:
        return torch.empty(tuple(shape), dtype=dtype, device=like.device)
    return _need_out(out, dtype, shape, name, like)


def _workspace(ws, need, like):
    """A caller-supplied workspace: dense uint8 bytes on the device of `like`,
    at least `need` of them.  Returns (tensor or None, its byte count)."""
    if ws is None:
        if need == 0:
            return None, 0
        ws = torch.empty((need,), dtype=torch.uint8, device=like.device)
    if ws.dtype != torch.uint8:
        raise TypeError(f"workspace must be torch.uint8, got {ws.dtype}")
    if ws.device != like.device:
        raise ValueError(f"workspace must be on {like.device}, got {ws.device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")
    return ws, ws.numel()


# ----------------------------------------------------------------------------- host packing

def pack_weights(W):
    """int8 W[N, K] in {-1, 0, +1} (host tensor) -> uint8 [N, K/4] (host)."""
    _need(W, torch.int8, "W", device=False)
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    N, K = W.shape
    out = torch.empty((N, K // 4), dtype=torch.uint8)
    _check(load_library().bitnet_pack_weights(_ptr(out), _ptr(W), N, K), "bitnet_pack_weights")
    return out


# ----------------------------------------------------------------------------- device calls

def quantize_activation(x, out=None, scale=None):
    """bf16 or f32 x[..., K] -> (int8 [M, K], bf16 scale [M]), M = prod of leading dims."""
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    _need(x, x.dtype, "x")
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    x2 = x.reshape(M, K)
    q = _out_or_new(out, torch.int8, (M, K), "out", x)
    s = _out_or_new(scale, torch.bfloat16, (M,), "scale", x)
    if x.dtype == torch.float32:
        _check(load_library().bitnet_quantize_act_f32(_ptr(q), _ptr(s), _ptr(x2), M, K, _stream(x)),
               "bitnet_quantize_act_f32")
    else:
        _check(load_library().bitnet_quantize_act(_ptr(q), _ptr(s), _ptr(x2), M, K, _stream(x)), "bitnet_quantize_act")
    return q, s


def bitnet_gemm(x_int8, w_packed, scale_act, scale_wt, out=None):
    """int8 x[M, K] x packed w[N, K/4] -> bf16 [M, N] with the scale epilogue."""
    _need(x_int8, torch.int8, "x_int8")
    _need(w_packed, torch.uint8, "w_packed")
    _need(scale_act, torch.bfloat16, "scale_act")
    _need(scale_wt, torch.bfloat16, "scale_wt")
    M, K = x_int8.shape
    N = w_packed.shape[0]
    if w_packed.shape[1] * 4 != K or scale_act.numel() != M or scale_wt.numel() != N:
        raise ValueError("bitnet_gemm: inconsistent shapes")
    o = _out_or_new(out, torch.bfloat16, (M, N), "out", x_int8)
    _check(load_library().bitnet_gemm(_ptr(o), _ptr(x_int8), _ptr(w_packed), _ptr(scale_act), _ptr(scale_wt),
                                      M, N, K, _stream(x_int8)), "bitnet_gemm")
    return o


def bitnet_gemv_fused(x, w_packed, scale_wt, out=None):
    """Fused quantise + GEMV for M <= 15: bf16 x[M, K] -> bf16 [M, N]."""
    _need(x, torch.bfloat16, "x")
    _need(w_packed, torch.uint8, "w_packed")
    _need(scale_wt, torch.bfloat16, "scale_wt")
    M, K = x.shape
    N = w_packed.shape[0]
    if w_packed.shape[1] * 4 != K or scale_wt.numel() != N:
        raise ValueError("bitnet_gemv_fused: inconsistent shapes")
    o = _out_or_new(out, torch.bfloat16, (M, N), "out", x)
    _check(load_library().bitnet_gemv_fused(_ptr(o), _ptr(x), _ptr(w_packed), _ptr(scale_wt), M, N, K, _stream(x)),
           "bitnet_gemv_fused")
    return o


def linear_workspace_bytes(M, K):
    return int(load_library().bitnet_linear_workspace_bytes(M, K))


DTYPE_BF16, DTYPE_F32 = 0, 1


def linear_ex_workspace_bytes(M, K, dtype=torch.bfloat16):
    code = DTYPE_F32 if dtype == torch.float32 else DTYPE_BF16
    return int(load_library().bitnet_linear_ex_workspace_bytes(M, K, code))


def bitnet_linear(x, w_packed, scale_wt, out=None, workspace=None, bias=None):
    """One-shot BitLinear forward: bf16 or f32 x[..., K] -> bf16 [..., N]; dispatches on M.

    bias (bf16 [N], optional) is added to the bf16 result as BitLinear does.
    bf16 input without bias calls bitnet_linear; anything else bitnet_linear_ex.
    """
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    _need(x, x.dtype, "x")
    _need(w_packed, torch.uint8, "w_packed")
    _need(scale_wt, torch.bfloat16, "scale_wt")
    if bias is not None:
        _need(bias, torch.bfloat16, "bias")
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    N = w_packed.shape[0]
    if w_packed.shape[1] * 4 != K or scale_wt.numel() != N or (bias is not None and bias.numel() != N):
        raise ValueError("bitnet_linear: inconsistent shapes")
    plain = x.dtype == torch.bfloat16 and bias is None
    ws_bytes = linear_workspace_bytes(M, K) if plain else linear_ex_workspace_bytes(M, K, x.dtype)
    ws, ws_n = _workspace(workspace, ws_bytes, x)
    o = _out_or_new(out, torch.bfloat16, (M, N), "out", x)
    lib = load_library()
    if plain:
        _check(lib.bitnet_linear(_ptr(o), _ptr(x), _ptr(w_packed), _ptr(scale_wt), M, N, K, _ptr(ws), ws_n,
                                 _stream(x)), "bitnet_linear")
    else:
        code = DTYPE_F32 if x.dtype == torch.float32 else DTYPE_BF16
        _check(lib.bitnet_linear_ex(_ptr(o), _ptr(x), code, _ptr(w_packed), _ptr(scale_wt), _ptr(bias), M, N, K,
                                    _ptr(ws), ws_n, _stream(x)), "bitnet_linear_ex")
    return o.view(*x.shape[:-1], N)


def bitnet_linear_noalloc(x, w_packed, scale_wt, out):
    """bitnet_linear for callers that cannot allocate: bf16 x[..., K] -> the
    given bf16 out [..., N].  The workspace is the library's static per-device
    scratch (NOALLOC_SCRATCH_BYTES); nothing is allocated, so `out` is required.
    Calls that overlap on one device race on that scratch."""
    _need(x, torch.bfloat16, "x")
    _need(w_packed, torch.uint8, "w_packed")
    _need(scale_wt, torch.bfloat16, "scale_wt")
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    N = w_packed.shape[0]
    if w_packed.shape[1] * 4 != K or scale_wt.numel() != N:
        raise ValueError("bitnet_linear_noalloc: inconsistent shapes")
    _need_out(out, torch.bfloat16, (M, N), "out", x)
    _check(load_library().bitnet_linear_noalloc(_ptr(out), _ptr(x), _ptr(w_packed), _ptr(scale_wt), M, N, K,
                                                _stream(x)), "bitnet_linear_noalloc")
    return out


def bitnet_gemm_i32(x_int8, w_packed, out=None):
    """Debug: int32 accumulators of the batched path."""
    _need(x_int8, torch.int8, "x_int8")
    _need(w_packed, torch.uint8, "w_packed")
    M, K = x_int8.shape
    N = w_packed.shape[0]
    if w_packed.shape[1] * 4 != K:
        raise ValueError("bitnet_gemm_i32: inconsistent shapes")
    o = _out_or_new(out, torch.int32, (M, N), "out", x_int8)
    _check(load_library().bitnet_gemm_i32(_ptr(o), _ptr(x_int8), _ptr(w_packed), M, N, K, _stream(x_int8)),
           "bitnet_gemm_i32")
    return o


def bitnet_gemv_fused_i32(x, w_packed):
    """Debug: (int32 accumulators [M, N], bf16 scales [M]) of the fused path."""
    _need(x, torch.bfloat16, "x")
    _need(w_packed, torch.uint8, "w_packed")
    M, K = x.shape
    N = w_packed.shape[0]
    if w_packed.shape[1] * 4 != K:
        raise ValueError("bitnet_gemv_fused_i32: inconsistent shapes")
    acc = torch.empty((M, N), dtype=torch.int32, device=x.device)
    sa = torch.empty((M,), dtype=torch.bfloat16, device=x.device)
    _check(load_library().bitnet_gemv_fused_i32(_ptr(acc), _ptr(sa), _ptr(x), _ptr(w_packed), M, N, K, _stream(x)),
           "bitnet_gemv_fused_i32")
    return acc, sa


def bitnet_scale_epilogue(acc, scale_act, scale_wt, out=None):
    """Debug: the scale epilogue on given int32 accumulators -> bf16."""
    _need(acc, torch.int32, "acc")
    _need(scale_act, torch.bfloat16, "scale_act")
    _need(scale_wt, torch.bfloat16, "scale_wt")
    M, N = acc.shape
    if scale_act.numel() != M or scale_wt.numel() != N:
        raise ValueError("bitnet_scale_epilogue: inconsistent shapes")
    o = _out_or_new(out, torch.bfloat16, (M, N), "out", acc)
    _check(load_library().bitnet_scale_epilogue(_ptr(o), _ptr(acc), _ptr(scale_act), _ptr(scale_wt), M, N,
                                                _stream(acc)), "bitnet_scale_epilogue")
    return o


W8A16_MAX_M = 64


def w8a16_gemv(x, q, scale, out=None):
    """INT8 weight-only matmul: bf16 x[M, K] (M <= 64), int8 q[N, K], fp32 scale[N] -> fp32 [M, N]."""
    _need(x, torch.bfloat16, "x")
    _need(q, torch.int8, "q")
    _need(scale, torch.float32, "scale")
    M, K = x.shape
    N = q.shape[0]
    if q.shape[1] != K or scale.numel() != N:
        raise ValueError("w8a16_gemv: inconsistent shapes")
    o = _out_or_new(out, torch.float32, (M, N), "out", x)
    _check(load_library().bitnet_w8a16_gemv(_ptr(o), _ptr(x), _ptr(q), _ptr(scale), M, N, K, _stream(x)),
           "bitnet_w8a16_gemv")
    return o


RMS_EPS_DEFAULT = 2.0 ** -23   # torch's rms_norm default eps (the fp32 epsilon)


def linear_rms_workspace_bytes(M, K):
    return load_library().bitnet_linear_rms_workspace_bytes(M, K)


def rmsnorm_quantize(x, gain=None, eps=RMS_EPS_DEFAULT, out=None, scale=None, x_norm=None):
    """RMSNorm then quantise: bf16 x[..., K], optional bf16 gain[K] -> (int8 [M, K], bf16 scale [M]).

    When x_norm (bf16 [M, K]) is given it receives the normalised activations."""
    _need(x, torch.bfloat16, "x")
    if gain is not None:
        _need(gain, torch.bfloat16, "gain")
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    if gain is not None and gain.numel() != K:
        raise ValueError("rmsnorm_quantize: gain must have K elements")
    if x_norm is not None:
        _need_out(x_norm, torch.bfloat16, (M, K), "x_norm", x)
    q = _out_or_new(out, torch.int8, (M, K), "out", x)
    sa = _out_or_new(scale, torch.bfloat16, (M,), "scale", x)
    _check(load_library().bitnet_rmsnorm_quantize(_ptr(q), _ptr(sa), _ptr(x_norm), _ptr(x), _ptr(gain), eps, M, K,
                                                  _stream(x)), "bitnet_rmsnorm_quantize")
    return q, sa


def bitnet_linear_rms(x, w_packed, scale_wt, gain=None, eps=RMS_EPS_DEFAULT, out=None, workspace=None):
    """RMSNorm then the BitLinear forward: bf16 x[..., K] -> bf16 [..., N]."""
    _need(x, torch.bfloat16, "x")
    _need(w_packed, torch.uint8, "w_packed")
    _need(scale_wt, torch.bfloat16, "scale_wt")
    if gain is not None:
        _need(gain, torch.bfloat16, "gain")
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    N = w_packed.shape[0]
    if w_packed.shape[1] * 4 != K or scale_wt.numel() != N or (gain is not None and gain.numel() != K):
        raise ValueError("bitnet_linear_rms: inconsistent shapes")
    ws, ws_n = _workspace(workspace, linear_rms_workspace_bytes(M, K), x)
    o = _out_or_new(out, torch.bfloat16, (M, N), "out", x)
    _check(load_library().bitnet_linear_rms(_ptr(o), _ptr(x), _ptr(gain), eps, _ptr(w_packed), _ptr(scale_wt), M, N,
                                            K, _ptr(ws), ws_n, _stream(x)), "bitnet_linear_rms")
    return o.view(*x.shape[:-1], N)
