"""Seeded synthetic inputs for the W1.58A8 linear layer.

This module only draws random numbers in the shapes and distributions of the
workloads; it holds none of the layer's arithmetic (no packing, no
quantisation, no contraction, no scaling).  Both the CPU oracle's tests and the
HIP library's tests/benchmark take their inputs from here, so that the two
sides see identical bytes.

Distributions (the workload descriptions of the BitNet-2B-4T and LLaMA-7B
shaped problems):
  * ternary weights: i.i.d. with P(-1) = 0.3, P(0) = 0.4, P(+1) = 0.3;
  * activations: N(0, 1) drawn in float32, rounded to bf16 (round to nearest
    even, by torch's dtype conversion); optionally a fixed 1% of the channels
    (columns of K) multiplied by 8 (exact in bf16) to stress the absmax;
  * weight scale: mean |W_fp| of W_fp ~ N(0, 0.02^2) (over at most 2^20
    draws), rounded to bf16 and broadcast to every output row;
  * per-row weight scales (an extra parity case): uniform in [0.004, 0.04],
    rounded to bf16.

Seeds: 0xB17E7000 + 16 * workload_index + tensor_id, one per tensor.
"""
import numpy as np
import torch

SEED_BASE = 0xB17E7000

# tensor ids within a workload
T_WEIGHT, T_ACT, T_SCALE, T_OUTLIER, T_ROWSCALE, T_BYTES = range(6)

# thresholds on a uniform 32-bit draw: u < T_NEG -> -1, u < T_ZERO -> 0, else +1
_T_NEG = int(round(0.3 * 2**32))
_T_ZERO = int(round(0.7 * 2**32))


def seed_for(workload, tensor):
    return SEED_BASE + 16 * int(workload) + int(tensor)


def rng(seed):
    return np.random.Generator(np.random.PCG64(int(seed)))


def ternary_weights(N, K, seed, rows_per_chunk=4096):
    """int8 [N, K] with P(-1)=0.3, P(0)=0.4, P(+1)=0.3."""
    g = rng(seed)
    W = np.empty((N, K), dtype=np.int8)
    for r0 in range(0, N, rows_per_chunk):
        r1 = min(N, r0 + rows_per_chunk)
        u = g.integers(0, 2**32, size=(r1 - r0, K), dtype=np.uint32)
        blk = np.ones((r1 - r0, K), dtype=np.int8)
        blk[u < _T_ZERO] = 0
        blk[u < _T_NEG] = -1
        W[r0:r1] = blk
    return W


def _to_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns to float32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def activations_bf16(M, K, seed, outlier_frac=0.0, outlier_mult=8.0, outlier_seed=None):
    """bf16 bit patterns [M, K] of N(0,1) draws; optional outlier channels x8."""
    g = rng(seed)
    x = g.standard_normal(size=(M, K), dtype=np.float32)
    bits = _to_bf16_bits(x)
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * K))
        go = rng(outlier_seed if outlier_seed is not None else seed + 1)
        cols = np.sort(go.choice(K, size=n_out, replace=False))
        f = bf16_bits_to_f32(bits)
        f[:, cols] *= np.float32(outlier_mult)   # power of two: exact in bf16
        bits = _to_bf16_bits(f)
    return bits


def weight_scale_bf16(N, K, seed, cap=1 << 20):
    """bf16 bits [N]: mean |W_fp| with W_fp ~ N(0, 0.02^2), broadcast."""
    g = rng(seed)
    n = min(int(N) * int(K), cap)
    w_fp = g.normal(0.0, 0.02, size=n)
    m = np.float32(np.mean(np.abs(w_fp)))
    bits = _to_bf16_bits(np.array([m], dtype=np.float32))[0]
    return np.full((N,), bits, dtype=np.uint16)


def row_scales_bf16(N, seed, lo=0.004, hi=0.04):
    g = rng(seed)
    return _to_bf16_bits(g.uniform(lo, hi, size=N).astype(np.float32))


def random_bytes(n, seed):
    """Uniform random bytes (for decode fuzzing: includes the unused code 0)."""
    return rng(seed).integers(0, 256, size=n, dtype=np.uint8)


def random_int8(shape, seed, lo=-127, hi=127):
    return rng(seed).integers(lo, hi + 1, size=shape, dtype=np.int16).astype(np.int8)


# The workloads (shapes of the BitNet-2B-4T decode layer set and the LLaMA-7B
# projections).
BITNET_2B_DECODE = [  # (name, N, K)
    ("qkv", 3840, 2560),
    ("o_proj", 2560, 2560),
    ("gate_up", 13824, 2560),
    ("down", 2560, 6912),
    ("lm_head", 128256, 2560),
]

LLAMA7B_SHAPES = [  # (name, N, K)
    ("qkvo", 4096, 4096),
    ("gate_up", 11008, 4096),
    ("down", 4096, 11008),
    ("lm_head", 32000, 4096),
]
