"""bitnet_linear_noalloc (the workspace in the library's static per-device
scratch) against bitnet_linear with a caller workspace, through the C ABI:
bit-identical outputs on two calls in a row, the second with a smaller input,
both also equal to the oracle; the size limit is a clean error."""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_int8_gemm_amd as tg

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bf16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def case(M, N, K, seed):
    x = synth.activations_bf16(M, K, seed, outlier_frac=0.01)
    x[M // 2] = 0                                        # an all-zero row: the eps floor
    W = synth.ternary_weights(N, K, seed + 1)
    P = tg.pack_weights(torch.from_numpy(W)).numpy()
    sw = synth.row_scales_bf16(N, seed + 2)
    return x, P, sw


# (M, N, K): quantise + GEMM through the scratch (a large call, then a smaller one), the largest
# M * K the scratch holds, and a fused-GEMV call that needs no scratch
CALLS = [[(300, 1000, 4096), (20, 500, 1024)], [(2048, 4096, 4096), (64, 11008, 4096)],
         [(16, 3840, 2560), (5, 2560, 6912)], [(1, 3000, 2560), (3, 100, 512)]]


@pytest.mark.parametrize("calls", CALLS, ids=["300x4096_then_20x1024", "2048x4096_then_64x4096",
                                              "16x2560_then_5x6912", "fused_1_then_3"])
def test_noalloc_matches_linear(calls):
    outs, refs, wants = [], [], []
    stream = torch.cuda.current_stream()
    for i, (M, N, K) in enumerate(calls):
        x, P, sw = case(M, N, K, seed=9000 + 31 * i + M)
        xd, Pd, swd = dev_bf16(x), torch.from_numpy(P).to(DEV), dev_bf16(sw)
        ws = torch.empty((max(tg.linear_workspace_bytes(M, K), 1),), dtype=torch.uint8, device=DEV)
        refs.append(tg.bitnet_linear(xd, Pd, swd, workspace=ws))
        o = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
        outs.append(tg.bitnet_linear_noalloc(xd, Pd, swd, out=o))   # the calls follow each other on one stream
        wants.append(oracle.linear(x, P, sw)["out"])
    stream.synchronize()
    for (M, N, K), o, r, w in zip(calls, outs, refs, wants):
        got = host_bf16(o)
        assert np.array_equal(got, host_bf16(r)), f"noalloc vs bitnet_linear at {M}x{N}x{K}"
        assert np.array_equal(got, w), f"noalloc vs oracle at {M}x{N}x{K}"


def test_noalloc_size_limit():
    K = 4096
    M_max = tg.NOALLOC_SCRATCH_BYTES // K                 # the most rows whose workspace fits
    while tg.linear_workspace_bytes(M_max, K) > tg.NOALLOC_SCRATCH_BYTES:
        M_max -= 1
    M_big = M_max + 1
    assert tg.linear_workspace_bytes(M_big, K) > tg.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M_big, K), dtype=torch.bfloat16, device=DEV)
    P = torch.zeros((8, K // 4), dtype=torch.uint8, device=DEV)
    sw = torch.ones((8,), dtype=torch.bfloat16, device=DEV)
    o = torch.empty((M_big, 8), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tg.BitnetError) as e:
        tg.bitnet_linear_noalloc(x, P, sw, out=o)
    assert e.value.status == 7
    # the largest size that fits runs, and matches bitnet_linear (all-zero x: +0.0 everywhere)
    xs = x[:M_max]
    o2 = torch.full((M_max, 8), 7.0, dtype=torch.bfloat16, device=DEV)
    tg.bitnet_linear_noalloc(xs, P, sw, out=o2)
    assert torch.equal(o2.view(torch.int16), tg.bitnet_linear(xs, P, sw).view(torch.int16))
