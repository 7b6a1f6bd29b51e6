"""GPU: exact integer pins of the MFMA GEMM paths and the shard sum.

Integer-valued operands in {-2..2} make every product and partial sum exact
in fp32 (and the bf16 outputs exact while |value| <= 256), so the GPU result
must equal the exact integer product bit for bit, in any tile configuration
and with ragged M / N / K tails.
"""
import numpy as np
import pytest

import megatron_tensor_transformer_col_amd as tp
import synth
from gpu_util import dev, empty, host, note, torch

pytestmark = pytest.mark.gpu


def _ints(rng, shape):
    return rng.integers(-2, 3, size=shape).astype(np.float32)


def _as(dtype, a):
    return synth.Tensor(a, dtype, synth.round_to_bf16_bits(a) if dtype == "bf16" else None)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,K,N", [(1, 8, 8), (37, 24, 40), (300, 56, 264), (2048, 64, 2048),
                                   # bf16: leading column-tiles on 256 x 256 tiles, the rest on
                                   # 128 x 128 ones (8 of 12; 13 of 17 with ragged M and N)
                                   (8192, 64, 3072), (3976, 64, 4104)])
def test_col_linear_identity_act_exact(dtype, M, K, N):
    # |sum| <= 4K <= 256: exact in bf16 storage too
    note(f"col NN exact {dtype} {M}x{K}x{N}")
    rng = np.random.default_rng(M + K + N)
    X, W = _ints(rng, (M, K)), _ints(rng, (K, N))
    H = empty((M, N), dtype)
    prev = tp.tp_set_gemv_max_m(0)
    try:
        tp.tp_col_linear_gelu(dev(_as(dtype, X)), dev(_as(dtype, W)), H, act="none")
    finally:
        tp.tp_set_gemv_max_m(prev)
    torch().cuda.synchronize()
    exact = X.astype(np.int64) @ W.astype(np.int64)
    assert np.array_equal(host(H), exact.astype(np.float64))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,K,N", [(5, 16, 8), (129, 200, 136), (1024, 1032, 520), (4096, 256, 1024),
                                   # K % 64 == 0 and >= 64 tiles: the LDS-DMA kernel, ragged M / N
                                   (1000, 640, 1352), (3000, 1024, 2056), (8192, 64, 1024),
                                   # bf16: column-tiles split between 256 x 256 and 128 x 128 tiles
                                   (3976, 256, 4104),
                                   # bf16, eight-wave 256 x 256 tiles with 2 and 3 slabs of K
                                   # (the second ragged in M and N, split with 128 x 128 tiles)
                                   (8192, 128, 4096), (3976, 192, 4104)])
def test_row_partial_exact(dtype, M, K, N):
    note(f"row NN exact {dtype} {M}x{K}x{N}")
    rng = np.random.default_rng(7 * M + K)
    X, W = _ints(rng, (M, K)), _ints(rng, (K, N))
    P = empty((M, N), "f32", fill=float("nan"))
    prev = tp.tp_set_gemv_max_m(0)
    try:
        tp.tp_row_linear_partial(dev(_as(dtype, X)), dev(_as(dtype, W)), P)
    finally:
        tp.tp_set_gemv_max_m(prev)
    torch().cuda.synchronize()
    exact = X.astype(np.int64) @ W.astype(np.int64)
    assert np.array_equal(host(P), exact.astype(np.float64))


def test_strided_views_and_identity_weight():
    # leading dimensions larger than the width; W = I gives X back exactly
    note("col NN strided identity")
    T = torch()
    rng = np.random.default_rng(3)
    Xbig = _ints(rng, (70, 96))
    Xd = dev(_as("bf16", Xbig))[:, 8:72]            # 70 x 64 view, ld 96
    Wd = dev(_as("bf16", np.eye(64, dtype=np.float32)))
    Hbig = empty((70, 80), "bf16", fill=7.0)
    H = Hbig[:, 16:80]                              # ld 80
    prev = tp.tp_set_gemv_max_m(0)
    try:
        tp.tp_col_linear_gelu(Xd, Wd, H, act="none")
    finally:
        tp.tp_set_gemv_max_m(prev)
    T.cuda.synchronize()
    assert np.array_equal(host(H), Xbig[:, 8:72].astype(np.float64))
    assert np.all(host(Hbig[:, :16]) == 7.0)        # untouched outside the view


@pytest.mark.parametrize("n", [1, 2, 4, 8])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_shard_sum_exact(n, out):
    note(f"shard_sum n={n} out={out}")
    rng = np.random.default_rng(n)
    M, N = 333, 264
    parts = [rng.integers(-20, 21, size=(M, N)).astype(np.float32) for _ in range(n)]
    bias = rng.integers(-3, 4, size=(N,)).astype(np.float32)
    Y = empty((M, N), out)
    tp.tp_shard_sum([dev(p) for p in parts], Y, bias=dev(bias[None, :])[0])
    torch().cuda.synchronize()
    exact = np.sum(np.stack(parts).astype(np.int64), axis=0) + bias.astype(np.int64)
    assert np.array_equal(host(Y), exact.astype(np.float64))


def test_zero_tokens_is_a_noop():
    note("M=0")
    T = torch()
    X = T.empty((0, 64), dtype=T.bfloat16, device="cuda:0")
    W = T.zeros((64, 64), dtype=T.bfloat16, device="cuda:0")
    H = T.empty((0, 64), dtype=T.bfloat16, device="cuda:0")
    tp.tp_col_linear_gelu(X, W, H)
    P = T.empty((0, 64), dtype=T.float32, device="cuda:0")
    tp.tp_row_linear_partial(X, W, P)
    T.cuda.synchronize()


def test_repeat_runs_are_bitwise_identical():
    note("determinism NN")
    rng = np.random.default_rng(9)
    X = rng.standard_normal((1000, 512)).astype(np.float32)
    W = (rng.standard_normal((512, 768)) * 0.02).astype(np.float32)
    Xd, Wd = dev(_as("bf16", X)), dev(_as("bf16", W))
    outs = []
    for _ in range(3):
        H = empty((1000, 768), "bf16")
        tp.tp_col_linear_gelu(Xd, Wd, H)
        outs.append(H)
    torch().cuda.synchronize()
    for h in outs[1:]:
        assert torch().equal(h, outs[0])


@pytest.mark.parametrize("M,K,N", [(37, 24, 40), (8, 1024, 1032), (2048, 64, 2048), (1000, 640, 1352)])
def test_bf16_output_rounding_nearest_even(M, K, N):
    """bf16 outputs are the exact fp32 sums rounded to nearest, ties to even.

    Integer operands up to 60 in magnitude give exact sums of 9-17 bits, so
    most outputs need rounding to bf16's 8 significant bits and many land
    exactly on a tie; every output's bits must equal the CPU rounding of
    the exact sum (general and LDS-DMA kernels, and the decode GEMV)."""
    note(f"bf16 rounding {M}x{K}x{N}")
    rng = np.random.default_rng(3 * M + N)
    X = rng.integers(-60, 61, size=(M, K)).astype(np.float32)
    W = rng.integers(-4, 5, size=(K, N)).astype(np.float32)
    exact = (X.astype(np.int64) @ W.astype(np.int64)).astype(np.float32)
    want = synth.round_to_bf16_bits(exact)
    ties = np.count_nonzero((exact.view(np.uint32) & 0xFFFF) == 0x8000)
    assert ties > 0 or M * N < 4096
    for gemv_max in (0, 16):
        H = empty((M, N), "bf16")
        prev = tp.tp_set_gemv_max_m(gemv_max)
        try:
            tp.tp_col_linear_gelu(dev(_as("bf16", X)), dev(_as("bf16", W)), H, act="none")
        finally:
            tp.tp_set_gemv_max_m(prev)
        torch().cuda.synchronize()
        got = H.view(torch().int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), (gemv_max, int(np.count_nonzero(got != want)))
