"""Largest sizes: outputs with more than 2^31 elements (64-bit row offsets
in every loader and epilogue) checked exactly on integer-valued inputs, and
a 16384-token attention sequence checked on sampled query rows (row q of a
causal head depends only on keys 0..q, so the oracle evaluates it on that
prefix)."""
import numpy as np
import pytest

import megatron_tensor_transformer_col_amd as tp
import oracle
import synth
from gpu_util import assert_close, dev, empty, host, note, torch

pytestmark = pytest.mark.gpu


def _ints(rng, shape):
    return rng.integers(-2, 3, size=shape).astype(np.float32)


def _bf16(a):
    return synth.Tensor(a, "bf16", synth.round_to_bf16_bits(a))


def _sample_rows(M, rng):
    return np.unique(np.concatenate([[0, 1, 127, 128, M // 2, M - 2, M - 1], rng.integers(0, M, 24)]))


def test_column_gemm_output_beyond_2_31_elements():
    """H [262144 x 8192] bf16 (2^31 elements, 4 GiB) = X [262144 x 64] W [64 x 8192]."""
    M, K, N = 262144, 64, 8192
    note(f"large col GEMM {M}x{K}x{N}")
    rng = np.random.default_rng(1)
    X, W = _ints(rng, (M, K)), _ints(rng, (K, N))
    H = empty((M, N), "bf16")
    tp.tp_col_linear_gelu(dev(_bf16(X)), dev(_bf16(W)), H, act="none")
    torch().cuda.synchronize()
    rows = _sample_rows(M, rng)
    exact = X[rows].astype(np.int64) @ W.astype(np.int64)  # |sum| <= 256: exact in bf16
    assert np.array_equal(host(H[torch().from_numpy(rows).to("cuda:0")]), exact.astype(np.float64))
    del H


def test_row_gemm_partial_beyond_2_31_elements():
    """P [262144 x 8192] fp32 (8 GiB) = H [262144 x 64] W2 [64 x 8192]."""
    M, K, N = 262144, 64, 8192
    note(f"large row GEMM {M}x{K}x{N}")
    rng = np.random.default_rng(2)
    X, W = _ints(rng, (M, K)), _ints(rng, (K, N))
    P = empty((M, N), "f32")
    tp.tp_row_linear_partial(dev(_bf16(X)), dev(_bf16(W)), P)
    torch().cuda.synchronize()
    rows = _sample_rows(M, rng)
    exact = X[rows].astype(np.int64) @ W.astype(np.int64)
    assert np.array_equal(host(P[torch().from_numpy(rows).to("cuda:0")]), exact.astype(np.float64))
    del P


def test_attention_16k_tokens_sampled_rows():
    """One sequence of 16384 tokens, 2 heads of 128 (causal): O on sampled
    query rows against the oracle on each row's key prefix."""
    b, s, heads = 1, 16384, 2
    h = heads * 128
    note(f"attention s={s}")
    d = synth.make_mha_inputs(b * s, h, "bf16", seed=21, w_std=0.05)
    Wqkv = synth.qkv_shard(d["Wq"], d["Wk"], d["Wv"], 0, 1, heads)
    Wo = synth.out_shard(d["Wo"], 0, 1)
    T = torch()
    ws = T.empty(tp.tp_attn_heads_shard_workspace(tp.TP_BF16, b, s, heads, 128), dtype=T.uint8, device="cuda:0")
    P = empty((s, h), "f32")
    tp.tp_attn_heads_shard(dev(d["X"]), dev(Wqkv), dev(Wo), P, b, s, heads, d=128, causal=True, ws=ws)
    T.cuda.synchronize()
    off = ((s * 3 * h * 2) + 255) // 256 * 256
    O = host(ws[off:off + s * h * 2].view(T.bfloat16).view(s, h))
    X = d["X"].f32.astype(np.float64)
    Q, K, V = (X @ d[k].f32.astype(np.float64) for k in ("Wq", "Wk", "Wv"))
    rng = np.random.default_rng(3)
    rows = _sample_rows(s, rng)
    ref = np.zeros((len(rows), h))
    for n, q in enumerate(rows):
        for t in range(heads):
            c = slice(t * 128, (t + 1) * 128)
            ref[n, c] = oracle.attention_heads(Q[q:q + 1, c], K[:q + 1, c], V[:q + 1, c], causal=False)[0]
    assert_close(O[rows], ref, "bf16", "O on sampled rows")
