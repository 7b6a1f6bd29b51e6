"""GPU parity of the sequence-parallel reduce-scatter + LayerNorm against the
fp64 oracle: each rank's row block of LN(sum_i P_i + bias + residual), the
pre-norm sum, and the all-gathered result when the ranks write into one
buffer."""
import numpy as np
import pytest

import megatron_tensor_transformer_col_amd as tp
import oracle
import synth
from gpu_util import assert_close, dev, empty, host, note, torch

pytestmark = pytest.mark.gpu
EPS = 1e-5


def _ranks(d, T, n, out_dtype, with_bias=True, with_res=True, with_sum=True):
    P = [dev(p) for p in d["P"]]
    N = P[0].shape[1]
    bias = dev(d["bias"]) if with_bias else None
    res = dev(d["residual"]) if with_res else None
    g, b = dev(d["gamma"]), dev(d["beta"])
    Y = empty((T, N), out_dtype)
    S = empty((T, N), "f32") if with_sum else None
    rows = T // n
    for r in range(n):
        sl = slice(r * rows, (r + 1) * rows)
        tp.tp_shard_reduce_scatter_layernorm([p[sl] for p in P], g, b, Y[sl], eps=EPS, bias=bias,
                                             residual=None if res is None else res[sl],
                                             Ysum=None if S is None else S[sl])
    torch().cuda.synchronize()
    return Y, S


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,N,n", [(200, 1024, 4), (64, 4096, 2), (48, 8192, 3), (40, 4000, 2), (8, 8, 1)])
def test_reduce_scatter_layernorm_medium(out_dtype, T, N, n):
    note(f"rs-layernorm T={T} N={N} n={n} {out_dtype}")
    d = synth.make_sp_inputs(T, N, n, seed=N + n)
    Y, S = _ranks(d, T, n, out_dtype)
    for r in range(n):
        ref = oracle.reduce_scatter_layernorm(d["P"], d["gamma"], d["beta"], EPS, n, r, bias=d["bias"],
                                              residual=d["residual"])
        sl = slice(r * T // n, (r + 1) * T // n)
        assert_close(host(Y[sl]), ref["Y"], out_dtype, f"Y rank {r}")
        assert_close(host(S[sl]), ref["Ysum"], "f32", f"Ysum rank {r}")


def test_optional_terms_absent():
    note("rs-layernorm without bias / residual / Ysum")
    T, N, n = 96, 1024, 2
    d = synth.make_sp_inputs(T, N, n, seed=3)
    Y, _ = _ranks(d, T, n, "f32", with_bias=False, with_res=False, with_sum=False)
    full = sum(p.astype(np.float64) for p in d["P"])
    assert_close(host(Y), oracle.layernorm(full, d["gamma"], d["beta"], EPS), "f32", "Y")


def test_full_size_all_gathered():
    """T = 8192, N = 1024, 4 ranks of 2048 rows writing into one buffer: the
    gathered output equals LN of the all-reduced sum."""
    W = synth.WORKLOADS["sp_ln_gpt2m"]
    note("rs-layernorm full size")
    d = synth.make_sp_inputs(W.tokens, W.h, W.n_shards, seed=W.seed)
    Y, S = _ranks(d, W.tokens, W.n_shards, "bf16")
    full = oracle.shard_sum(d["P"], d["bias"]) + d["residual"].astype(np.float64)
    assert_close(host(S), full, "f32", "Ysum")
    assert_close(host(Y), oracle.layernorm(full, d["gamma"], d["beta"], EPS), "bf16", "Y")


def test_repeat_bitwise():
    note("rs-layernorm determinism")
    d = synth.make_sp_inputs(256, 4096, 4, seed=9)
    a, _ = _ranks(d, 256, 4, "f32")
    b, _ = _ranks(d, 256, 4, "f32")
    assert torch().equal(a, b)
