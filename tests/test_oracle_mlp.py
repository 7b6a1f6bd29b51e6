"""Pins for the oracle's MLP blocks (GELU and SwiGLU), forward and backward.

Against: brute-force loops, exact integer arithmetic, torch float64 (an
independent library implementation of GELU/SiLU, matmul and autograd), the
pages' sharding identities, central finite differences and the adjoint
identity.  The tiny fp32 two-shard MLP workload (T = 2*16, h = 128,
ffn = 512, N = 2) is the main case.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import brute

W = synth.WORKLOADS["tiny_mlp_f32"]


def _tiny(T=W.tokens, h=W.h, ffn=W.ffn, seed=0, **kw):
    return synth.make_mlp_inputs(T, h, ffn, "f32", seed=seed, **kw)


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------- forward
def test_mlp_gelu_vs_brute_force():
    d = _tiny()
    o = oracle.mlp_gelu(d["X"].f32, d["W1"].f32, d["W2"].f32)
    b = brute.mlp_gelu(d["X"].f32, d["W1"].f32, d["W2"].f32)
    assert _rel(o["H"], b["H"]) < 1e-14
    assert _rel(o["Y"], b["Y"]) < 1e-14


def test_linear_exact_on_integers():
    rng = np.random.default_rng(3)
    X = rng.integers(-2, 3, size=(17, 40)).astype(np.float32)
    Wm = rng.integers(-2, 3, size=(40, 24)).astype(np.float32)
    exact = (X.astype(np.int64) @ Wm.astype(np.int64)).astype(np.float64)
    assert np.array_equal(oracle.linear(X, Wm), exact)
    assert np.array_equal(np.array(brute.matmul(X, Wm)), exact)
    # identity weight: X I = X
    assert np.array_equal(oracle.linear(X, np.eye(40)), X.astype(np.float64))


def test_mlp_gelu_vs_torch_float64():
    d = _tiny(with_bias=True)
    X, W1, W2 = (torch.from_numpy(d[k].f64()) for k in ("X", "W1", "W2"))
    b1, b2 = torch.from_numpy(d["b1"].f64()[0]), torch.from_numpy(d["b2"].f64()[0])
    ref = torch.nn.functional.gelu(X @ W1 + b1, approximate="none") @ W2 + b2
    o = oracle.mlp_gelu(d["X"].f32, d["W1"].f32, d["W2"].f32, d["b1"].f32[0], d["b2"].f32[0])
    assert _rel(o["Y"], ref.numpy()) < 1e-14


def test_mlp_swiglu_vs_torch_and_brute():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((12, 32))
    Wg, Wu, Wd = (rng.standard_normal(s) * 0.3 for s in ((32, 48), (32, 48), (48, 32)))
    o = oracle.mlp_swiglu(X, Wg, Wu, Wd)
    t = lambda a: torch.from_numpy(a)
    ref = (torch.nn.functional.silu(t(X) @ t(Wg)) * (t(X) @ t(Wu))) @ t(Wd)
    assert _rel(o["Y"], ref.numpy()) < 1e-14
    assert _rel(o["Y"], brute.mlp_swiglu(X, Wg, Wu, Wd)["Y"]) < 1e-14
    # W_up = 0  =>  Y = 0
    assert np.all(oracle.mlp_swiglu(X, Wg, np.zeros_like(Wu), Wd)["Y"] == 0.0)


# ---------------------------------------------------------------- sharding identities
def test_column_split_concat_identity():
    # X [B_1 B_2 ...] = [X B_1  X B_2 ...]
    d = _tiny()
    full = oracle.linear(d["X"].f32, d["W1"].f32)
    parts = [oracle.linear(d["X"].f32, synth.column_shard(d["W1"], i, W.n_shards).f32)
             for i in range(W.n_shards)]
    assert _rel(np.concatenate(parts, axis=1), full) < 1e-15


def test_row_split_sum_identity():
    # [X_1 X_2 ...] [A_1; A_2; ...] = sum_i X_i A_i
    d = _tiny()
    H = oracle.gelu(oracle.linear(d["X"].f32, d["W1"].f32))
    n, w = W.n_shards, W.ffn_shard
    parts = [oracle.row_partial(H[:, i * w:(i + 1) * w], synth.row_shard(d["W2"], i, n).f32)
             for i in range(n)]
    assert _rel(oracle.shard_sum(parts), H @ d["W2"].f64()) < 1e-14


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_megatron_mlp_identity(n):
    # Y = GELU(X [A_1 A_2]) [B_1; B_2] = sum_i GELU(X A_i) B_i, with b2 added once
    d = _tiny(with_bias=True)
    Y = oracle.mlp_gelu(d["X"].f32, d["W1"].f32, d["W2"].f32, d["b1"].f32[0], d["b2"].f32[0])["Y"]
    parts = []
    for i in range(n):
        W1i = synth.column_shard(d["W1"], i, n).f32
        b1i = synth.column_shard(d["b1"], i, n).f32[0]
        W2i = synth.row_shard(d["W2"], i, n).f32
        Hi = oracle.gelu(oracle.linear(d["X"].f32, W1i, b1i))
        parts.append(oracle.row_partial(Hi, W2i))
    assert _rel(oracle.shard_sum(parts, d["b2"].f32[0]), Y) < 1e-14
    # adding the row bias in every shard would be wrong by (n-1) b2
    if n > 1:
        wrong = oracle.shard_sum([p + d["b2"].f64() for p in parts])
        assert _rel(wrong, Y) > 1e-3


def test_gelu_not_additive_across_row_split():
    # GELU(sum_i X_i A_i) != sum_i GELU(X_i A_i): splitting W1 by rows cannot
    # apply GELU per shard.  The gap must dwarf the fp32 tolerance (1e-4).
    d = _tiny()
    n, w = W.n_shards, W.h // W.n_shards
    X, W1 = d["X"].f64(), d["W1"].f64()
    parts = [X[:, i * w:(i + 1) * w] @ W1[i * w:(i + 1) * w] for i in range(n)]
    good = oracle.gelu(sum(parts))
    bad = sum(oracle.gelu(p) for p in parts)
    assert _rel(bad, good) > 100 * 1e-4


# ---------------------------------------------------------------- backward
def _loss_gelu(X, W1, W2, dY, b1=None):
    return float(np.sum(oracle.mlp_gelu(X, W1, W2, b1)["Y"] * dY))


def test_mlp_gelu_backward_vs_brute_force():
    d = _tiny(T=8, with_dy=True)
    g = oracle.mlp_gelu_backward(d["X"].f32, d["W1"].f32, d["W2"].f32, d["dY"].f32)
    b = brute.mlp_gelu_backward(d["X"].f32, d["W1"].f32, d["W2"].f32, d["dY"].f32)
    for k in ("dX", "dW1", "dW2", "db1"):
        assert _rel(g[k], b[k]) < 1e-13, k


def test_mlp_gelu_backward_vs_torch_autograd():
    d = _tiny(with_dy=True, with_bias=True)
    X, W1, W2, b1 = (torch.from_numpy(d[k].f64()).requires_grad_() for k in ("X", "W1", "W2", "b1"))
    dY = torch.from_numpy(d["dY"].f64())
    Y = torch.nn.functional.gelu(X @ W1 + b1, approximate="none") @ W2
    (Y * dY).sum().backward()
    g = oracle.mlp_gelu_backward(d["X"].f32, d["W1"].f32, d["W2"].f32, d["dY"].f32, d["b1"].f32[0])
    assert _rel(g["dX"], X.grad.numpy()) < 1e-13
    assert _rel(g["dW1"], W1.grad.numpy()) < 1e-13
    assert _rel(g["dW2"], W2.grad.numpy()) < 1e-13
    assert _rel(g["db1"], b1.grad.numpy()[0]) < 1e-13


def test_mlp_gelu_backward_finite_differences():
    """Central differences of L = <Y, dY> in fp64 for every entry of X and 512
    random entries of each weight (tiny fp32 workload)."""
    d = _tiny(with_dy=True)
    X, W1, W2, dY = (d[k].f64() for k in ("X", "W1", "W2", "dY"))
    g = oracle.mlp_gelu_backward(X, W1, W2, dY)
    eps = 1e-6
    # X: rows are independent, so perturb one column of every row at once per pass
    for j in range(X.shape[1]):
        Xp, Xm = X.copy(), X.copy()
        Xp[:, j] += eps
        Xm[:, j] -= eps
        Yp = oracle.mlp_gelu(Xp, W1, W2)["Y"]
        Ym = oracle.mlp_gelu(Xm, W1, W2)["Y"]
        fd = np.sum((Yp - Ym) * dY, axis=1) / (2 * eps)
        np.testing.assert_allclose(g["dX"][:, j], fd, rtol=1e-6, atol=1e-7)
    rng = np.random.default_rng(7)
    for name, Wm in (("dW1", W1), ("dW2", W2)):
        idx = rng.integers(0, Wm.size, 512)
        for flat in idx:
            i, j = np.unravel_index(flat, Wm.shape)
            Wp, Wn = Wm.copy(), Wm.copy()
            Wp[i, j] += eps
            Wn[i, j] -= eps
            args_p = (X, Wp, W2) if name == "dW1" else (X, W1, Wp)
            args_m = (X, Wn, W2) if name == "dW1" else (X, W1, Wn)
            fd = (_loss_gelu(*args_p, dY) - _loss_gelu(*args_m, dY)) / (2 * eps)
            assert abs(g[name][i, j] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, i, j)


def test_mlp_backward_adjoint_identity():
    # <dY, J delta> = <J^T dY, delta> for a random direction delta of (X, W1, W2)
    d = _tiny(with_dy=True)
    X, W1, W2, dY = (d[k].f64() for k in ("X", "W1", "W2", "dY"))
    g = oracle.mlp_gelu_backward(X, W1, W2, dY)
    rng = np.random.default_rng(11)
    dX, dA, dB = (rng.standard_normal(a.shape) for a in (X, W1, W2))
    t = 1e-6
    jv = (oracle.mlp_gelu(X + t * dX, W1 + t * dA, W2 + t * dB)["Y"]
          - oracle.mlp_gelu(X - t * dX, W1 - t * dA, W2 - t * dB)["Y"]) / (2 * t)
    lhs = np.sum(dY * jv)
    rhs = np.sum(g["dX"] * dX) + np.sum(g["dW1"] * dA) + np.sum(g["dW2"] * dB)
    assert abs(lhs - rhs) <= 1e-7 * abs(rhs)


def test_column_backward_dx_is_sum_over_shards():
    # dX = sum_i dZ_i W1_i^T over column shards (Infra: Tensor Parallel, column-wise backward)
    d = _tiny(with_dy=True)
    g = oracle.mlp_gelu_backward(d["X"].f32, d["W1"].f32, d["W2"].f32, d["dY"].f32)
    n, w = W.n_shards, W.ffn_shard
    parts = [g["dZ"][:, i * w:(i + 1) * w] @ d["W1"].f64()[:, i * w:(i + 1) * w].T for i in range(n)]
    assert _rel(oracle.shard_sum(parts), g["dX"]) < 1e-14
    # and each shard's dW1_i / dW2_i is the same computation restricted to shard i
    for i in range(n):
        gi = oracle.mlp_gelu_backward(d["X"].f32, synth.column_shard(d["W1"], i, n).f32,
                                      synth.row_shard(d["W2"], i, n).f32, d["dY"].f32)
        assert _rel(gi["dW1"], g["dW1"][:, i * w:(i + 1) * w]) < 1e-14
        assert _rel(gi["dW2"], g["dW2"][i * w:(i + 1) * w]) < 1e-14


def test_mlp_swiglu_backward_vs_autograd_and_brute():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((10, 24))
    Wg, Wu, Wd = (rng.standard_normal(s) * 0.3 for s in ((24, 40), (24, 40), (40, 24)))
    dY = rng.standard_normal((10, 24))
    g = oracle.mlp_swiglu_backward(X, Wg, Wu, Wd, dY)
    tX, tg, tu, td = (torch.from_numpy(a).requires_grad_() for a in (X, Wg, Wu, Wd))
    Y = (torch.nn.functional.silu(tX @ tg) * (tX @ tu)) @ td
    (Y * torch.from_numpy(dY)).sum().backward()
    for k, ref in (("dX", tX), ("dWg", tg), ("dWu", tu), ("dWd", td)):
        assert _rel(g[k], ref.grad.numpy()) < 1e-13, k
    b = brute.mlp_swiglu_backward(X, Wg, Wu, Wd, dY)
    for k in ("dX", "dWg", "dWu", "dWd"):
        assert _rel(g[k], b[k]) < 1e-13, k
    # finite differences on a few weight entries
    eps = 1e-6
    L = lambda *a: float(np.sum(oracle.mlp_swiglu(*a)["Y"] * dY))
    for (i, j) in ((0, 0), (3, 7), (23, 39)):
        for name, idx in (("dWg", 1), ("dWu", 2)):
            args_p = [X, Wg.copy(), Wu.copy(), Wd]
            args_m = [X, Wg.copy(), Wu.copy(), Wd]
            args_p[idx][i, j] += eps
            args_m[idx][i, j] -= eps
            fd = (L(*args_p) - L(*args_m)) / (2 * eps)
            assert abs(g[name][i, j] - fd) <= 1e-6 * max(1.0, abs(fd))
