"""Pins for the oracle's LayerNorm and sequence-parallel reduce-scatter.

Against: brute-force loops, torch float64 layer_norm (an independent library
routine), closed forms (two-element rows, constant rows), the invariances of
the definition (shift and positive scale of a row with eps = 0; zero mean and
unit population variance of the normalised row) and the reduce-scatter
identity: the ranks' row blocks concatenate to LN of the all-reduced sum.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def _row_data(T=6, N=24, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, N)) * 3 + 1, 1 + 0.1 * rng.standard_normal(N),
            0.1 * rng.standard_normal(N))


def test_layernorm_vs_brute_force():
    x, g, b = _row_data()
    assert _rel(oracle.layernorm(x, g, b, 1e-5), brute.layernorm(x, g, b, 1e-5)) < 1e-14


@pytest.mark.parametrize("eps", [1e-5, 1e-12, 0.3])
def test_layernorm_vs_torch_float64(eps):
    x, g, b = _row_data(T=33, N=1024, seed=1)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (1024,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps)
    assert _rel(oracle.layernorm(x, g, b, eps), ref.numpy()) < 1e-14


def test_layernorm_closed_forms():
    one, zero = np.ones(2), np.zeros(2)
    # two-element row [a, b]: mean (a+b)/2, variance ((a-b)/2)^2
    a, b, eps = 3.0, -1.0, 0.25
    c = ((a - b) / 2) / math.sqrt(((a - b) / 2) ** 2 + eps)
    np.testing.assert_allclose(oracle.layernorm([[a, b]], one, zero, eps), [[c, -c]], rtol=1e-15)
    # constant row: x - mu = 0, the output is beta
    beta = np.array([0.5, -2.0, 7.0])
    np.testing.assert_array_equal(oracle.layernorm([[4.0, 4.0, 4.0]], np.full(3, 3.0), beta, 1e-5)[0], beta)


def test_layernorm_invariances():
    x, _, _ = _row_data(T=5, N=64, seed=2)
    g, b = np.ones(64), np.zeros(64)
    y = oracle.layernorm(x, g, b, 0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-14)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1, rtol=1e-13)
    # shift by a per-row constant and positive per-row scale: unchanged (eps = 0)
    z = x * np.array([[0.5], [2.0], [3.0], [10.0], [0.1]]) + np.array([[7.0], [-3.0], [0.0], [1e3], [-5.0]])
    assert _rel(oracle.layernorm(z, g, b, 0.0), y) < 1e-12


@pytest.mark.parametrize("n", [1, 2, 4])
def test_reduce_scatter_blocks_concatenate_to_full_layernorm(n):
    rng = np.random.default_rng(3 + n)
    T, N = 16, 48
    P = [rng.standard_normal((T, N)) for _ in range(3)]
    bias, res = rng.standard_normal(N), rng.standard_normal((T, N))
    g, b = 1 + 0.1 * rng.standard_normal(N), rng.standard_normal(N)
    full_sum = P[0] + P[1] + P[2] + bias + res
    blocks = [oracle.reduce_scatter_layernorm(P, g, b, 1e-5, n, r, bias=bias, residual=res) for r in range(n)]
    assert _rel(np.concatenate([x["Ysum"] for x in blocks]), full_sum) < 1e-15
    assert _rel(np.concatenate([x["Y"] for x in blocks]), brute.layernorm(full_sum, g, b, 1e-5)) < 1e-14
    with pytest.raises(ValueError):
        oracle.reduce_scatter_layernorm(P, g, b, 1e-5, 5, 0)


def test_unbiased_variance_mistake_is_caught():
    """A plausible mistake (sample variance 1/(N-1) instead of the population
    variance) must fail the torch pin's tolerance."""
    x, g, b = _row_data(T=8, N=64, seed=4)
    mu = x.mean(axis=1, keepdims=True)
    wrong = g * (x - mu) / np.sqrt(((x - mu) ** 2).sum(axis=1, keepdims=True) / 63 + 1e-5) + b
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), torch.from_numpy(b), 1e-5)
    assert _rel(wrong, ref.numpy()) > 1e-3
    assert _rel(oracle.layernorm(x, g, b, 1e-5), ref.numpy()) < 1e-14
