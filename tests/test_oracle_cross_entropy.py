"""Pins for the oracle's vocabulary-parallel cross-entropy.

Against: brute-force loops, torch float64 cross_entropy (an independent
library routine), closed forms (uniform logits -> log V per row; a single
dominant logit), the shift invariance of softmax, and the decomposition's
identity: combining the shards' row statistics gives the unsharded
log-sum-exp, and the shard losses sum to the unsharded total.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute


def _data(T=12, V=40, seed=0, scale=3.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, V)) * scale, rng.integers(0, V, size=T)


def test_rows_vs_brute_force():
    Z, t = _data()
    np.testing.assert_allclose(oracle.cross_entropy_rows(Z, t), brute.cross_entropy_rows(Z, t), rtol=1e-13)


def test_rows_vs_torch_float64():
    Z, t = _data(T=64, V=1000, seed=1, scale=8.0)
    ref = torch.nn.functional.cross_entropy(torch.from_numpy(Z), torch.from_numpy(t), reduction="none")
    np.testing.assert_allclose(oracle.cross_entropy_rows(Z, t), ref.numpy(), rtol=1e-13)


def test_closed_forms():
    V = 37
    # uniform logits: every token has probability 1/V
    np.testing.assert_allclose(oracle.cross_entropy_rows(np.full((3, V), 2.5), [0, 5, 36]), math.log(V), rtol=1e-15)
    # one dominant logit L at the target: loss = log(1 + (V-1) e^{-L})
    L = 5.0
    Z = np.zeros((1, V)); Z[0, 7] = L
    np.testing.assert_allclose(oracle.cross_entropy_rows(Z, [7]), math.log1p((V - 1) * math.exp(-L)), rtol=1e-12)
    # large shift: softmax is shift invariant (no overflow with the max factored out)
    Z, t = _data(seed=2)
    np.testing.assert_allclose(oracle.cross_entropy_rows(Z + 1e4, t), oracle.cross_entropy_rows(Z, t), rtol=1e-9)


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_vocab_parallel_identity(n):
    Z, t = _data(T=32, V=64, seed=3 + n, scale=5.0)
    r = oracle.vocab_parallel_cross_entropy(Z, t, n)
    full = brute.cross_entropy_rows(Z, t)
    np.testing.assert_allclose(r["rows"], full, rtol=1e-12)
    np.testing.assert_allclose(r["total"], sum(full), rtol=1e-12)
    ref_lse = torch.logsumexp(torch.from_numpy(Z), dim=1).numpy()
    np.testing.assert_allclose(r["lse"], ref_lse, rtol=1e-14)
    # each shard's statistics are the plain row max and sum of exponentials
    w = 64 // n
    for i, (m, s) in enumerate(r["stats"]):
        Zi = Z[:, i * w:(i + 1) * w]
        np.testing.assert_array_equal(m, Zi.max(axis=1))
        np.testing.assert_allclose(s, [sum(math.exp(v - mm) for v in row) for row, mm in zip(Zi, m)], rtol=1e-14)
    with pytest.raises(ValueError):
        oracle.vocab_parallel_cross_entropy(Z, t, 5)


def test_dropped_rescale_mistake_is_caught():
    """A plausible mistake in the combination (adding the shards' sums of
    exponentials without rescaling them to a common max) must fail the
    torch log-sum-exp pin."""
    Z, t = _data(T=16, V=64, seed=9, scale=5.0)
    stats = [oracle.vocab_shard_stats(Z[:, i * 16:(i + 1) * 16]) for i in range(4)]
    M = np.max(np.stack([m for m, _ in stats]), axis=0)
    wrong = M + np.log(sum(s for _, s in stats))
    ref = torch.logsumexp(torch.from_numpy(Z), dim=1).numpy()
    assert np.max(np.abs(wrong - ref)) > 1e-2
