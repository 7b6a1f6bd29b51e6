"""Pins for the oracle's head-sharded multi-head attention.

Against: brute-force loops, torch float64 scaled_dot_product_attention (an
independent library routine), closed forms (s = 1, zero queries -> prefix
mean / mean of V, first causal row, explicit two-token weights) and the
head-sharding identity  Y = sum_i O_i Wo_i.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import brute


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def _tiny(b=2, s=6, h=16, seed=0, std=0.3):
    return synth.make_mha_inputs(b * s, h, "f32", seed=seed, w_std=std)


@pytest.mark.parametrize("causal", [True, False])
def test_mha_vs_brute_force(causal):
    b, s, h, heads = 2, 6, 16, 4
    d = _tiny(b, s, h)
    args = [d[k].f32 for k in ("X", "Wq", "Wk", "Wv", "Wo")]
    o = oracle.mha(*args, heads=heads, b=b, s=s, causal=causal)
    r = brute.mha(*args, heads=heads, b=b, s=s, causal=causal)
    assert _rel(o["O"], r["O"]) < 1e-14
    assert _rel(o["Y"], r["Y"]) < 1e-14


@pytest.mark.parametrize("causal", [True, False])
def test_attention_vs_torch_sdpa_float64(causal):
    rng = np.random.default_rng(2)
    s, dh = 37, 16
    Q, K, V = (rng.standard_normal((s, dh)) for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a)[None, None] for a in (Q, K, V)), is_causal=causal)[0, 0]
    assert _rel(oracle.attention_heads(Q, K, V, causal), ref.numpy()) < 1e-14


def test_attention_closed_forms():
    rng = np.random.default_rng(4)
    s, dh = 9, 8
    K, V = rng.standard_normal((s, dh)), rng.standard_normal((s, dh))
    Q = rng.standard_normal((s, dh))
    # s = 1: the only weight is 1
    np.testing.assert_array_equal(oracle.attention_heads(Q[:1], K[:1], V[:1], True), V[:1])
    # causal first query sees only key 0
    np.testing.assert_allclose(oracle.attention_heads(Q, K, V, True)[0], V[0], rtol=0, atol=1e-15)
    # zero queries: uniform weights -> prefix mean (causal) / mean (non-causal)
    Z = np.zeros_like(Q)
    prefix = np.cumsum(V, axis=0) / np.arange(1, s + 1)[:, None]
    np.testing.assert_allclose(oracle.attention_heads(Z, K, V, True), prefix, rtol=0, atol=1e-14)
    np.testing.assert_allclose(oracle.attention_heads(Z, K, V, False),
                               np.broadcast_to(V.mean(axis=0), V.shape), rtol=0, atol=1e-14)


def test_attention_two_token_explicit_weights():
    # q = (a, 0), keys k0 = (1, 0), k1 = (0, 1) (d = 2): scores a/sqrt2 and 0,
    # so the second query (non-causal or causal row 1) weights are
    # w0 = sigmoid(a/sqrt2), w1 = 1 - w0.
    a = 1.7
    Q = np.array([[0.0, 0.0], [a, 0.0]])
    K = np.array([[1.0, 0.0], [0.0, 1.0]])
    V = np.array([[2.0, -1.0], [0.5, 3.0]])
    w0 = 1.0 / (1.0 + math.exp(-a / math.sqrt(2.0)))
    expect = w0 * V[0] + (1 - w0) * V[1]
    for causal in (True, False):
        got = oracle.attention_heads(Q, K, V, causal)[1]
        np.testing.assert_allclose(got, expect, rtol=0, atol=1e-15)


@pytest.mark.parametrize("n", [1, 2, 4])
def test_head_sharding_identity(n):
    # Y = [O_1 ... O_H] Wo = sum_i O_(heads of shard i) Wo_i   (no gather needed)
    b, s, h, heads = 2, 5, 32, 4
    d = _tiny(b, s, h, std=0.2)
    full = oracle.mha(*(d[k].f32 for k in ("X", "Wq", "Wk", "Wv", "Wo")), heads=heads, b=b, s=s)
    dh = h // heads
    parts = []
    for i in range(n):
        Wqkv = synth.qkv_shard(d["Wq"], d["Wk"], d["Wv"], i, n, heads).f32
        w = Wqkv.shape[1] // 3
        o = oracle.mha(d["X"].f32, Wqkv[:, :w], Wqkv[:, w:2 * w], Wqkv[:, 2 * w:],
                       synth.out_shard(d["Wo"], i, n).f32, heads=heads, b=b, s=s)
        np.testing.assert_allclose(o["O"], full["O"][:, i * w:(i + 1) * w], rtol=0, atol=1e-14)
        parts.append(o["Y"])
        assert w == (heads // n) * dh
    assert _rel(oracle.shard_sum(parts), full["Y"]) < 1e-14
