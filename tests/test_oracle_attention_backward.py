"""Pins for the oracle's attention-block backward (multi-head and
grouped-query).

Against: torch float64 autograd through scaled_dot_product_attention (an
independent library routine); central finite differences of L = <Y, dY>
evaluated with the pure-Python loop forward ``oracle.brute``; closed forms
(s = 1: the softmax is constant, so dQ = dK = 0 and dV = dO; zero queries:
uniform causal weights give dV_j = sum_{i >= j} dO_i / (i + 1)); torch's
logsumexp for the saved row statistic; and the head-sharding identities
dX = sum_i dX_i, dWqkv_i = column blocks of dWq/dWk/dWv, dWo_i = row block of
dWo, with kv heads replicated on several shards adding their dWk / dWv.
Planted mistakes (the dropped D term of the softmax Jacobian, a missing
1/sqrt(d) in dK) must fail a pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import block, brute

KEYS = ("X", "Wq", "Wk", "Wv", "Wo")


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def _inputs(b, s, h, heads, kv, seed=0, std=0.3):
    d = synth.make_gqa_inputs(b * s, h, heads, kv, "f32", seed=seed, w_std=std)
    args = [d[k].f32.astype(np.float64) for k in KEYS]
    dY = np.random.default_rng(seed + 100).standard_normal((b * s, h))
    return args, dY


def _torch_grads(args, dY, heads, kv, b, s, causal):
    X, Wq, Wk, Wv, Wo = (torch.tensor(a, requires_grad=True) for a in args)
    h = X.shape[1]
    d = h // heads

    def split(M, nh):  # [b*s, nh*d] -> [b, nh, s, d]
        return M.reshape(b, s, nh, d).permute(0, 2, 1, 3)

    O = torch.nn.functional.scaled_dot_product_attention(
        split(X @ Wq, heads), split(X @ Wk, kv), split(X @ Wv, kv), is_causal=causal, enable_gqa=True)
    Y = O.permute(0, 2, 1, 3).reshape(b * s, heads * d) @ Wo
    (Y * torch.from_numpy(dY)).sum().backward()
    return {"dX": X.grad, "dWq": Wq.grad, "dWk": Wk.grad, "dWv": Wv.grad, "dWo": Wo.grad}


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("heads,kv", [(4, 4), (4, 2), (4, 1)])
def test_vs_torch_autograd_float64(causal, heads, kv):
    b, s, h = 2, 23, 32
    args, dY = _inputs(b, s, h, heads, kv, seed=heads + kv)
    o = oracle.mha_backward(*args, dY, heads=heads, b=b, s=s, causal=causal, kv_heads=kv)
    ref = _torch_grads(args, dY, heads, kv, b, s, causal)
    for k, v in ref.items():
        assert _rel(o[k], v.numpy()) < 1e-12, k
    # the forward it carries is the GQA oracle's
    fwd = oracle.mha_gqa(*args, heads=heads, kv_heads=kv, b=b, s=s, causal=causal)
    assert _rel(o["Y"], fwd["Y"]) < 1e-14


def test_saved_row_statistic_is_torch_logsumexp():
    b, s, h, heads = 1, 19, 16, 2
    args, dY = _inputs(b, s, h, heads, heads, seed=7)
    o = oracle.mha_backward(*args, dY, heads=heads, b=b, s=s, causal=True)
    d = h // heads
    for t in range(heads):
        c = slice(t * d, (t + 1) * d)
        S = torch.from_numpy(o["Q"][:, c] @ o["K"][:, c].T / math.sqrt(d))
        S = S.masked_fill(torch.triu(torch.ones(s, s, dtype=torch.bool), 1), -math.inf)
        assert _rel(o["lse"][:, t], torch.logsumexp(S, dim=1).numpy()) < 1e-14
        # D = sum_c dO * O row by row
        assert _rel(o["D"][:, t], (o["dO"][:, c] * o["O"][:, c]).sum(axis=1)) < 1e-13


@pytest.mark.parametrize("causal", [True, False])
def test_finite_differences_against_brute_forward(causal):
    b, s, h, heads, kv = 1, 4, 8, 2, 1
    args, dY = _inputs(b, s, h, heads, kv, seed=11, std=0.5)
    o = oracle.mha_backward(*args, dY, heads=heads, b=b, s=s, causal=causal, kv_heads=kv)
    grads = dict(zip(KEYS, (o["dX"], o["dWq"], o["dWk"], o["dWv"], o["dWo"])))

    def loss(a):
        Y = brute.mha_gqa(*a, heads=heads, kv_heads=kv, b=b, s=s, causal=causal)["Y"]
        return float(np.sum(np.asarray(Y) * dY))

    eps = 1e-6
    rng = np.random.default_rng(3)
    for n, name in enumerate(KEYS):
        A = args[n]
        idx = [np.unravel_index(k, A.shape) for k in rng.choice(A.size, size=min(A.size, 12), replace=False)]
        for ij in idx:
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[n][ij] += eps
            minus[n][ij] -= eps
            fd = (loss(plus) - loss(minus)) / (2 * eps)
            assert abs(fd - grads[name][ij]) <= 1e-7 * max(1.0, np.max(np.abs(grads[name]))), (name, ij)


def test_closed_forms():
    rng = np.random.default_rng(5)
    s, d = 7, 8
    Q, K, V, dO = (rng.standard_normal((s, d)) for _ in range(4))
    # one key: the softmax is the constant 1
    g = oracle.attention_head_backward(Q[:1], K[:1], V[:1], dO[:1], causal=True)
    np.testing.assert_array_equal(g["dQ"], 0)
    np.testing.assert_array_equal(g["dK"], 0)
    np.testing.assert_array_equal(g["dV"], dO[:1])
    # zero queries: causal weights 1/(i+1) on keys j <= i
    g = oracle.attention_head_backward(np.zeros((s, d)), K, V, dO, causal=True)
    ref = np.array([sum(dO[i] / (i + 1) for i in range(j, s)) for j in range(s)])
    np.testing.assert_allclose(g["dV"], ref, rtol=1e-14, atol=1e-15)
    # causal query 0 sees one key: its dQ row is 0; the last key is seen only
    # by the last query
    g = oracle.attention_head_backward(Q, K, V, dO, causal=True)
    np.testing.assert_array_equal(g["dQ"][0], 0)
    np.testing.assert_allclose(g["dV"][-1], g["P"][-1, -1] * dO[-1], rtol=1e-14)


def _shard_args(args, heads, kv, n, i):
    """Shard i's weights in the unsharded layout: its query heads, the kv
    heads they read (replicated when n > kv), the rows of Wo of its heads."""
    X, Wq, Wk, Wv, Wo = args
    d = X.shape[1] // heads
    hl = heads // n
    u = synth.gqa_kv_heads_of_shard(i, n, heads, kv)
    qc = np.r_[i * hl * d:(i + 1) * hl * d]
    kc = np.concatenate([np.r_[j * d:(j + 1) * d] for j in u])
    return [X, Wq[:, qc], Wk[:, kc], Wv[:, kc], Wo[qc, :]], qc, kc, len(u)


@pytest.mark.parametrize("heads,kv,n", [(4, 4, 2), (8, 2, 2), (8, 2, 4), (4, 1, 4)])
def test_head_sharding_identity(heads, kv, n):
    b, s, h = 2, 9, 32
    args, dY = _inputs(b, s, h, heads, kv, seed=heads * n + kv)
    full = oracle.mha_backward(*args, dY, heads=heads, b=b, s=s, causal=True, kv_heads=kv)
    dX = np.zeros_like(full["dX"])
    dWk, dWv = np.zeros_like(full["dWk"]), np.zeros_like(full["dWv"])
    for i in range(n):
        sa, qc, kc, kvl = _shard_args(args, heads, kv, n, i)
        g = oracle.mha_backward(*sa, dY, heads=heads // n, b=b, s=s, causal=True, kv_heads=kvl, head_dim=h // heads)
        dX += g["dX"]
        assert _rel(g["dWq"], full["dWq"][:, qc]) < 1e-13
        assert _rel(g["dWo"], full["dWo"][qc, :]) < 1e-13
        dWk[:, kc] += g["dWk"]
        dWv[:, kc] += g["dWv"]
    assert _rel(dX, full["dX"]) < 1e-13
    assert _rel(dWk, full["dWk"]) < 1e-13
    assert _rel(dWv, full["dWv"]) < 1e-13


def _planted(monkeypatch, mistake):
    real = block.attention_head_backward

    def wrong(Q, K, V, dO, causal):
        g = real(Q, K, V, dO, causal)
        d = Q.shape[1]
        if mistake == "drop_D":
            dS = g["P"] * (np.asarray(dO) @ np.asarray(V).T)
            g["dQ"] = dS @ np.asarray(K) / np.sqrt(d)
            g["dK"] = dS.T @ np.asarray(Q) / np.sqrt(d)
        else:
            g["dK"] = g["dK"] * np.sqrt(d)
        return g

    monkeypatch.setattr(block, "attention_head_backward", wrong)


@pytest.mark.parametrize("mistake", ["drop_D", "unscaled_dK"])
def test_planted_mistake_is_caught(monkeypatch, mistake):
    b, s, h, heads = 1, 12, 16, 2
    args, dY = _inputs(b, s, h, heads, heads, seed=9)
    ref = _torch_grads(args, dY, heads, heads, b, s, True)
    _planted(monkeypatch, mistake)
    o = oracle.mha_backward(*args, dY, heads=heads, b=b, s=s, causal=True)
    errs = [_rel(o[k], ref[k].numpy()) for k in ("dX", "dWq", "dWk")]
    assert max(errs) > 1e-3
