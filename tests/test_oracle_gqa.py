"""Pins for the oracle's grouped-query attention ("张量并行", 相关分析: GQA).

Against: brute-force loops, torch float64 scaled_dot_product_attention with
enable_gqa (an independent library routine), the reduction to multi-head
attention (kv_heads == heads, and K/V weight blocks repeated per group), and
the head-sharding identity Y = sum_i O_i Wo_i with the shard packing the
kernel consumes, including shards that replicate a key/value head.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import brute


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def _inputs(b, s, h, heads, kv, seed=0, std=0.3):
    d = synth.make_gqa_inputs(b * s, h, heads, kv, "f32", seed=seed, w_std=std)
    return [d[k].f32 for k in ("X", "Wq", "Wk", "Wv", "Wo")], d


@pytest.mark.parametrize("causal", [True, False])
def test_gqa_vs_brute_force(causal):
    b, s, h, heads, kv = 2, 5, 16, 4, 2
    args, _ = _inputs(b, s, h, heads, kv)
    o = oracle.mha_gqa(*args, heads=heads, kv_heads=kv, b=b, s=s, causal=causal)
    r = brute.mha_gqa(*args, heads=heads, kv_heads=kv, b=b, s=s, causal=causal)
    assert _rel(o["O"], r["O"]) < 1e-14
    assert _rel(o["Y"], r["Y"]) < 1e-14


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("heads,kv", [(8, 2), (8, 1), (8, 8)])
def test_gqa_vs_torch_sdpa_float64(causal, heads, kv):
    b, s, h = 2, 37, 128
    args, _ = _inputs(b, s, h, heads, kv, seed=3)
    o = oracle.mha_gqa(*args, heads=heads, kv_heads=kv, b=b, s=s, causal=causal)
    d = h // heads
    def split(M, nh):  # [b*s, nh*d] -> [b, nh, s, d]
        return torch.from_numpy(M).reshape(b, s, nh, d).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        split(o["Q"], heads), split(o["K"], kv), split(o["V"], kv), is_causal=causal, enable_gqa=True)
    ref = ref.permute(0, 2, 1, 3).reshape(b * s, heads * d).numpy()
    assert _rel(o["O"], ref) < 1e-14


def test_gqa_reduces_to_mha():
    b, s, h, heads, kv = 2, 9, 32, 4, 2
    args, _ = _inputs(b, s, h, heads, kv, seed=5)
    X, Wq, Wk, Wv, Wo = args
    d, g = h // heads, heads // kv
    # every query head reads the kv head of its group: repeating each kv
    # weight block g times gives the equivalent multi-head attention
    rep = lambda W: np.concatenate([W[:, (t // g) * d:(t // g + 1) * d] for t in range(heads)], axis=1)
    o = oracle.mha_gqa(X, Wq, Wk, Wv, Wo, heads=heads, kv_heads=kv, b=b, s=s)
    m = oracle.mha(X, Wq, rep(Wk), rep(Wv), Wo, heads=heads, b=b, s=s)
    assert _rel(o["Y"], m["Y"]) < 1e-14
    # kv_heads == heads is multi-head attention
    args2, _ = _inputs(b, s, h, heads, heads, seed=6)
    assert _rel(oracle.mha_gqa(*args2, heads=heads, kv_heads=heads, b=b, s=s)["Y"],
                oracle.mha(*args2, heads=heads, b=b, s=s)["Y"]) < 1e-14


@pytest.mark.parametrize("heads,kv,n", [(8, 4, 2), (8, 2, 2), (8, 2, 4), (8, 2, 8), (8, 1, 4)])
def test_gqa_head_sharding_identity(heads, kv, n):
    """Each shard attends with its packed [Wq_i | Wk_i | Wv_i]: local query
    head t reads local kv head t // (heads_local / kv_local); the partials
    O_i Wo_i sum to the unsharded Y (kv heads replicated when n > kv)."""
    b, s, h = 2, 7, 64
    args, dd = _inputs(b, s, h, heads, kv, seed=7)
    X, Wq, Wk, Wv, Wo = args
    full = oracle.mha_gqa(*args, heads=heads, kv_heads=kv, b=b, s=s)
    d, hl = h // heads, heads // n
    Y = np.zeros_like(full["Y"])
    for i in range(n):
        kvs = synth.gqa_kv_heads_of_shard(i, n, heads, kv)
        kvl = len(kvs)
        W = synth.gqa_qkv_shard(dd["Wq"], dd["Wk"], dd["Wv"], i, n, heads, kv).f32
        assert W.shape[1] == (hl + 2 * kvl) * d
        QKV = X.astype(np.float64) @ W
        O = np.zeros((b * s, hl * d))
        for bi in range(b):
            r = slice(bi * s, (bi + 1) * s)
            for t in range(hl):
                u = t // (hl // kvl)
                O[r, t * d:(t + 1) * d] = oracle.attention_heads(
                    QKV[r, t * d:(t + 1) * d], QKV[r, (hl + u) * d:(hl + u + 1) * d],
                    QKV[r, (hl + kvl + u) * d:(hl + kvl + u + 1) * d], True)
        Y += O @ synth.out_shard(dd["Wo"], i, n).f64()
    assert _rel(Y, full["Y"]) < 1e-13


def test_wrong_group_mapping_is_caught(monkeypatch):
    """A plausible mistake (query head t reading kv head t % kv_heads instead
    of t // g) must fail the torch pin."""
    b, s, h, heads, kv = 1, 11, 64, 4, 2
    args, _ = _inputs(b, s, h, heads, kv, seed=9)
    X, Wq, Wk, Wv, Wo = (a.astype(np.float64) for a in args)
    d = h // heads
    Q, K, V = X @ Wq, X @ Wk, X @ Wv
    wrong = np.zeros((s, h))
    for t in range(heads):
        u = t % kv
        wrong[:, t * d:(t + 1) * d] = oracle.attention_heads(Q[:, t * d:(t + 1) * d], K[:, u * d:(u + 1) * d],
                                                             V[:, u * d:(u + 1) * d], True)
    right = oracle.mha_gqa(*args, heads=heads, kv_heads=kv, b=b, s=s)["O"]
    assert _rel(wrong, right) > 1e-3
