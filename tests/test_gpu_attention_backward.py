"""GPU parity of the attention-shard backward against the fp64 oracle.

Each shard's gradients are compared with the oracle's backward of the same
shard (its query heads, the kv heads they read, its rows of W_o; the
shard-local problem), and the sum of the shards' dX partials with the
oracle's unsharded dX.  Also: the forward's saved row statistic (log2 of the
softmax denominators) against the oracle's log-sum-exp, repeatability, and
the full Llama-size shard on sampled outputs."""
import math

import numpy as np
import pytest

import megatron_tensor_transformer_col_amd as tp
import oracle
import synth
from gpu_util import assert_close, dev, empty, host, note, torch

pytestmark = pytest.mark.gpu

HD = 128


def _r256(x):
    return (x + 255) // 256 * 256


def _inputs(b, s, heads, kv, seed, w_std=0.05):
    h = heads * HD
    d = synth.make_gqa_inputs(b * s, h, heads, kv, "bf16", seed=seed, w_std=w_std)
    d["dY"] = synth.draw_normal(np.random.default_rng(seed + 1), (b * s, h), 1.0, "bf16")
    return d


def _shard(d, i, n, heads, kv):
    hl = heads // n
    kvl = len(synth.gqa_kv_heads_of_shard(i, n, heads, kv))
    Wqkv = synth.gqa_qkv_shard(d["Wq"], d["Wk"], d["Wv"], i, n, heads, kv)
    Wo = synth.out_shard(d["Wo"], i, n)
    return hl, kvl, Wqkv, Wo


def _run(d, b, s, hl, kvl, Wqkv, Wo, causal, X=None, dY=None):
    T = torch()
    T_, h = d["X"].shape
    X = dev(d["X"]) if X is None else X
    dY = dev(d["dY"]) if dY is None else dY
    Wq, Wo_ = dev(Wqkv), dev(Wo)
    fws = T.empty(tp.tp_attn_gqa_shard_workspace(tp.TP_BF16, b, s, hl, kvl, HD), dtype=T.uint8, device="cuda:0")
    P = empty((T_, h), "f32")
    tp.tp_attn_gqa_shard(X, Wq, Wo_, P, b, s, hl, kvl, d=HD, causal=causal, ws=fws)
    nq = (hl + 2 * kvl) * HD
    dWqkv = empty((h, nq), "f32")
    dWo = empty((hl * HD, h), "f32")
    dX = empty((T_, h), "f32")
    tp.tp_attn_shard_backward(X, Wq, Wo_, dY, fws, dWqkv, dWo, dX, b, s, hl, kvl, d=HD, causal=causal)
    T.cuda.synchronize()
    return {"dWqkv": dWqkv, "dWo": dWo, "dX": dX, "fws": fws, "P": P}


def _shard_oracle(d, hl, kvl, Wqkv, Wo, b, s, causal, rows=None):
    q, k = hl * HD, (hl + kvl) * HD
    W = Wqkv.f32
    X, dY = d["X"].f32, d["dY"].f32
    if rows is not None:
        X, dY = X[rows], dY[rows]
    return oracle.mha_backward(X, W[:, :q], W[:, q:k], W[:, k:], Wo.f32, dY, heads=hl, b=b, s=s, causal=causal,
                               kv_heads=kvl, head_dim=HD)


def _close_or_zero(gpu, ref, scale, what):
    """Relative error against max|ref|; where the exact gradient is 0 (one
    visible key: the softmax is constant, so dQ = dK = 0), the rounding
    residue must stay within the tolerance of a related gradient's scale."""
    if np.max(np.abs(ref)) > 0:
        assert_close(gpu, ref, "bf16", what)
    else:
        assert np.max(np.abs(gpu)) <= 2e-2 * np.max(np.abs(scale)), what


def _check_shard(r, ref, hl, kvl, tag):
    q, k = hl * HD, (hl + kvl) * HD
    dW = host(r["dWqkv"])
    _close_or_zero(dW[:, :q], ref["dWq"], ref["dWv"], f"{tag} dWq")
    _close_or_zero(dW[:, q:k], ref["dWk"], ref["dWv"], f"{tag} dWk")
    assert_close(dW[:, k:], ref["dWv"], "bf16", f"{tag} dWv")
    assert_close(host(r["dWo"]), ref["dWo"], "bf16", f"{tag} dWo")
    assert_close(host(r["dX"]), ref["dX"], "bf16", f"{tag} dX")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("b,s,heads,kv,n", [(2, 200, 4, 4, 2), (1, 333, 8, 2, 2), (2, 130, 8, 2, 4),
                                            (1, 96, 4, 1, 4), (1, 70, 4, 4, 1), (1, 1, 2, 2, 1)])
def test_attention_backward_medium(causal, b, s, heads, kv, n):
    """Multi-head (kv = heads) and grouped-query shards with 1, 2 or 4 query
    heads per kv head, kv heads replicated when n > kv; ragged sequence
    lengths (several 64- and 128-row tiles plus a tail; s = 1)."""
    note(f"attn bwd b={b} s={s} heads={heads} kv={kv} n={n} causal={causal}")
    d = _inputs(b, s, heads, kv, seed=s + heads)
    dX_sum = np.zeros(d["X"].shape)
    for i in range(n):
        hl, kvl, Wqkv, Wo = _shard(d, i, n, heads, kv)
        r = _run(d, b, s, hl, kvl, Wqkv, Wo, causal)
        ref = _shard_oracle(d, hl, kvl, Wqkv, Wo, b, s, causal)
        _check_shard(r, ref, hl, kvl, f"shard {i}")
        dX_sum += host(r["dX"])
    full = oracle.mha_backward(*(d[k].f32 for k in ("X", "Wq", "Wk", "Wv", "Wo")), d["dY"].f32, heads=heads, b=b,
                               s=s, causal=causal, kv_heads=kv)
    assert_close(dX_sum, full["dX"], "bf16", "sum_i dX_i")


def test_forward_row_statistic():
    """The forward's saved statistic is log2(e) times the oracle's natural
    log-sum-exp of each row's scaled scores."""
    b, s, heads, kv = 2, 150, 4, 2
    note("attn fwd lse")
    d = _inputs(b, s, heads, kv, seed=4)
    hl, kvl, Wqkv, Wo = _shard(d, 0, 1, heads, kv)
    r = _run(d, b, s, hl, kvl, Wqkv, Wo, True)
    T_ = b * s
    off = _r256(T_ * (hl + 2 * kvl) * HD * 2) + _r256(T_ * hl * HD * 2)
    lse = host(r["fws"][off:off + T_ * hl * 4].view(torch().float32)).reshape(b, hl, s)
    ref = _shard_oracle(d, hl, kvl, Wqkv, Wo, b, s, True)["lse"].reshape(b, s, hl).transpose(0, 2, 1)
    assert_close(lse, ref * math.log2(math.e), "bf16", "lse2")


def test_backward_is_repeatable():
    b, s, heads, kv = 1, 300, 4, 2
    note("attn bwd determinism")
    d = _inputs(b, s, heads, kv, seed=5)
    hl, kvl, Wqkv, Wo = _shard(d, 0, 1, heads, kv)
    r1 = _run(d, b, s, hl, kvl, Wqkv, Wo, True)
    r2 = _run(d, b, s, hl, kvl, Wqkv, Wo, True)
    for k in ("dWqkv", "dWo", "dX"):
        assert torch().equal(r1[k], r2[k]), k


@pytest.mark.parametrize("name", ["mha_heads_bf16", "gqa_heads_bf16"])
def test_full_size_shard_sampled(name):
    """Shard 0 at full size (b 4, s 2048, h 4096, 32 query heads of 128 over
    4 shards; kv heads 32 or 8): the weight gradients of local kv head 0 and
    the query heads that read it over all 8192 tokens (dWq, dWk, dWv, dWo
    rows), and dX_0 on batch element 3 (sequences are independent)."""
    W = synth.WORKLOADS[name]
    kv = W.kv_heads or W.heads
    note(f"attn bwd full size {name}")
    # the workload's weight scale N(0, 0.02^2): larger weights at h = 4096
    # make the scores large and the softmax nearly one-hot, where the bf16
    # storage of the forward's Q, K, V alone moves dX by ~2% of its maximum
    d = _inputs(W.b, W.s, W.heads, kv, seed=W.seed, w_std=0.02)
    hl, kvl, Wqkv, Wo = _shard(d, 0, W.n_shards, W.heads, kv)
    r = _run(d, W.b, W.s, hl, kvl, Wqkv, Wo, True)
    dW = host(r["dWqkv"])
    Wf = Wqkv.f32
    q, k = hl * HD, (hl + kvl) * HD
    g = hl // kvl
    # the g local query heads that read local kv head 0, over all tokens
    ref = oracle.mha_backward(d["X"].f32, Wf[:, :g * HD], Wf[:, q:q + HD], Wf[:, k:k + HD], Wo.f32[:g * HD],
                              d["dY"].f32, heads=g, b=W.b, s=W.s, causal=True, kv_heads=1, head_dim=HD)
    assert_close(dW[:, :g * HD], ref["dWq"], "bf16", "dWq group 0")
    assert_close(dW[:, q:q + HD], ref["dWk"], "bf16", "dWk kv head 0")
    assert_close(dW[:, k:k + HD], ref["dWv"], "bf16", "dWv kv head 0")
    assert_close(host(r["dWo"])[:g * HD], ref["dWo"], "bf16", "dWo group 0")
    bi = W.b - 1
    rows = slice(bi * W.s, (bi + 1) * W.s)
    ref3 = _shard_oracle(d, hl, kvl, Wqkv, Wo, 1, W.s, True, rows=rows)
    assert_close(host(r["dX"][rows]), ref3["dX"], "bf16", "dX_0 batch element 3")


def test_empty_sequence_gives_zero_weight_gradients():
    """s = 0: nothing to differentiate; the weight gradients are exactly 0
    (the sum over no tokens) and no kernel reads the (empty) workspaces."""
    note("attn bwd s=0")
    T = torch()
    hl, kvl, h = 2, 1, 256
    X = T.empty((0, h), dtype=T.bfloat16, device="cuda:0")
    Wqkv = T.zeros((h, (hl + 2 * kvl) * HD), dtype=T.bfloat16, device="cuda:0")
    Wo = T.zeros((hl * HD, h), dtype=T.bfloat16, device="cuda:0")
    P = empty((0, h), "f32")
    fws = T.empty(max(1, tp.tp_attn_gqa_shard_workspace(tp.TP_BF16, 1, 0, hl, kvl, HD)), dtype=T.uint8,
                  device="cuda:0")
    tp.tp_attn_gqa_shard(X, Wqkv, Wo, P, 1, 0, hl, kvl, d=HD, ws=fws)
    dWqkv = empty((h, (hl + 2 * kvl) * HD), "f32", fill=float("nan"))
    dWo = empty((hl * HD, h), "f32", fill=float("nan"))
    dX = empty((0, h), "f32")
    tp.tp_attn_shard_backward(X, Wqkv, Wo, X, fws, dWqkv, dWo, dX, 1, 0, hl, kvl, d=HD)
    T.cuda.synchronize()
    assert T.count_nonzero(dWqkv).item() == 0 and T.count_nonzero(dWo).item() == 0
