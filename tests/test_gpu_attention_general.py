"""GPU parity of the attention shard (forward and backward) on the general
path: fp32 operands and head dims other than 128, against the fp64 oracle.

The first case is the pages' own tensor-parallel attention example (hidden
size 128, 8 heads, so d = 16, fp32, 2 shards); the others cover grouped-query
shards, bf16 with d = 40 / 64, ragged sequence lengths, s = 1 and the
largest head dim (256).  Each shard's forward output O_i and its backward
gradients are compared with the oracle's shard-local problem, the shard sum
of the forward partials with the unsharded block."""
import numpy as np
import pytest

import megatron_tensor_transformer_col_amd as tp
import oracle
import synth
from gpu_util import assert_close, dev, empty, host, note, torch

pytestmark = pytest.mark.gpu

CODE = {"f32": tp.TP_F32, "bf16": tp.TP_BF16}
ES = {"f32": 4, "bf16": 2}


def _r256(x):
    return (x + 255) // 256 * 256


def _inputs(dt, b, s, heads, kv, hd, seed):
    h = heads * hd
    d = synth.make_gqa_inputs(b * s, h, heads, kv, dt, seed=seed, w_std=0.3 / np.sqrt(h))
    d["dY"] = synth.draw_normal(np.random.default_rng(seed + 1), (b * s, h), 1.0, dt)
    return d


def _shard(d, i, n, heads, kv):
    hl = heads // n
    kvl = len(synth.gqa_kv_heads_of_shard(i, n, heads, kv))
    return (hl, kvl, synth.gqa_qkv_shard(d["Wq"], d["Wk"], d["Wv"], i, n, heads, kv),
            synth.out_shard(d["Wo"], i, n))


def _forward(dt, d, b, s, hl, kvl, hd, Wqkv, Wo, causal):
    T = torch()
    T_, h = d["X"].shape
    fws = T.empty(tp.tp_attn_gqa_shard_workspace(CODE[dt], b, s, hl, kvl, hd), dtype=T.uint8, device="cuda:0")
    P = empty((T_, h), "f32")
    X, Wq, Wo_ = dev(d["X"]), dev(Wqkv), dev(Wo)
    tp.tp_attn_gqa_shard(X, Wq, Wo_, P, b, s, hl, kvl, d=hd, causal=causal, ws=fws)
    T.cuda.synchronize()
    off = _r256(T_ * (hl + 2 * kvl) * hd * ES[dt])
    tdt = T.float32 if dt == "f32" else T.bfloat16
    O = fws[off:off + T_ * hl * hd * ES[dt]].view(tdt).view(T_, hl * hd)
    return X, Wq, Wo_, fws, P, O


CASES = [
    # dtype, b, s, heads, kv, n, head dim
    ("f32", 2, 10, 8, 8, 2, 16),    # the pages' example: hidden 128, 8 heads, 2 shards
    ("f32", 1, 37, 4, 2, 2, 32),    # grouped-query, one kv head per shard
    ("f32", 2, 1, 2, 2, 1, 64),     # s = 1
    ("bf16", 2, 50, 4, 4, 2, 64),
    ("bf16", 1, 33, 6, 3, 3, 40),   # d = 40, one kv head per shard
    ("f32", 1, 20, 2, 1, 1, 256),   # largest head dim
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dt,b,s,heads,kv,n,hd", CASES)
def test_general_attention_forward(causal, dt, b, s, heads, kv, n, hd):
    note(f"general attention fwd {dt} b={b} s={s} heads={heads} kv={kv} n={n} d={hd} causal={causal}")
    d = _inputs(dt, b, s, heads, kv, hd, seed=s + hd)
    ref = oracle.mha_gqa(*(d[k].f32 for k in ("X", "Wq", "Wk", "Wv", "Wo")), heads=heads, kv_heads=kv, b=b, s=s,
                         causal=causal)
    Ps = []
    w = (heads // n) * hd
    for i in range(n):
        hl, kvl, Wqkv, Wo = _shard(d, i, n, heads, kv)
        _, _, _, _, P, O = _forward(dt, d, b, s, hl, kvl, hd, Wqkv, Wo, causal)
        assert_close(host(O), ref["O"][:, i * w:(i + 1) * w], dt, f"O_{i}")
        Ps.append(P)
    Y = empty(tuple(d["X"].shape), "f32")
    tp.tp_shard_sum(Ps, Y)
    torch().cuda.synchronize()
    assert_close(host(Y), ref["Y"], dt, "Y")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dt,b,s,heads,kv,n,hd", CASES)
def test_general_attention_backward(causal, dt, b, s, heads, kv, n, hd):
    note(f"general attention bwd {dt} b={b} s={s} heads={heads} kv={kv} n={n} d={hd} causal={causal}")
    d = _inputs(dt, b, s, heads, kv, hd, seed=2 * s + hd)
    T_, h = d["X"].shape
    dX_sum = np.zeros((T_, h))
    for i in range(n):
        hl, kvl, Wqkv, Wo = _shard(d, i, n, heads, kv)
        X, Wq, Wo_, fws, _, _ = _forward(dt, d, b, s, hl, kvl, hd, Wqkv, Wo, causal)
        nq = (hl + 2 * kvl) * hd
        dWqkv, dWo, dX = empty((h, nq), "f32"), empty((hl * hd, h), "f32"), empty((T_, h), "f32")
        tp.tp_attn_shard_backward(X, Wq, Wo_, dev(d["dY"]), fws, dWqkv, dWo, dX, b, s, hl, kvl, d=hd, causal=causal)
        torch().cuda.synchronize()
        q, k = hl * hd, (hl + kvl) * hd
        W = Wqkv.f32
        ref = oracle.mha_backward(d["X"].f32, W[:, :q], W[:, q:k], W[:, k:], Wo.f32, d["dY"].f32, heads=hl, b=b,
                                  s=s, causal=causal, kv_heads=kvl, head_dim=hd)
        dW = host(dWqkv)
        for name, got, exp in (("dWq", dW[:, :q], ref["dWq"]), ("dWk", dW[:, q:k], ref["dWk"])):
            if np.max(np.abs(exp)) > 0:
                assert_close(got, exp, dt, f"shard {i} {name}")
            else:
                # one visible key (s = 1, or causal row 0 alone): the softmax
                # is constant and dQ = dK = 0 exactly; the residue must stay
                # within the tolerance of dWv's scale
                assert np.max(np.abs(got)) <= 1e-2 * np.max(np.abs(ref["dWv"])), name
        assert_close(dW[:, k:], ref["dWv"], dt, f"shard {i} dWv")
        assert_close(host(dWo), ref["dWo"], dt, f"shard {i} dWo")
        assert_close(host(dX), ref["dX"], dt, f"shard {i} dX")
        dX_sum += host(dX)
    full = oracle.mha_backward(*(d[k].f32 for k in ("X", "Wq", "Wk", "Wv", "Wo")), d["dY"].f32, heads=heads, b=b,
                               s=s, causal=causal, kv_heads=kv)
    assert_close(dX_sum, full["dX"], dt, "sum_i dX_i")


def test_general_attention_lse_and_repeat():
    """The general forward's saved statistic equals log2(e) times the
    oracle's log-sum-exp, and repeated backward calls give identical bits."""
    dt, b, s, heads, kv, hd = "f32", 2, 45, 4, 2, 32
    note("general attention lse / repeat")
    d = _inputs(dt, b, s, heads, kv, hd, seed=9)
    hl, kvl, Wqkv, Wo = _shard(d, 0, 1, heads, kv)
    X, Wq, Wo_, fws, _, _ = _forward(dt, d, b, s, hl, kvl, hd, Wqkv, Wo, True)
    T_, h = d["X"].shape
    off = _r256(T_ * (hl + 2 * kvl) * hd * 4) + _r256(T_ * hl * hd * 4)
    lse = host(fws[off:off + T_ * hl * 4].view(torch().float32)).reshape(b, hl, s)
    q, k = hl * hd, (hl + kvl) * hd
    W = Wqkv.f32
    ref = oracle.mha_backward(d["X"].f32, W[:, :q], W[:, q:k], W[:, k:], Wo.f32, d["dY"].f32, heads=hl, b=b, s=s,
                              causal=True, kv_heads=kvl, head_dim=hd)
    exp2 = ref["lse"].reshape(b, s, hl).transpose(0, 2, 1) * np.log2(np.e)
    assert_close(lse, exp2, "f32", "lse2")
    outs = []
    for _ in range(2):
        dWqkv, dWo, dX = empty((h, k + kvl * hd), "f32"), empty((q, h), "f32"), empty((T_, h), "f32")
        tp.tp_attn_shard_backward(X, Wq, Wo_, dev(d["dY"]), fws, dWqkv, dWo, dX, b, s, hl, kvl, d=hd, causal=True)
        torch().cuda.synchronize()
        outs.append([t.clone() for t in (dWqkv, dWo, dX)])
    for a_, b_ in zip(*outs):
        assert torch().equal(a_, b_)
