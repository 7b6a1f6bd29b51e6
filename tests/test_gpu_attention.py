"""GPU parity of the head-sharded attention shard against the fp64 oracle:
QKV projection -> head-local causal (or full) softmax attention -> row
partial with the shard's W_o rows; sum over shards = unsharded MHA."""
import numpy as np
import pytest

import megatron_tensor_transformer_col_amd as tp
import oracle
import synth
from gpu_util import assert_close, dev, empty, host, note, torch

pytestmark = pytest.mark.gpu


def _run_shards(d, b, s, heads, n, causal):
    T_, h = d["X"].shape
    X = dev(d["X"])
    Ps, Os = [], []
    hl = heads // n
    for i in range(n):
        Wqkv = synth.qkv_shard(d["Wq"], d["Wk"], d["Wv"], i, n, heads)
        Wo = synth.out_shard(d["Wo"], i, n)
        P = empty((T_, h), "f32")
        ws = torch().empty(tp.tp_attn_heads_shard_workspace(tp.TP_BF16, b, s, hl, h // heads),
                           dtype=torch().uint8, device="cuda:0")
        tp.tp_attn_heads_shard(X, dev(Wqkv), dev(Wo), P, b, s, hl, d=h // heads, causal=causal, ws=ws)
        Ps.append(P)
        # O_i lives after QKV_i in the workspace: [T x hl*d] bf16
        off = ((T_ * 3 * hl * (h // heads) * 2) + 255) // 256 * 256
        Os.append(ws[off:off + T_ * hl * (h // heads) * 2].view(torch().bfloat16).view(T_, hl * (h // heads)))
    Y = empty((T_, h), "f32")
    tp.tp_shard_sum(Ps, Y)
    torch().cuda.synchronize()
    return Ps, Os, Y


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("b,s,heads,n", [(2, 200, 4, 2), (1, 1, 2, 1), (3, 64, 2, 2), (1, 333, 4, 4)])
def test_attention_medium(causal, b, s, heads, n):
    h = heads * 128
    note(f"attention b={b} s={s} heads={heads} n={n} causal={causal}")
    d = synth.make_mha_inputs(b * s, h, "bf16", seed=5, w_std=0.05)
    Ps, Os, Y = _run_shards(d, b, s, heads, n, causal)
    ref = oracle.mha(*(d[k].f32 for k in ("X", "Wq", "Wk", "Wv", "Wo")), heads=heads, b=b, s=s,
                     causal=causal)
    w = (heads // n) * 128
    for i in range(n):
        assert_close(host(Os[i]), ref["O"][:, i * w:(i + 1) * w], "bf16", f"O_{i}")
    assert_close(host(Y), ref["Y"], "bf16", "Y")


def test_attention_s1_returns_v_projection():
    # s = 1: the only weight is 1, so O = V = X Wv exactly up to bf16 rounding
    note("attention s=1")
    d = synth.make_mha_inputs(5, 256, "bf16", seed=8, w_std=0.05)
    _, Os, _ = _run_shards(d, 5, 1, 2, 1, True)
    V = d["X"].f64() @ d["Wv"].f64()
    assert_close(host(Os[0]), V, "bf16", "O == V")


def test_mha_heads_full_size_sampled():
    """b=4, s=2048, h=4096, 32 heads x 128, N=4: shard 0 and the shard sum,
    checked on batch element 3 (batches are independent)."""
    W = synth.WORKLOADS["mha_heads_bf16"]
    note("MHA full size")
    d = synth.make_mha_inputs(W.tokens, W.h, "bf16", seed=W.seed)
    Ps, Os, Y = _run_shards(d, W.b, W.s, W.heads, W.n_shards, True)
    bi = W.b - 1
    r = slice(bi * W.s, (bi + 1) * W.s)
    ref = oracle.mha(d["X"].f32[r], d["Wq"].f32, d["Wk"].f32, d["Wv"].f32, d["Wo"].f32,
                     heads=W.heads, b=1, s=W.s, causal=True)
    w = W.heads_shard * W.head_dim
    assert_close(host(Os[0][r]), ref["O"][:, :w], "bf16", "O_0")
    assert_close(host(Y[r]), ref["Y"], "bf16", "Y")


def test_attention_repeat_bitwise():
    note("attention determinism")
    d = synth.make_mha_inputs(2 * 256, 512, "bf16", seed=4)
    a = _run_shards(d, 2, 256, 4, 1, True)[2]
    b = _run_shards(d, 2, 256, 4, 1, True)[2]
    assert torch().equal(a, b)
