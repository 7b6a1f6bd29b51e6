"""GPU parity of the grouped-query attention shard against the fp64 oracle:
QKV projection (shard's query heads + the kv heads they read) -> head-local
attention with query head t reading kv head t / group -> row partial; the
shard sum equals the unsharded grouped-query attention block."""
import pytest

import megatron_tensor_transformer_col_amd as tp
import oracle
import synth
from gpu_util import assert_close, dev, empty, host, note, torch

pytestmark = pytest.mark.gpu


def _run_shards(d, b, s, heads, kv, n, causal):
    T_, h = d["X"].shape
    hd = h // heads
    X = dev(d["X"])
    Ps, Os = [], []
    hl = heads // n
    for i in range(n):
        kvl = len(synth.gqa_kv_heads_of_shard(i, n, heads, kv))
        Wqkv = synth.gqa_qkv_shard(d["Wq"], d["Wk"], d["Wv"], i, n, heads, kv)
        Wo = synth.out_shard(d["Wo"], i, n)
        P = empty((T_, h), "f32")
        ws = torch().empty(tp.tp_attn_gqa_shard_workspace(tp.TP_BF16, b, s, hl, kvl, hd),
                           dtype=torch().uint8, device="cuda:0")
        tp.tp_attn_gqa_shard(X, dev(Wqkv), dev(Wo), P, b, s, hl, kvl, d=hd, causal=causal, ws=ws)
        Ps.append(P)
        off = ((T_ * (hl + 2 * kvl) * hd * 2) + 255) // 256 * 256
        Os.append(ws[off:off + T_ * hl * hd * 2].view(torch().bfloat16).view(T_, hl * hd))
    Y = empty((T_, h), "f32")
    tp.tp_shard_sum(Ps, Y)
    torch().cuda.synchronize()
    return Ps, Os, Y


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("b,s,heads,kv,n", [(2, 200, 4, 2, 2), (1, 333, 8, 2, 2), (2, 130, 8, 2, 4),
                                            (1, 96, 4, 1, 4), (1, 70, 8, 4, 1)])
def test_gqa_medium(causal, b, s, heads, kv, n):
    """kv heads per shard: 1 (n >= kv: replicated when n > kv), 2, 4."""
    h = heads * 128
    note(f"gqa b={b} s={s} heads={heads} kv={kv} n={n} causal={causal}")
    d = synth.make_gqa_inputs(b * s, h, heads, kv, "bf16", seed=11, w_std=0.05)
    Ps, Os, Y = _run_shards(d, b, s, heads, kv, n, causal)
    ref = oracle.mha_gqa(*(d[k].f32 for k in ("X", "Wq", "Wk", "Wv", "Wo")), heads=heads, kv_heads=kv,
                         b=b, s=s, causal=causal)
    w = (heads // n) * 128
    for i in range(n):
        assert_close(host(Os[i]), ref["O"][:, i * w:(i + 1) * w], "bf16", f"O_{i}")
    assert_close(host(Y), ref["Y"], "bf16", "Y")


def test_gqa_full_size_sampled():
    """b=4, s=2048, h=4096, 32 query / 8 kv heads of 128, N=4 (8 query and
    2 kv heads per shard): shard 0 and the shard sum on batch element 3."""
    W = synth.WORKLOADS["gqa_heads_bf16"]
    note("GQA full size")
    d = synth.make_gqa_inputs(W.tokens, W.h, W.heads, W.kv_heads, "bf16", seed=W.seed)
    Ps, Os, Y = _run_shards(d, W.b, W.s, W.heads, W.kv_heads, W.n_shards, True)
    bi = W.b - 1
    r = slice(bi * W.s, (bi + 1) * W.s)
    ref = oracle.mha_gqa(d["X"].f32[r], d["Wq"].f32, d["Wk"].f32, d["Wv"].f32, d["Wo"].f32,
                         heads=W.heads, kv_heads=W.kv_heads, b=1, s=W.s, causal=True)
    w = W.heads_shard * W.head_dim
    assert_close(host(Os[0][r]), ref["O"][:, :w], "bf16", "O_0")
    assert_close(host(Y[r]), ref["Y"], "bf16", "Y")


def test_gqa_with_one_group_equals_mha_entry():
    """kv_heads_local == heads_local through the GQA entry point gives the
    same bits as tp_attn_heads_shard."""
    note("gqa == mha entry")
    b, s, heads, n = 2, 160, 4, 1
    h = heads * 128
    d = synth.make_mha_inputs(b * s, h, "bf16", seed=12, w_std=0.05)
    Wqkv = dev(synth.qkv_shard(d["Wq"], d["Wk"], d["Wv"], 0, n, heads))
    Wo = dev(synth.out_shard(d["Wo"], 0, n))
    X = dev(d["X"])
    P1, P2 = empty((b * s, h), "f32"), empty((b * s, h), "f32")
    tp.tp_attn_heads_shard(X, Wqkv, Wo, P1, b, s, heads, d=128)
    tp.tp_attn_gqa_shard(X, Wqkv, Wo, P2, b, s, heads, heads, d=128)
    torch().cuda.synchronize()
    assert torch().equal(P1, P2)
