"""GPU parity of the MLP shard path (column GEMM + GELU/SwiGLU, row partial,
shard sum, backward) against the fp64 oracle of the UNSHARDED block.

Tolerance: max|gpu - ref| / max|ref| <= 1e-4 (fp32) / 2e-2 (bf16).
Full-size workloads are checked on sampled token rows / weight columns that
the oracle computes exactly (rows are independent; columns of the column
shard are separable), in the launch configuration the benchmark uses.
"""
import numpy as np
import pytest

import megatron_tensor_transformer_col_amd as tp
import oracle
import synth
from gpu_util import assert_close, dev, empty, host, note, torch

pytestmark = pytest.mark.gpu


def _shards(d, n, key1, key2):
    return ([synth.column_shard(d[key1], i, n) for i in range(n)],
            [synth.row_shard(d[key2], i, n) for i in range(n)])


def _forward_gelu(d, n, dtype, bias=False):
    """Run all n shards + shard sum on the GPU; return (H_i, P_i, Y) device tensors."""
    X = dev(d["X"])
    W1s, W2s = _shards(d, n, "W1", "W2")
    T_, h = d["X"].shape
    Hs, Ps = [], []
    for i in range(n):
        b1 = dev(synth.column_shard(d["b1"], i, n))[0] if bias else None
        H = empty((T_, W1s[i].shape[1]), dtype)
        tp.tp_col_linear_gelu(X, dev(W1s[i]), H, bias=b1)
        P = empty((T_, h), "f32")
        tp.tp_row_linear_partial(H, dev(W2s[i]), P)
        Hs.append(H)
        Ps.append(P)
    Y = empty((T_, h), "f32")
    tp.tp_shard_sum(Ps, Y, bias=dev(d["b2"])[0] if bias else None)
    torch().cuda.synchronize()
    return Hs, Ps, Y


# ---------------------------------------------------------------- tiny fp32 workload
def test_tiny_mlp_f32_forward():
    W = synth.WORKLOADS["tiny_mlp_f32"]
    note("tiny fp32 MLP forward")
    d = synth.make_mlp_inputs(W.tokens, W.h, W.ffn, "f32", seed=W.seed)
    Hs, Ps, Y = _forward_gelu(d, W.n_shards, "f32")
    ref = oracle.mlp_gelu(d["X"].f32, d["W1"].f32, d["W2"].f32)
    w = W.ffn_shard
    for i in range(W.n_shards):
        assert_close(host(Hs[i]), ref["H"][:, i * w:(i + 1) * w], "f32", f"H_{i}")
        assert_close(host(Ps[i]), oracle.row_partial(ref["H"][:, i * w:(i + 1) * w],
                                                      synth.row_shard(d["W2"], i, W.n_shards).f32),
                     "f32", f"P_{i}")
    assert_close(host(Y), ref["Y"], "f32", "Y")


def test_tiny_mlp_f32_forward_with_bias():
    note("tiny fp32 MLP forward + bias")
    W = synth.WORKLOADS["tiny_mlp_f32"]
    d = synth.make_mlp_inputs(W.tokens, W.h, W.ffn, "f32", seed=W.seed, with_bias=True)
    _, _, Y = _forward_gelu(d, W.n_shards, "f32", bias=True)
    ref = oracle.mlp_gelu(d["X"].f32, d["W1"].f32, d["W2"].f32, d["b1"].f32[0], d["b2"].f32[0])
    assert_close(host(Y), ref["Y"], "f32", "Y with biases")


def _backward(d, n, dtype, act, with_bias=False):
    """Per-shard backward on the GPU; dX summed with tp_shard_sum."""
    T_, h = d["X"].shape
    X, dY = dev(d["X"]), dev(d["dY"])
    k1, k2 = ("W1", "W2") if act == "gelu" else ("Wg", "Wd")
    W1s, W2s = _shards(d, n, k1, k2)
    Wus = [synth.column_shard(d["Wu"], i, n) for i in range(n)] if act == "swiglu" else None
    outs = []
    for i in range(n):
        Ni = W1s[i].shape[1]
        o = {"dW1": empty((h, Ni), "f32"), "dW2": empty((Ni, h), "f32"),
             "dX": empty((T_, h), "f32")}
        kw = {}
        if act == "swiglu":
            o["dWu"] = empty((h, Ni), "f32")
            kw = dict(Wup=dev(Wus[i]), dWup=o["dWu"])
        elif with_bias:
            o["db1"] = empty((1, Ni), "f32")
            kw = dict(b1=dev(synth.column_shard(d["b1"], i, n))[0], db1=o["db1"][0])
        tp.tp_mlp_shard_backward(X, dev(W1s[i]), dev(W2s[i]), dY, o["dW1"], o["dW2"], o["dX"],
                                 act=act, **kw)
        outs.append(o)
    dX = empty((T_, h), "f32")
    tp.tp_shard_sum([o["dX"] for o in outs], dX)
    torch().cuda.synchronize()
    return outs, dX


@pytest.mark.parametrize("with_bias", [False, True])
def test_tiny_mlp_f32_backward(with_bias):
    note(f"tiny fp32 MLP backward bias={with_bias}")
    W = synth.WORKLOADS["tiny_mlp_f32"]
    d = synth.make_mlp_inputs(W.tokens, W.h, W.ffn, "f32", seed=W.seed, with_dy=True,
                              with_bias=with_bias)
    outs, dX = _backward(d, W.n_shards, "f32", "gelu", with_bias)
    ref = oracle.mlp_gelu_backward(d["X"].f32, d["W1"].f32, d["W2"].f32, d["dY"].f32,
                                   d["b1"].f32[0] if with_bias else None)
    w = W.ffn_shard
    for i, o in enumerate(outs):
        assert_close(host(o["dW1"]), ref["dW1"][:, i * w:(i + 1) * w], "f32", f"dW1_{i}")
        assert_close(host(o["dW2"]), ref["dW2"][i * w:(i + 1) * w], "f32", f"dW2_{i}")
        if with_bias:
            assert_close(host(o["db1"])[0], ref["db1"][i * w:(i + 1) * w], "f32", f"db1_{i}")
    assert_close(host(dX), ref["dX"], "f32", "dX")


# ---------------------------------------------------------------- medium bf16, ragged tails
@pytest.mark.parametrize("T_,h,ffn,n", [(300, 264, 1056, 2), (77, 128, 512, 4), (1030, 512, 2048, 1)])
def test_mlp_gelu_bf16_medium(T_, h, ffn, n):
    note(f"bf16 MLP GELU fwd {T_}x{h}x{ffn} n={n}")
    d = synth.make_mlp_inputs(T_, h, ffn, "bf16", seed=1, with_bias=True)
    Hs, Ps, Y = _forward_gelu(d, n, "bf16", bias=True)
    ref = oracle.mlp_gelu(d["X"].f32, d["W1"].f32, d["W2"].f32, d["b1"].f32[0], d["b2"].f32[0])
    w = ffn // n
    for i in range(n):
        assert_close(host(Hs[i]), ref["H"][:, i * w:(i + 1) * w], "bf16", f"H_{i}")
    assert_close(host(Y), ref["Y"], "bf16", "Y")


@pytest.mark.parametrize("T_,h,ffn,n", [(300, 264, 1056, 2), (1030, 512, 1024, 1),
                                        # token count % 64 == 0: every GEMM on the LDS-DMA kernel
                                        (1024, 1024, 2048, 2),
                                        # db1: 64 row splits of 65 rows, ragged last split
                                        (4160, 256, 512, 1),
                                        # weight gradients [512 x 1024]: 32 tiles, 4 K-range
                                        # splits added in order from the dead dH scratch
                                        (4096, 512, 1024, 1),
                                        # ragged [264 x 520] weight gradients, 8 splits
                                        (8192, 264, 520, 1),
                                        # dW1 and dW2 of one shape [512 x 512]: one launch,
                                        # 4 K-range splits each, one launch adds both
                                        (4096, 512, 512, 1),
                                        # the GPT-2-medium shard's shapes (h 1024, ffn 1024)
                                        (8192, 1024, 1024, 1),
                                        # ragged [1032 x 1032] weight gradients in one launch,
                                        # 2 K-range splits each
                                        (8192, 1032, 1032, 1)])
def test_mlp_gelu_bf16_backward_medium(T_, h, ffn, n):
    note(f"bf16 MLP GELU bwd {T_}x{h}x{ffn} n={n}")
    d = synth.make_mlp_inputs(T_, h, ffn, "bf16", seed=2, with_dy=True, with_bias=True)
    outs, dX = _backward(d, n, "bf16", "gelu", with_bias=True)
    ref = oracle.mlp_gelu_backward(d["X"].f32, d["W1"].f32, d["W2"].f32, d["dY"].f32,
                                   d["b1"].f32[0])
    w = ffn // n
    for i, o in enumerate(outs):
        assert_close(host(o["dW1"]), ref["dW1"][:, i * w:(i + 1) * w], "bf16", f"dW1_{i}")
        assert_close(host(o["dW2"]), ref["dW2"][i * w:(i + 1) * w], "bf16", f"dW2_{i}")
        assert_close(host(o["db1"])[0], ref["db1"][i * w:(i + 1) * w], "bf16", f"db1_{i}")
    assert_close(host(dX), ref["dX"], "bf16", "dX")


# the last three take the 64-deep dual GEMM with ragged token and ffn edges:
# 128 x 128 output tiles only, 256 x 128 ones only, and 15 column-tiles of
# 256 x 128 followed by 128 x 128 ones
@pytest.mark.parametrize("T_,h,ffn,n", [(300, 264, 1056, 2), (520, 256, 2048, 1), (1024, 1024, 2048, 2),
                                        (1100, 256, 2048, 1), (2100, 512, 2064, 1), (4200, 256, 2056, 1),
                                        # the K-concatenated dX [3976 x 4104]: 13 of its 17 column-tiles
                                        # on 256 x 256 tiles, the rest on 128 x 128 ones
                                        (3976, 4104, 512, 1)])
def test_mlp_swiglu_bf16_medium(T_, h, ffn, n):
    note(f"bf16 SwiGLU fwd+bwd {T_}x{h}x{ffn} n={n}")
    d = synth.make_swiglu_inputs(T_, h, ffn, "bf16", seed=3, with_dy=True)
    X = dev(d["X"])
    w = ffn // n
    ref = oracle.mlp_swiglu(d["X"].f32, d["Wg"].f32, d["Wu"].f32, d["Wd"].f32)
    Ps = []
    for i in range(n):
        H = empty((T_, w), "bf16")
        tp.tp_col_linear_gelu(X, dev(synth.column_shard(d["Wg"], i, n)), H, act="swiglu",
                              Wup=dev(synth.column_shard(d["Wu"], i, n)))
        P = empty((T_, h), "f32")
        tp.tp_row_linear_partial(H, dev(synth.row_shard(d["Wd"], i, n)), P)
        torch().cuda.synchronize()
        assert_close(host(H), ref["H"][:, i * w:(i + 1) * w], "bf16", f"H_{i}")
        Ps.append(P)
    Y = empty((T_, h), "f32")
    tp.tp_shard_sum(Ps, Y)
    torch().cuda.synchronize()
    assert_close(host(Y), ref["Y"], "bf16", "Y")

    outs, dX = _backward(d, n, "bf16", "swiglu")
    g = oracle.mlp_swiglu_backward(d["X"].f32, d["Wg"].f32, d["Wu"].f32, d["Wd"].f32, d["dY"].f32)
    for i, o in enumerate(outs):
        assert_close(host(o["dW1"]), g["dWg"][:, i * w:(i + 1) * w], "bf16", f"dWg_{i}")
        assert_close(host(o["dWu"]), g["dWu"][:, i * w:(i + 1) * w], "bf16", f"dWu_{i}")
        assert_close(host(o["dW2"]), g["dWd"][i * w:(i + 1) * w], "bf16", f"dWd_{i}")
    assert_close(host(dX), g["dX"], "bf16", "dX")


# ---------------------------------------------------------------- full-size workloads
def _rows(T_, k=48, seed=0):
    rng = np.random.default_rng(seed)
    r = np.unique(np.concatenate([[0, T_ - 1], rng.integers(0, T_, k)]))
    return r


def test_gpt2_medium_mlp_full_size_sampled():
    """b=8, s=1024, h=1024, ffn=4096, N=4: all shards + shard sum as benchmarked."""
    W = synth.WORKLOADS["gpt2m_mlp_bf16"]
    note("gpt2-medium MLP full size")
    d = synth.make_mlp_inputs(W.tokens, W.h, W.ffn, "bf16", seed=W.seed)
    Hs, Ps, Y = _forward_gelu(d, W.n_shards, "bf16")
    rows = _rows(W.tokens)
    ref = oracle.mlp_gelu(d["X"].f32[rows], d["W1"].f32, d["W2"].f32)
    w = W.ffn_shard
    for i in range(W.n_shards):
        Hi = host(Hs[i][torch().from_numpy(rows).cuda()])
        assert_close(Hi, ref["H"][:, i * w:(i + 1) * w], "bf16", f"H_{i}")
        Pi = host(Ps[i][torch().from_numpy(rows).cuda()])
        Pref = oracle.row_partial(ref["H"][:, i * w:(i + 1) * w], synth.row_shard(d["W2"], i, W.n_shards).f32)
        assert_close(Pi, Pref, "bf16", f"P_{i}")
    assert_close(host(Y[torch().from_numpy(rows).cuda()]), ref["Y"], "bf16", "Y")


def test_llama_swiglu_full_size_sampled():
    """T=8192, h=4096, ffn=14336, N=4, shard 0 forward + backward."""
    W = synth.WORKLOADS["llama_swiglu_bf16"]
    note("llama SwiGLU full size shard 0")
    T = torch()
    d = synth.make_swiglu_inputs(W.tokens, W.h, W.ffn, "bf16", seed=W.seed, with_dy=True)
    n, i = W.n_shards, 0
    Wg, Wu, Wd = (synth.column_shard(d["Wg"], i, n), synth.column_shard(d["Wu"], i, n),
                  synth.row_shard(d["Wd"], i, n))
    X, dY = dev(d["X"]), dev(d["dY"])
    Ni = Wg.shape[1]
    H = empty((W.tokens, Ni), "bf16")
    P = empty((W.tokens, W.h), "f32")
    Wgd, Wud, Wdd = dev(Wg), dev(Wu), dev(Wd)
    tp.tp_col_linear_gelu(X, Wgd, H, act="swiglu", Wup=Wud)
    tp.tp_row_linear_partial(H, Wdd, P)
    dWg, dWu = empty((W.h, Ni), "f32"), empty((W.h, Ni), "f32")
    dWd, dXi = empty((Ni, W.h), "f32"), empty((W.tokens, W.h), "f32")
    tp.tp_mlp_shard_backward(X, Wgd, Wdd, dY, dWg, dWd, dXi, act="swiglu", Wup=Wud, dWup=dWu)
    T.cuda.synchronize()

    rows = _rows(W.tokens, k=24)
    ri = T.from_numpy(rows).cuda()
    f = oracle.mlp_swiglu(d["X"].f32[rows], Wg.f32, Wu.f32, Wd.f32)
    assert_close(host(H[ri]), f["H"], "bf16", "H_0 rows")
    assert_close(host(P[ri]), f["Y"], "bf16", "P_0 rows")
    gx = oracle.mlp_swiglu_backward(d["X"].f32[rows], Wg.f32, Wu.f32, Wd.f32, d["dY"].f32[rows])
    assert_close(host(dXi[ri]), gx["dX"], "bf16", "dX_0 rows")
    cols = np.unique(np.concatenate([[0, Ni - 1], np.random.default_rng(1).integers(0, Ni, 30)]))
    ci = T.from_numpy(cols).cuda()
    gw = oracle.mlp_swiglu_backward(d["X"].f32, Wg.f32[:, cols], Wu.f32[:, cols], Wd.f32[cols], d["dY"].f32)
    assert_close(host(dWg[:, ci]), gw["dWg"], "bf16", "dWg_0 cols")
    assert_close(host(dWu[:, ci]), gw["dWu"], "bf16", "dWu_0 cols")
    assert_close(host(dWd[ci]), gw["dWd"], "bf16", "dWd_0 rows")


@pytest.mark.parametrize("h,ffn", [(512, 1024), (512, 512)])
def test_mlp_backward_repeats_bitwise(h, ffn):
    # split-K weight gradients (4 splits here; the [512 x 512] pair in one
    # launch) and db1 add their partials in a fixed order: repeated calls give
    # identical bits, whatever the workspace held before
    note(f"bf16 MLP GELU bwd repeatability 4096x{h}x{ffn}")
    T = torch()
    d = synth.make_mlp_inputs(4096, h, ffn, "bf16", seed=5, with_dy=True, with_bias=True)
    X, W1, W2, dY, b1 = dev(d["X"]), dev(d["W1"]), dev(d["W2"]), dev(d["dY"]), dev(d["b1"])[0]
    nbytes = tp.tp_mlp_shard_backward_workspace(tp.TP_BF16, tp.TP_ACT_GELU_ERF, 4096, ffn)
    ws = T.empty((nbytes,), dtype=T.uint8, device="cuda:0")
    runs = []
    for it in range(3):
        ws.fill_(it * 85)
        o = {"dW1": empty((h, ffn), "f32"), "dW2": empty((ffn, h), "f32"),
             "dX": empty((4096, h), "f32"), "db1": empty((1, ffn), "f32")}
        tp.tp_mlp_shard_backward(X, W1, W2, dY, o["dW1"], o["dW2"], o["dX"], act="gelu", b1=b1,
                                 db1=o["db1"][0], ws=ws)
        T.cuda.synchronize()
        runs.append({k: v.clone() for k, v in o.items()})
    for r in runs[1:]:
        for k in r:
            assert T.equal(r[k], runs[0][k]), k


@pytest.mark.parametrize("act,h,ffn", [("gelu", 512, 512), ("swiglu", 256, 512)])
def test_mlp_backward_graph_replays(act, h, ffn):
    # a captured backward call (recompute, paired split-K weight gradients
    # and their sums, db1, dX) replays to the eager call's bits, with eager
    # calls and workspace clobbering in between
    note(f"bf16 MLP {act} bwd graph replay 4096x{h}x{ffn}")
    T = torch()
    if act == "gelu":
        d = synth.make_mlp_inputs(4096, h, ffn, "bf16", seed=6, with_dy=True, with_bias=True)
        W1, W2 = dev(d["W1"]), dev(d["W2"])
        kw = dict(b1=dev(d["b1"])[0])
    else:
        d = synth.make_swiglu_inputs(4096, h, ffn, "bf16", seed=6, with_dy=True)
        W1, W2 = dev(d["Wg"]), dev(d["Wd"])
        kw = dict(Wup=dev(d["Wu"]))
    X, dY = dev(d["X"]), dev(d["dY"])
    code = tp.TP_ACT_GELU_ERF if act == "gelu" else tp.TP_ACT_SWIGLU
    ws = T.empty((tp.tp_mlp_shard_backward_workspace(tp.TP_BF16, code, 4096, ffn),), dtype=T.uint8, device="cuda:0")
    o = {"dW1": empty((h, ffn), "f32"), "dW2": empty((ffn, h), "f32"), "dX": empty((4096, h), "f32")}
    if act == "gelu":
        o["db1"] = empty((1, ffn), "f32")
        kw["db1"] = o["db1"][0]
    else:
        o["dWu"] = empty((h, ffn), "f32")
        kw["dWup"] = o["dWu"]

    def call():
        tp.tp_mlp_shard_backward(X, W1, W2, dY, o["dW1"], o["dW2"], o["dX"], act=act, ws=ws, **kw)

    call()
    T.cuda.synchronize()
    ref = {k: v.clone() for k, v in o.items()}
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g):
        call()
    T.cuda.synchronize()
    for it in range(3):
        for v in o.values():
            v.fill_(float("nan"))
        ws.fill_(it * 37)
        T.cuda.synchronize()
        g.replay()
        T.cuda.synchronize()
        for k in o:
            assert T.equal(o[k], ref[k]), (it, k)
        call()
        T.cuda.synchronize()
        for k in o:
            assert T.equal(o[k], ref[k]), (it, "eager", k)
