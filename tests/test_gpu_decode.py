"""GPU parity of the decode (M <= 16) weight-streaming GEMV path."""
import numpy as np
import pytest

import megatron_tensor_transformer_col_amd as tp
import oracle
import synth
from gpu_util import assert_close, dev, empty, host, note, torch

pytestmark = pytest.mark.gpu


def test_decode_mlp_full_size():
    """16 tokens, h=8192, ffn=28672, N=8: all 8 shards + shard sum."""
    W = synth.WORKLOADS["decode_mlp_bf16"]
    note("decode MLP full size")
    d = synth.make_mlp_inputs(W.tokens, W.h, W.ffn, "bf16", seed=W.seed, row_block=1024)
    X = dev(d["X"])
    n, w = W.n_shards, W.ffn_shard
    ref = oracle.mlp_gelu(d["X"].f32, d["W1"].f32, d["W2"].f32)
    Ps = []
    for i in range(n):
        H = empty((W.tokens, w), "bf16")
        tp.tp_col_linear_gelu(X, dev(synth.column_shard(d["W1"], i, n)), H)
        P = empty((W.tokens, W.h), "f32")
        tp.tp_row_linear_partial(H, dev(synth.row_shard(d["W2"], i, n)), P)
        torch().cuda.synchronize()
        assert_close(host(H), ref["H"][:, i * w:(i + 1) * w], "bf16", f"H_{i}")
        Ps.append(P)
    Y = empty((W.tokens, W.h), "f32")
    tp.tp_shard_sum(Ps, Y)
    torch().cuda.synchronize()
    assert_close(host(Y), ref["Y"], "bf16", "Y")


@pytest.mark.parametrize("M", [1, 3, 8, 16])
@pytest.mark.parametrize("K,N", [(64, 136), (1024, 520), (4104, 1032)])
def test_gemv_integer_exact(M, K, N):
    note(f"gemv exact M={M} K={K} N={N}")
    rng = np.random.default_rng(M * 131 + K)
    X = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    Wm = rng.integers(-2, 3, size=(K, N)).astype(np.float32)
    P = empty((M, N), "f32", fill=float("nan"))
    tp.tp_row_linear_partial(dev(synth.Tensor(X, "bf16", synth.round_to_bf16_bits(X))),
                             dev(synth.Tensor(Wm, "bf16", synth.round_to_bf16_bits(Wm))), P)
    torch().cuda.synchronize()
    assert np.array_equal(host(P), (X.astype(np.int64) @ Wm.astype(np.int64)).astype(np.float64))


@pytest.mark.parametrize("M", [1, 7, 16])
def test_gemv_matches_gemm_path_and_oracle(M):
    note(f"gemv vs gemm M={M}")
    d = synth.make_mlp_inputs(M, 2048, 1536, "bf16", seed=M, with_bias=True)
    X, W1 = dev(d["X"]), dev(d["W1"])
    b1 = dev(d["b1"])[0]
    Hv = empty((M, 1536), "bf16")
    tp.tp_col_linear_gelu(X, W1, Hv, bias=b1)
    prev = tp.tp_set_gemv_max_m(0)
    try:
        Hm = empty((M, 1536), "bf16")
        tp.tp_col_linear_gelu(X, W1, Hm, bias=b1)
    finally:
        tp.tp_set_gemv_max_m(prev)
    torch().cuda.synchronize()
    ref = oracle.gelu(oracle.linear(d["X"].f32, d["W1"].f32, d["b1"].f32[0]))
    assert_close(host(Hv), ref, "bf16", "H gemv")
    assert_close(host(Hm), ref, "bf16", "H gemm")


def test_gemv_repeated_calls():
    # split-K partials live in a shared workspace: back-to-back calls must not see stale data
    note("gemv repeated")
    rng = np.random.default_rng(0)
    X = rng.integers(-2, 3, size=(16, 2048)).astype(np.float32)
    Wm = rng.integers(-2, 3, size=(2048, 1024)).astype(np.float32)
    Xd = dev(synth.Tensor(X, "bf16", synth.round_to_bf16_bits(X)))
    Wd = dev(synth.Tensor(Wm, "bf16", synth.round_to_bf16_bits(Wm)))
    exact = (X.astype(np.int64) @ Wm.astype(np.int64)).astype(np.float64)
    for it in range(5):
        P = empty((16, 1024), "f32", fill=float("nan"))
        tp.tp_row_linear_partial(Xd, Wd, P)
        torch().cuda.synchronize()
        assert np.array_equal(host(P), exact), it


def _int_operands(M, K, N, seed):
    rng = np.random.default_rng(seed)
    X = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    Wm = rng.integers(-2, 3, size=(K, N)).astype(np.float32)
    Xd = dev(synth.Tensor(X, "bf16", synth.round_to_bf16_bits(X)))
    Wd = dev(synth.Tensor(Wm, "bf16", synth.round_to_bf16_bits(Wm)))
    return Xd, Wd, (X.astype(np.int64) @ Wm.astype(np.int64)).astype(np.float64)


@pytest.mark.parametrize("fill", [0x00, 0xFF, "random"])
def test_gemv_workspace_contents_do_not_matter(fill):
    # the workspace is never cleared: whatever bytes it holds, every call
    # writes the split-K partials it reads
    note(f"gemv workspace fill {fill}")
    T = torch()
    Xd, Wd, exact = _int_operands(16, 4096, 1024, seed=7)
    nbytes = tp.tp_row_linear_partial_workspace(tp.TP_BF16, 16, 4096, 1024)
    assert nbytes > 0
    ws = T.empty((nbytes,), dtype=T.uint8, device="cuda:0")
    for it in range(3):
        if fill == "random":
            ws.copy_(T.randint(0, 256, (nbytes,), dtype=T.uint8, generator=T.Generator().manual_seed(it)))
        else:
            ws.fill_(fill)
        P = empty((16, 1024), "f32", fill=float("nan"))
        tp.tp_row_linear_partial(Xd, Wd, P, ws=ws)
        torch().cuda.synchronize()
        assert np.array_equal(host(P), exact), it


def test_gemv_graph_replays_share_one_workspace():
    # captured GEMVs replay against one workspace that the column and row
    # GEMVs (different split counts) share, with eager calls in between
    note("gemv graph replay")
    T = torch()
    Xd, W1, ex1 = _int_operands(16, 2048, 1536, seed=11)
    _, W2, _ = _int_operands(16, 1536, 2048, seed=12)
    nbytes = max(tp.tp_col_linear_gelu_workspace(tp.TP_BF16, tp.TP_ACT_NONE, 16, 2048, 1536),
                 tp.tp_row_linear_partial_workspace(tp.TP_BF16, 16, 1536, 2048))
    ws = T.empty((nbytes,), dtype=T.uint8, device="cuda:0")
    H = empty((16, 1536), "bf16")
    P = empty((16, 2048), "f32")

    def step():
        tp.tp_col_linear_gelu(Xd, W1, H, act="none", ws=ws)
        tp.tp_row_linear_partial(H, W2, P, ws=ws)

    step()
    T.cuda.synchronize()
    ref_P = host(P)
    # H holds small integers (|h| <= 2 * 2048), exact in bf16 only where they fit
    assert np.array_equal(host(H), synth.bf16_bits_to_f32(synth.round_to_bf16_bits(ex1)).astype(np.float64))
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g):
        step()
    T.cuda.synchronize()
    for it in range(4):
        H.fill_(float("nan"))
        P.fill_(float("nan"))
        T.cuda.synchronize()
        g.replay()
        T.cuda.synchronize()
        assert np.array_equal(host(P), ref_P), it
        step()
        T.cuda.synchronize()
        assert np.array_equal(host(P), ref_P), it


# ---------------------------------------------------------------- pre-packed decode weights
def _panels_host(Wf, K, N):
    """The panel layout written out on the host from its definition:
    Wp[s][k][c] = W[k][64 s + c] for k < K, 64 s + c < N, zero elsewhere."""
    S, Kp = (N + 63) // 64, (K + 63) // 64 * 64
    out = np.zeros((S, Kp, 64), dtype=np.uint16)
    bits = synth.round_to_bf16_bits(Wf)
    for s in range(S):
        c1 = min(N, 64 * s + 64)
        out[s, :K, :c1 - 64 * s] = bits[:, 64 * s:c1]
    return out


@pytest.mark.parametrize("M,K,N,act,out,bias", [
    (1, 72, 8, "none", "f32", False), (5, 1000, 200, "gelu", "bf16", True), (3, 64, 136, "none", "bf16", False),
    (16, 4104, 1032, "gelu", "bf16", True), (16, 1536, 2048, "none", "f32", False)])
def test_decode_packed_matches_row_major_and_oracle(M, K, N, act, out, bias):
    """Ragged K and N: the pack writes the documented panels, and the GEMV
    over them equals the row-major decode path bit for bit and the oracle
    within the bf16 tolerance."""
    note(f"decode packed M={M} K={K} N={N} act={act} out={out}")
    d = synth.make_mlp_inputs(M, K, N, "bf16", seed=K + N, with_bias=bias)
    X, W = dev(d["X"]), dev(d["W1"])
    b = dev(d["b1"])[0] if bias else None
    Wp = tp.tp_decode_pack_weight(W)
    assert Wp.numel() == tp.tp_decode_packed_weight_bytes(K, N)
    Y0 = empty((M, N), out, fill=float("nan"))
    Y1 = empty((M, N), out, fill=float("nan"))
    if out == "f32":
        assert b is None
        tp.tp_row_linear_partial(X, W, Y0)
    else:
        tp.tp_col_linear_gelu(X, W, Y0, act=act, bias=b)
    tp.tp_decode_linear_packed(X, Wp, Y1, act=act, bias=b)
    torch().cuda.synchronize()
    got = Wp.cpu().numpy().view(np.uint16).reshape((N + 63) // 64, (K + 63) // 64 * 64, 64)
    assert np.array_equal(got, _panels_host(d["W1"].f32, K, N))
    raw = torch().int32 if out == "f32" else torch().int16
    assert torch().equal(Y0.view(raw), Y1.view(raw))
    z = oracle.linear(d["X"].f32, d["W1"].f32, d["b1"].f32[0] if bias else None)
    assert_close(host(Y1), oracle.gelu(z) if act == "gelu" else z, out, "Y packed")


@pytest.mark.parametrize("M,K,N", [(16, 4096, 1024), (7, 2112, 520)])
def test_decode_packed_integer_exact(M, K, N):
    note(f"decode packed exact M={M} K={K} N={N}")
    Xd, Wd, exact = _int_operands(M, K, N, seed=M + K)
    Wp = tp.tp_decode_pack_weight(Wd)
    for it in range(3):  # the shared split-K workspace holds the previous call's partials
        P = empty((M, N), "f32", fill=float("nan"))
        tp.tp_decode_linear_packed(Xd, Wp, P, act="none")
        torch().cuda.synchronize()
        assert np.array_equal(host(P), exact), it


def test_decode_packed_mlp_full_size():
    """The decode MLP at full size (16 tokens, h 8192, ffn 28672, 8 shards)
    on packed weights, as the bench's packed decode row runs it: every shard's
    H_i and the shard sum against the oracle, bit for bit the row-major
    path's results."""
    W = synth.WORKLOADS["decode_mlp_bf16"]
    note("decode MLP packed full size")
    d = synth.make_mlp_inputs(W.tokens, W.h, W.ffn, "bf16", seed=W.seed, row_block=1024)
    X = dev(d["X"])
    n, w = W.n_shards, W.ffn_shard
    ref = oracle.mlp_gelu(d["X"].f32, d["W1"].f32, d["W2"].f32)
    Ps = []
    for i in range(n):
        W1 = dev(synth.column_shard(d["W1"], i, n))
        W2 = dev(synth.row_shard(d["W2"], i, n))
        H, H0 = empty((W.tokens, w), "bf16"), empty((W.tokens, w), "bf16")
        P, P0 = empty((W.tokens, W.h), "f32"), empty((W.tokens, W.h), "f32")
        tp.tp_decode_linear_packed(X, tp.tp_decode_pack_weight(W1), H, act="gelu")
        tp.tp_decode_linear_packed(H, tp.tp_decode_pack_weight(W2), P, act="none")
        tp.tp_col_linear_gelu(X, W1, H0)
        tp.tp_row_linear_partial(H0, W2, P0)
        torch().cuda.synchronize()
        assert torch().equal(H.view(torch().int16), H0.view(torch().int16)), i
        assert torch().equal(P.view(torch().int32), P0.view(torch().int32)), i
        assert_close(host(H), ref["H"][:, i * w:(i + 1) * w], "bf16", f"H_{i}")
        Ps.append(P)
    Y = empty((W.tokens, W.h), "f32")
    tp.tp_shard_sum(Ps, Y)
    torch().cuda.synchronize()
    assert_close(host(Y), ref["Y"], "bf16", "Y")
