"""CPU checks of the C ABI: the library loads, exports every symbol that
include/tpcol.h declares, and rejects bad arguments on the host before any
launch.  No GPU compute is issued from here."""
import ctypes
import os
import re

import pytest

import megatron_tensor_transformer_col_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpcol.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = tp.lib()
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), f"{n} declared in tpcol.h but not exported"
    assert set(names) == set(tp.EXPORTED_SYMBOLS)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = tp.tp_status_string(code)
        assert s and s != "unknown status"
    assert tp.tp_status_string(42) == "unknown status"


@pytest.mark.parametrize("h,ffn,heads,n", [(128, 512, 8, 2), (4096, 14336, 32, 4), (1024, 4096, 16, 4),
                                           (8192, 28672, 64, 8), (4096, 14336, 30, 4),
                                           (4096, 14336, 32, 3), (100, 512, 8, 2), (128, 513, 8, 2),
                                           (128, 512, 0, 2), (128, 512, 8, 0)])
def test_check_split_matches_divisibility(h, ffn, heads, n):
    ok = n >= 1 and ffn % n == 0 and (heads == 0 or (h % heads == 0 and heads % n == 0))
    assert (tp.tp_check_split(h, ffn, heads, n) == 0) == ok


@pytest.mark.parametrize("env,expect", [("4", 4), ("0", 0), ("17", 16), ("x", 16)])
def test_gemv_threshold_environment(env, expect):
    # TPCOL_GEMV_MAX_M sets the initial threshold when the library loads
    import subprocess
    import sys
    code = ("import megatron_tensor_transformer_col_amd as tp; "
            "print(tp.tp_set_gemv_max_m(16))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, TPCOL_GEMV_MAX_M=env))
    assert r.returncode == 0, r.stderr[-2000:]
    assert int(r.stdout.split()[-1]) == expect


def test_gemv_threshold_option():
    prev = tp.tp_set_gemv_max_m(8)
    try:
        assert tp.tp_set_gemv_max_m(16) == 8
        with pytest.raises(tp.TpError):
            tp.tp_set_gemv_max_m(17)
        with pytest.raises(tp.TpError):
            tp.tp_set_gemv_max_m(-1)
    finally:
        tp.tp_set_gemv_max_m(prev)


def test_workspace_sizes():
    # attention: QKV [T x 3 hl d] + O [T x hl d] bf16 + row statistic [b hl s] fp32,
    # 256-byte aligned regions
    T = 4 * 2048
    assert tp.tp_attn_heads_shard_workspace(1, 4, 2048, 8, 128) == T * 3 * 1024 * 2 + T * 1024 * 2 + T * 8 * 4
    assert tp.tp_attn_gqa_shard_workspace(1, 4, 2048, 8, 2, 128) == T * 12 * 128 * 2 + T * 1024 * 2 + T * 8 * 4
    # attention backward: dO [T x hl d] bf16 + D [b hl s] fp32 + dQKV bf16, plus for
    # grouped-query shards with few (sequence, kv head, 128-key block) pairs the
    # fp32 dK/dV partials of the 4 head splits [4][T][kvl][2][d]
    assert tp.tp_attn_shard_backward_workspace(1, 4, 2048, 8, 8, 128) == T * 1024 * 2 + T * 8 * 4 + T * 24 * 128 * 2
    assert tp.tp_attn_shard_backward_workspace(1, 4, 2048, 8, 2, 128) == (
        T * 1024 * 2 + T * 8 * 4 + T * 12 * 128 * 2 + 4 * T * 2 * 2 * 128 * 4)
    # fp32 / other head dims (general kernels): element size 4, no head-split partials
    t = 2 * 10
    r = lambda x: (x + 255) // 256 * 256
    assert tp.tp_attn_heads_shard_workspace(0, 2, 10, 4, 16) == r(t * 12 * 16 * 4) + r(t * 64 * 4) + r(t * 4 * 4)
    assert tp.tp_attn_shard_backward_workspace(0, 2, 10, 4, 4, 16) == r(t * 64 * 4) + r(t * 4 * 4) + r(t * 12 * 16 * 4)
    assert tp.tp_attn_shard_backward_workspace(1, 4, 2048, 8, 2, 64) == T * 512 * 2 + T * 8 * 4 + T * 12 * 64 * 2
    assert tp.tp_attn_heads_shard_workspace(7, 2, 10, 4, 16) == 0  # unknown dtype
    # backward: dH, a dH-sized partial region, H, dZ and 64 fp32 rows of db1
    # column-sum partials (GELU) /
    # dH, H, [dZg | dZu] (SwiGLU, no bias)
    assert tp.tp_mlp_shard_backward_workspace(1, 1, 8192, 1024) == 4 * 8192 * 1024 * 2 + 64 * 1024 * 4
    assert tp.tp_mlp_shard_backward_workspace(1, 2, 8192, 3584) == 4 * 8192 * 3584 * 2
    assert tp.tp_mlp_shard_backward_workspace(0, 1, 32, 256) == 4 * 32 * 256 * 4 + 64 * 256 * 4
    # db1 partials: one row per 128-row tile of dZ once that exceeds 64 rows
    assert tp.tp_mlp_shard_backward_workspace(1, 1, 16384, 1024) == 4 * 16384 * 1024 * 2 + 128 * 1024 * 4
    # large-M linear calls need no workspace; the decode path needs split-K partials
    assert tp.tp_col_linear_gelu_workspace(1, 1, 8192, 1024, 1024) == 0
    assert tp.tp_col_linear_gelu_workspace(1, 1, 16, 8192, 3584) > 0
    assert tp.tp_col_linear_gelu_workspace(0, 1, 16, 8192, 3584) == 0   # fp32 has no GEMV path
    assert tp.tp_row_linear_partial_workspace(1, 16, 3584, 8192) > 0


# ---------------------------------------------------------------- host validation
# Fake device addresses are never dereferenced: each case must be rejected by
# the host-side checks.  Skipped where a GPU is visible so that a validation
# bug can never turn into a launch on bogus pointers.
def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


host_only = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer validation runs on CPU hosts only")

A = 1 << 20          # 16-byte aligned fake address
MIS = A + 2          # misaligned
V = ctypes.c_void_p


@host_only
@pytest.mark.parametrize("case,expect", [
    ("bad_dtype", -4), ("bad_act", -1), ("null_x", -1), ("misaligned_w", -3), ("ld_small", -2),
    ("odd_width", -3), ("swiglu_no_up", -1), ("swiglu_bias", -1), ("gemv_no_ws", -5),
    ("neg_m", -2),
])
def test_col_linear_validation(case, expect):
    lib = tp.lib()
    a = dict(dt=1, act=1, M=64, K=256, N=512, X=A, ldx=256, W=A, ldw=512, Wu=None, ldwu=0,
             bias=None, H=A, ldh=512, ws=None, nws=0)
    if case == "bad_dtype": a["dt"] = 7
    if case == "bad_act": a["act"] = 9
    if case == "null_x": a["X"] = None
    if case == "misaligned_w": a["W"] = MIS
    if case == "ld_small": a["ldh"] = 256
    if case == "odd_width": a.update(N=500, ldw=504, ldh=504)
    if case == "swiglu_no_up": a["act"] = 2
    if case == "swiglu_bias": a.update(act=2, Wu=A, ldwu=512, bias=A)
    if case == "gemv_no_ws": a.update(M=4, K=4096, ldx=4096)
    if case == "neg_m": a["M"] = -1
    st = lib.tp_col_linear_gelu(a["dt"], a["act"], a["M"], a["K"], a["N"], a["X"], a["ldx"], a["W"],
                                a["ldw"], a["Wu"], a["ldwu"], a["bias"], a["H"], a["ldh"], a["ws"],
                                a["nws"], None)
    assert st == expect, tp.tp_last_error()
    assert tp.tp_last_error()


@host_only
@pytest.mark.parametrize("case,expect", [
    ("bad_dtype", -4), ("bad_act", -1), ("null_x", -1), ("misaligned_w", -3), ("ld_small", -2),
    ("odd_width", -3), ("swiglu_no_up", -1), ("swiglu_bias", -1), ("neg_m", -2),
])
def test_col_linear_noalloc_validation(case, expect):
    """The allocation-free variant validates like tp_col_linear_gelu."""
    lib = tp.lib()
    a = dict(dt=1, act=1, M=64, K=256, N=512, X=A, ldx=256, W=A, ldw=512, Wu=None, ldwu=0,
             bias=None, H=A, ldh=512)
    if case == "bad_dtype": a["dt"] = 7
    if case == "bad_act": a["act"] = 9
    if case == "null_x": a["X"] = None
    if case == "misaligned_w": a["W"] = MIS
    if case == "ld_small": a["ldh"] = 256
    if case == "odd_width": a.update(N=500, ldw=504, ldh=504)
    if case == "swiglu_no_up": a["act"] = 2
    if case == "swiglu_bias": a.update(act=2, Wu=A, ldwu=512, bias=A)
    if case == "neg_m": a["M"] = -1
    st = lib.tp_col_linear_gelu_noalloc(a["dt"], a["act"], a["M"], a["K"], a["N"], a["X"], a["ldx"], a["W"],
                                        a["ldw"], a["Wu"], a["ldwu"], a["bias"], a["H"], a["ldh"], None)
    assert st == expect, tp.tp_last_error()
    assert tp.tp_last_error()


@host_only
def test_attention_validation():
    lib = tp.lib()
    f = lib.tp_attn_heads_shard
    # unknown dtype
    assert f(5, 4, 2048, 4096, 8, 128, 1, A, 4096, A, 3072, A, 4096, A, 4096, A, 1 << 30, None) == -4
    # head dim beyond 256 (fp32 and other head dims run the general kernels)
    assert f(1, 4, 2048, 4096, 8, 300, 1, A, 4096, A, 7200, A, 4096, A, 4096, A, 1 << 30, None) == -2
    # fp32, 1 head of 3: the 12-byte O rows are not 16-byte multiples
    assert f(0, 1, 16, 64, 1, 3, 1, A, 64, A, 12, A, 64, A, 64, A, 1 << 30, None) == -3
    # fp32 head dim 16 (the pages' example shape): workspace too small
    assert f(0, 2, 10, 128, 4, 16, 1, A, 128, A, 192, A, 128, A, 128, A, 1024, None) == -5
    # workspace too small
    assert f(1, 4, 2048, 4096, 8, 128, 1, A, 4096, A, 3072, A, 4096, A, 4096, A, 1024, None) == -5
    # Wqkv narrower than 3 * heads_local * d
    assert f(1, 4, 2048, 4096, 8, 128, 1, A, 4096, A, 2048, A, 4096, A, 4096, A, 1 << 30, None) == -2


@host_only
def test_gqa_attention_validation():
    lib = tp.lib()
    g = lib.tp_attn_gqa_shard
    # 8 query heads, 2 kv heads: Wqkv is (8 + 2*2)*128 = 1536 wide
    assert g(1, 4, 2048, 4096, 8, 2, 128, 1, A, 4096, A, 1536, A, 4096, A, 4096, A, 1024, None) == -5
    # heads_local not a multiple of kv_heads_local
    assert g(1, 4, 2048, 4096, 8, 3, 128, 1, A, 4096, A, 1536, A, 4096, A, 4096, A, 1 << 30, None) == -2
    assert g(1, 4, 2048, 4096, 8, 0, 128, 1, A, 4096, A, 1536, A, 4096, A, 4096, A, 1 << 30, None) == -2
    # Wqkv narrower than (hl + 2 kvl) d
    assert g(1, 4, 2048, 4096, 8, 2, 128, 1, A, 4096, A, 1024, A, 4096, A, 4096, A, 1 << 30, None) == -2
    # workspace: QKV block (hl + 2 kvl) d wide, then O
    T = 4 * 2048
    assert tp.tp_attn_gqa_shard_workspace(1, 4, 2048, 8, 2, 128) == T * 1536 * 2 + T * 1024 * 2 + T * 8 * 4
    assert tp.tp_attn_gqa_shard_workspace(1, 4, 2048, 8, 8, 128) == tp.tp_attn_heads_shard_workspace(1, 4, 2048, 8, 128)


@host_only
def test_reduce_scatter_layernorm_validation():
    lib = tp.lib()
    f = lib.tp_shard_reduce_scatter_layernorm
    arr = (V * 2)(A, A)
    ok = dict(dt=1, rows=2048, N=1024, n=2, p=arr, ldp=1024, bias=None, res=None, ldr=0, g=A, b=A,
              eps=1e-5, ys=None, ldys=0, Y=A, ldy=1024)
    def call(**kw):
        a = dict(ok, **kw)
        return f(a["dt"], a["rows"], a["N"], a["n"], a["p"], a["ldp"], a["bias"], a["res"], a["ldr"],
                 a["g"], a["b"], a["eps"], a["ys"], a["ldys"], a["Y"], a["ldy"], None)
    assert call(g=None) == -1                        # gamma required
    assert call(eps=-1.0) == -1                      # negative eps
    assert call(N=16384, ldp=16384, ldy=16384) == -2  # hidden size beyond the register row
    assert call(n=0) == -1
    assert call(p=(V * 2)(A, None)) == -1            # NULL partial
    assert call(dt=5) == -4
    assert call(N=1028, ldp=1028, ldy=1028) == -3    # bf16 row of 1028 is not 16-byte aligned
    assert call(rows=0) == 0                         # nothing to do


@host_only
def test_vocab_cross_entropy_validation():
    lib = tp.lib()
    assert lib.tp_vocab_ce_shard_stats(1, 64, 32064, A, 32064, None, None) == -1     # stats NULL
    assert lib.tp_vocab_ce_shard_stats(1, 64, 32064, A, 32000, A, None) == -2       # ld < width
    assert lib.tp_vocab_ce_shard_stats(1, 64, 17, A + 1, 17, A, None) == -3          # bf16 logits odd address
    assert lib.tp_vocab_ce_shard_stats(1, 64, 32064, A, 32064, MIS, None) == -3     # stats misaligned
    assert lib.tp_vocab_ce_shard_stats(1, 0, 32064, None, 32064, None, None) == 0   # empty
    arr = (V * 2)(A, None)
    assert lib.tp_vocab_ce_lse(64, 2, arr, A, None) == -1                           # NULL stats
    assert lib.tp_vocab_ce_lse(64, 0, arr, A, None) == -1
    assert lib.tp_vocab_ce_shard_loss(1, 64, 32064, -1, A, 32064, A, A, None, A, None) == -2  # vocab_start < 0
    assert lib.tp_vocab_ce_shard_loss(1, 64, 32064, 0, A, 32064, A, A, None, None, None) == -1  # no output
    assert lib.tp_vocab_ce_total(2, (V * 2)(A, None), A, None) == -1


@host_only
def test_shard_sum_and_backward_validation():
    lib = tp.lib()
    arr = (V * 3)(A, A, None)
    assert lib.tp_shard_sum(0, 16, 64, 3, arr, 64, None, A, 64, None) == -1     # NULL partial
    assert lib.tp_shard_sum(0, 16, 64, 0, arr, 64, None, A, 64, None) == -1     # n = 0
    assert lib.tp_shard_sum(0, 16, 64, 65, arr, 64, None, A, 64, None) == -1    # n > 64
    assert lib.tp_shard_sum(1, 16, 68, 2, arr, 68, None, A, 68, None) == -3     # bf16 width 68
    bw = lib.tp_mlp_shard_backward
    common = (A, 256, A, 128, None, 0, None, A, 256, A, 256, A, None, A, None, A, 256)
    assert bw(1, 0, 64, 256, 128, *common, A, 1 << 30, None) == -1               # act NONE
    assert bw(1, 1, 64, 256, 128, *common, A, 100, None) == -5                   # tiny workspace
    assert bw(1, 2, 64, 256, 128, *common, A, 1 << 30, None) == -1               # SwiGLU w/o Wup


@host_only
def test_attention_backward_validation():
    lib = tp.lib()
    g = lib.tp_attn_shard_backward
    T = 4 * 2048
    fw = tp.tp_attn_gqa_shard_workspace(1, 4, 2048, 8, 2, 128)
    bw = tp.tp_attn_shard_backward_workspace(1, 4, 2048, 8, 2, 128)

    def call(dt=1, hl=8, kvl=2, d=128, X=A, dWqkv=A, dWo=A, dX=A, fws=A, fwn=fw, ws=A, wsn=bw, ldwqkv=1536):
        return g(dt, 4, 2048, 4096, hl, kvl, d, 1, X, 4096, A, ldwqkv, A, 4096, A, 4096, fws, fwn, dWqkv, dWo, dX,
                 4096, ws, wsn, None)

    assert call(dt=3) == -4                        # unknown dtype
    assert call(kvl=3) == -2                       # 8 query heads do not group over 3 kv heads
    assert call(d=300) == -2                       # head dim 1..256
    assert call(ldwqkv=1024) == -2                 # ld < (hl + 2 kvl) d
    assert call(X=None) == -1
    assert call(dWo=None) == -1
    assert call(dWqkv=MIS) == -3
    assert call(fws=None) == -5                    # the forward's workspace is required
    assert call(fwn=fw - 256) == -5
    assert call(wsn=bw - 1) == -5
    assert call(ws=A + 16) == -3                   # workspace not 256-byte aligned


def test_decode_packed_sizes():
    """Panel bytes: ceil(N / 64) panels x (K rounded up to 64) rows x 64 bf16;
    the packed GEMV's workspace is the row-major decode path's."""
    assert tp.tp_decode_packed_weight_bytes(8192, 3584) == 56 * 8192 * 64 * 2
    assert tp.tp_decode_packed_weight_bytes(1000, 200) == 4 * 1024 * 64 * 2
    assert tp.tp_decode_packed_weight_bytes(0, 64) == 0
    for K, N in [(8192, 3584), (3584, 8192), (1000, 200)]:
        assert tp.tp_decode_linear_packed_workspace(16, K, N) == tp.tp_row_linear_partial_workspace(1, 16, K, N)
    assert tp.tp_decode_linear_packed_workspace(17, 8192, 3584) == 0


@host_only
@pytest.mark.parametrize("case,expect", [
    ("fp32", -4), ("null_wp", -1), ("misaligned_wp", -3), ("small_wp", -2), ("odd_width", -3), ("zero_k", -2)])
def test_decode_pack_validation(case, expect):
    lib = tp.lib()
    a = dict(dt=1, K=1000, N=200, W=A, ldw=200, Wp=A, nwp=tp.tp_decode_packed_weight_bytes(1000, 200))
    if case == "fp32": a["dt"] = 0
    if case == "null_wp": a["Wp"] = None
    if case == "misaligned_wp": a["Wp"] = MIS
    if case == "small_wp": a["nwp"] -= 16
    if case == "odd_width": a.update(N=196, ldw=200)
    if case == "zero_k": a["K"] = 0
    st = lib.tp_decode_pack_weight(a["dt"], a["K"], a["N"], a["W"], a["ldw"], a["Wp"], a["nwp"], None)
    assert st == expect, tp.tp_last_error()
    assert tp.tp_last_error()


@host_only
@pytest.mark.parametrize("case,expect", [
    ("bad_act", -1), ("swiglu", -1), ("bad_out", -4), ("f32_gelu", -1), ("m17", -2), ("null_x", -1),
    ("null_wp", -1), ("misaligned_wp", -3), ("small_wp", -2), ("no_ws", -5), ("misaligned_ws", -3),
    ("ld_small", -2)])
def test_decode_linear_packed_validation(case, expect):
    lib = tp.lib()
    K, N = 4096, 1024
    a = dict(act=1, out=1, M=16, X=A, ldx=K, Wp=A, nwp=tp.tp_decode_packed_weight_bytes(K, N), bias=None,
             Y=A, ldy=N, ws=A, nws=tp.tp_decode_linear_packed_workspace(16, K, N))
    assert a["nws"] > 0
    if case == "bad_act": a["act"] = 9
    if case == "swiglu": a["act"] = 2
    if case == "bad_out": a["out"] = 5
    if case == "f32_gelu": a["out"] = 0
    if case == "m17": a["M"] = 17
    if case == "null_x": a["X"] = None
    if case == "null_wp": a["Wp"] = None
    if case == "misaligned_wp": a["Wp"] = MIS
    if case == "small_wp": a["nwp"] -= 16
    if case == "no_ws": a["ws"] = None
    if case == "misaligned_ws": a["ws"] = A + 16
    if case == "ld_small": a["ldy"] = N - 8
    st = lib.tp_decode_linear_packed(a["act"], a["out"], a["M"], K, N, a["X"], a["ldx"], a["Wp"], a["nwp"],
                                     a["bias"], a["Y"], a["ldy"], a["ws"], a["nws"], None)
    assert st == expect, tp.tp_last_error()
    assert tp.tp_last_error()
