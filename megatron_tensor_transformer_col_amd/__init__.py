"""Python binding of libtpcol, the gfx950 tensor-parallel shard library.

Argument marshalling only: every function below forwards to the C entry
point of the same name in ``libtpcol.so`` (declared in ``include/tpcol.h``).
Tensors are torch device tensors used purely as device memory; shapes and
row strides are read from them, pointers and the current HIP stream are
passed through.  Nothing here computes: if the library is missing or a call
fails, a ``TpError`` is raised.

    import megatron_tensor_transformer_col_amd as tp
    tp.tp_col_linear_gelu(X, W1_i, H_i)              # H_i = GELU(X W1_i)
    tp.tp_row_linear_partial(H_i, W2_i, P_i)         # P_i = H_i W2_i
    tp.tp_shard_sum([P_0, ..., P_3], Y)              # Y = sum_i P_i
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "TpError", "lib", "library_path", "TP_F32", "TP_BF16", "TP_ACT_NONE", "TP_ACT_GELU_ERF",
    "TP_ACT_SWIGLU", "tp_col_linear_gelu", "tp_col_linear_gelu_noalloc", "tp_row_linear_partial",
    "tp_attn_heads_shard",
    "tp_attn_gqa_shard", "tp_attn_gqa_shard_workspace", "tp_attn_shard_backward",
    "tp_attn_shard_backward_workspace", "tp_shard_reduce_scatter_layernorm",
    "tp_vocab_ce_shard_stats", "tp_vocab_ce_lse", "tp_vocab_ce_shard_loss", "tp_vocab_ce_total",
    "tp_shard_sum", "tp_mlp_shard_backward", "tp_check_split", "tp_set_gemv_max_m",
    "tp_status_string", "tp_last_error", "tp_col_linear_gelu_workspace",
    "tp_row_linear_partial_workspace", "tp_attn_heads_shard_workspace",
    "tp_mlp_shard_backward_workspace", "tp_decode_packed_weight_bytes", "tp_decode_pack_weight",
    "tp_decode_linear_packed", "tp_decode_linear_packed_workspace", "EXPORTED_SYMBOLS",
]

TP_F32, TP_BF16 = 0, 1
TP_ACT_NONE, TP_ACT_GELU_ERF, TP_ACT_SWIGLU = 0, 1, 2
_ACTS = {"none": TP_ACT_NONE, "gelu": TP_ACT_GELU_ERF, "swiglu": TP_ACT_SWIGLU}

# TPCOL_LIBRARY selects another build of the same library (the sanitizer
# build of the host code, for the CPU ABI tests)
library_path = os.environ.get("TPCOL_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                               "libtpcol.so")

_i64, _sz, _vp, _int = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
_SIGS = {
    "tp_col_linear_gelu": (_int, [_int, _int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                  _vp, _vp, _i64, _vp, _sz, _vp]),
    "tp_col_linear_gelu_workspace": (_sz, [_int, _int, _i64, _i64, _i64]),
    "tp_col_linear_gelu_noalloc": (_int, [_int, _int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                          _vp, _vp, _i64, _vp]),
    "tp_row_linear_partial": (_int, [_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                     _vp, _sz, _vp]),
    "tp_row_linear_partial_workspace": (_sz, [_int, _i64, _i64, _i64]),
    "tp_decode_packed_weight_bytes": (_sz, [_i64, _i64]),
    "tp_decode_pack_weight": (_int, [_int, _i64, _i64, _vp, _i64, _vp, _sz, _vp]),
    "tp_decode_linear_packed": (_int, [_int, _int, _i64, _i64, _i64, _vp, _i64, _vp, _sz, _vp, _vp, _i64,
                                       _vp, _sz, _vp]),
    "tp_decode_linear_packed_workspace": (_sz, [_i64, _i64, _i64]),
    "tp_attn_heads_shard": (_int, [_int, _i64, _i64, _i64, _i64, _i64, _int, _vp, _i64, _vp,
                                   _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "tp_attn_heads_shard_workspace": (_sz, [_int, _i64, _i64, _i64, _i64]),
    "tp_attn_gqa_shard": (_int, [_int, _i64, _i64, _i64, _i64, _i64, _i64, _int, _vp, _i64, _vp,
                                 _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "tp_attn_gqa_shard_workspace": (_sz, [_int, _i64, _i64, _i64, _i64, _i64]),
    "tp_attn_shard_backward": (_int, [_int, _i64, _i64, _i64, _i64, _i64, _i64, _int, _vp, _i64, _vp, _i64,
                                      _vp, _i64, _vp, _i64, _vp, _sz, _vp, _vp, _vp, _i64, _vp, _sz, _vp]),
    "tp_attn_shard_backward_workspace": (_sz, [_int, _i64, _i64, _i64, _i64, _i64]),
    "tp_shard_sum": (_int, [_int, _i64, _i64, _int, ctypes.POINTER(_vp), _i64, _vp, _vp, _i64,
                            _vp]),
    "tp_shard_reduce_scatter_layernorm": (_int, [_int, _i64, _i64, _int, ctypes.POINTER(_vp), _i64, _vp,
                                                 _vp, _i64, _vp, _vp, ctypes.c_float, _vp, _i64, _vp,
                                                 _i64, _vp]),
    "tp_vocab_ce_shard_stats": (_int, [_int, _i64, _i64, _vp, _i64, _vp, _vp]),
    "tp_vocab_ce_lse": (_int, [_i64, _int, ctypes.POINTER(_vp), _vp, _vp]),
    "tp_vocab_ce_shard_loss": (_int, [_int, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp]),
    "tp_vocab_ce_total": (_int, [_int, ctypes.POINTER(_vp), _vp, _vp]),
    "tp_mlp_shard_backward": (_int, [_int, _int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp,
                                     _i64, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp,
                                     _i64, _vp, _sz, _vp]),
    "tp_mlp_shard_backward_workspace": (_sz, [_int, _int, _i64, _i64]),
    "tp_check_split": (_int, [_i64, _i64, _i64, _i64]),
    "tp_set_gemv_max_m": (_int, [_int]),
    "tp_status_string": (ctypes.c_char_p, [_int]),
    "tp_last_error": (ctypes.c_char_p, []),
}
EXPORTED_SYMBOLS = tuple(_SIGS)

_lib = None
_lock = threading.Lock()


class TpError(RuntimeError):
    def __init__(self, fn, status, detail):
        self.status = status
        self.detail = detail
        super().__init__(f"{fn} failed: {_status_text(status)}: {detail}")


def lib() -> ctypes.CDLL:
    """The loaded libtpcol.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(library_path):
                    raise TpError("load", -6, f"{library_path} is missing; build it with "
                                  "`python -m megatron_tensor_transformer_col_amd._build`")
                handle = ctypes.CDLL(library_path)
                for name, (res, args) in _SIGS.items():
                    f = getattr(handle, name)
                    f.restype, f.argtypes = res, args
                _lib = handle
    return _lib


def _status_text(status):
    try:
        return lib().tp_status_string(status).decode()
    except Exception:  # library not loadable: still report the number
        return f"status {status}"


def tp_status_string(status: int) -> str:
    return lib().tp_status_string(status).decode()


def tp_last_error() -> str:
    return lib().tp_last_error().decode()


def _check(fn, status):
    if status != 0:
        raise TpError(fn, status, tp_last_error())


# --------------------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return TP_BF16
    if t.dtype == torch.float32:
        return TP_F32
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _mat(t, name):
    """(pointer, rows, cols, ld) of a 2-D row-major tensor (or None)."""
    if t is None:
        return None, 0, 0, 0
    if t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D row-major tensor view")
    if t.numel() == 0:  # no element is read: any strides, row stride = width
        return t.data_ptr(), t.size(0), t.size(1), max(t.size(1), 1)
    if t.size(1) > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major tensor view")
    return t.data_ptr(), t.size(0), t.size(1), t.stride(0)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, ref):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    torch = _torch()
    return torch.cuda.current_stream(ref.device).cuda_stream


class _WorkspaceCache:
    """Scratch buffers owned by the binding for calls made without ws=, one per
    (device, stream, zeroed): a call's workspace must not be used by another
    call that can run at the same time, and calls on one stream are ordered.
    A buffer that grows is replaced on the same stream, so torch's allocator
    reuses the old block only after the work already queued there."""

    def __init__(self):
        self._bufs = {}
        self._lock = threading.Lock()

    def get(self, nbytes, device, stream, zeroed):
        if nbytes == 0:
            return None
        torch = _torch()
        key = (str(device), int(stream or 0), zeroed)
        with self._lock:
            buf = self._bufs.get(key)
            if buf is None or buf.numel() < nbytes:
                alloc = torch.zeros if zeroed else torch.empty
                s = torch.cuda.ExternalStream(stream, device=device) if stream else None
                with torch.cuda.stream(s) if s is not None else _nullcontext():
                    buf = alloc(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
                self._bufs[key] = buf
            return buf


_ws_cache = _WorkspaceCache()


class _nullcontext:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


def _workspace(ws, nbytes, device, zeroed, stream=None):
    if ws is not None:
        return ws.data_ptr(), ws.numel() * ws.element_size()
    buf = _ws_cache.get(nbytes, device, stream, zeroed)
    return (None, 0) if buf is None else (buf.data_ptr(), buf.numel())


# --------------------------------------------------------------------------- entry points
def tp_col_linear_gelu_workspace(dtype, act, M, K, Ni) -> int:
    return lib().tp_col_linear_gelu_workspace(dtype, act, M, K, Ni)


def tp_row_linear_partial_workspace(dtype, M, Ki, N) -> int:
    return lib().tp_row_linear_partial_workspace(dtype, M, Ki, N)


def tp_attn_heads_shard_workspace(dtype, b, s, heads_local, d) -> int:
    return lib().tp_attn_heads_shard_workspace(dtype, b, s, heads_local, d)


def tp_attn_gqa_shard_workspace(dtype, b, s, heads_local, kv_heads_local, d) -> int:
    return lib().tp_attn_gqa_shard_workspace(dtype, b, s, heads_local, kv_heads_local, d)


def tp_mlp_shard_backward_workspace(dtype, act, M, Ni) -> int:
    return lib().tp_mlp_shard_backward_workspace(dtype, act, M, Ni)


def tp_col_linear_gelu(X, W, H, act="gelu", Wup=None, bias=None, ws=None, stream=None):
    """H = act(X W + bias) (or SiLU(X W) * (X Wup) for act='swiglu')."""
    dt = _dtype_code(X)
    a = _ACTS[act] if isinstance(act, str) else int(act)
    px, M, K, ldx = _mat(X, "X")
    pw, _, Ni, ldw = _mat(W, "W")
    pu, _, _, ldu = _mat(Wup, "Wup")
    ph, _, _, ldh = _mat(H, "H")
    need = tp_col_linear_gelu_workspace(dt, a, M, K, Ni)
    st = _stream(stream, X)
    pws, nws = _workspace(ws, need, X.device, zeroed=True, stream=st)
    _check("tp_col_linear_gelu", lib().tp_col_linear_gelu(
        dt, a, M, K, Ni, px, ldx, pw, ldw, pu, ldu, _ptr(bias), ph, ldh, pws, nws,
        _stream(stream, X)))
    return H


def tp_col_linear_gelu_noalloc(X, W, H, act="gelu", Wup=None, bias=None, stream=None):
    """tp_col_linear_gelu without a workspace (the library's static scratch)."""
    dt = _dtype_code(X)
    a = _ACTS[act] if isinstance(act, str) else int(act)
    px, M, K, ldx = _mat(X, "X")
    pw, _, Ni, ldw = _mat(W, "W")
    pu, _, _, ldu = _mat(Wup, "Wup")
    ph, _, _, ldh = _mat(H, "H")
    _check("tp_col_linear_gelu_noalloc", lib().tp_col_linear_gelu_noalloc(
        dt, a, M, K, Ni, px, ldx, pw, ldw, pu, ldu, _ptr(bias), ph, ldh, _stream(stream, X)))
    return H


def tp_row_linear_partial(Xi, Wi, P, ws=None, stream=None):
    """P = Xi Wi (float32 partial of the row-parallel layer)."""
    dt = _dtype_code(Xi)
    px, M, Ki, ldx = _mat(Xi, "Xi")
    pw, _, N, ldw = _mat(Wi, "Wi")
    pp, _, _, ldp = _mat(P, "P")
    need = tp_row_linear_partial_workspace(dt, M, Ki, N)
    st = _stream(stream, Xi)
    pws, nws = _workspace(ws, need, Xi.device, zeroed=True, stream=st)
    _check("tp_row_linear_partial", lib().tp_row_linear_partial(
        dt, M, Ki, N, px, ldx, pw, ldw, pp, ldp, pws, nws, _stream(stream, Xi)))
    return P


def tp_decode_packed_weight_bytes(K, N) -> int:
    return lib().tp_decode_packed_weight_bytes(K, N)


def tp_decode_linear_packed_workspace(M, K, N) -> int:
    return lib().tp_decode_linear_packed_workspace(M, K, N)


def tp_decode_pack_weight(W, Wp=None, stream=None):
    """The 64-column panel copy of the bf16 weight W [K x N] for
    tp_decode_linear_packed; allocates Wp (uint8) unless one is given."""
    pw, K, N, ldw = _mat(W, "W")
    nbytes = tp_decode_packed_weight_bytes(K, N)
    if Wp is None:
        Wp = _torch().empty(nbytes, dtype=_torch().uint8, device=W.device)
    _check("tp_decode_pack_weight", lib().tp_decode_pack_weight(
        _dtype_code(W), K, N, pw, ldw, Wp.data_ptr(), Wp.numel() * Wp.element_size(), _stream(stream, W)))
    return Wp


def tp_decode_linear_packed(X, Wp, Y, act="gelu", bias=None, ws=None, stream=None):
    """Y = act(X W + bias) from W's panels (Y bf16), or the float32 partial
    Y = X W (Y float32, act 'none'); N is Y's width."""
    a = _ACTS[act] if isinstance(act, str) else int(act)
    if _dtype_code(X) != TP_BF16:
        raise TypeError("tp_decode_linear_packed takes a bfloat16 X")
    px, M, K, ldx = _mat(X, "X")
    py, _, N, ldy = _mat(Y, "Y")
    need = tp_decode_linear_packed_workspace(M, K, N)
    st = _stream(stream, X)
    pws, nws = _workspace(ws, need, X.device, zeroed=True, stream=st)
    _check("tp_decode_linear_packed", lib().tp_decode_linear_packed(
        a, _dtype_code(Y), M, K, N, px, ldx, Wp.data_ptr(), Wp.numel() * Wp.element_size(), _ptr(bias),
        py, ldy, pws, nws, st))
    return Y


def tp_attn_heads_shard(X, Wqkv, Wo, P, b, s, heads_local, d=128, causal=True, ws=None,
                        stream=None):
    """P = [Attention over this shard's heads] Wo_i (float32 partial)."""
    dt = _dtype_code(X)
    px, _, h, ldx = _mat(X, "X")
    pq, _, _, ldq = _mat(Wqkv, "Wqkv")
    po, _, _, ldo = _mat(Wo, "Wo")
    pp, _, _, ldp = _mat(P, "P")
    need = tp_attn_heads_shard_workspace(dt, b, s, heads_local, d)
    st = _stream(stream, X)
    pws, nws = _workspace(ws, need, X.device, zeroed=False, stream=st)
    _check("tp_attn_heads_shard", lib().tp_attn_heads_shard(
        dt, b, s, h, heads_local, d, 1 if causal else 0, px, ldx, pq, ldq, po, ldo, pp, ldp,
        pws, nws, _stream(stream, X)))
    return P


def tp_attn_gqa_shard(X, Wqkv, Wo, P, b, s, heads_local, kv_heads_local, d=128, causal=True,
                      ws=None, stream=None):
    """Grouped-query attention over this shard's query heads (each group of
    heads_local / kv_heads_local consecutive query heads reads one of the
    shard's kv heads), then the float32 partial P = O_i Wo_i."""
    dt = _dtype_code(X)
    px, _, h, ldx = _mat(X, "X")
    pq, _, _, ldq = _mat(Wqkv, "Wqkv")
    po, _, _, ldo = _mat(Wo, "Wo")
    pp, _, _, ldp = _mat(P, "P")
    need = tp_attn_gqa_shard_workspace(dt, b, s, heads_local, kv_heads_local, d)
    st = _stream(stream, X)
    pws, nws = _workspace(ws, need, X.device, zeroed=False, stream=st)
    _check("tp_attn_gqa_shard", lib().tp_attn_gqa_shard(
        dt, b, s, h, heads_local, kv_heads_local, d, 1 if causal else 0, px, ldx, pq, ldq, po, ldo,
        pp, ldp, pws, nws, _stream(stream, X)))
    return P


def tp_attn_shard_backward_workspace(dtype, b, s, heads_local, kv_heads_local, d=128):
    return lib().tp_attn_shard_backward_workspace(dtype, b, s, heads_local, kv_heads_local, d)


def tp_attn_shard_backward(X, Wqkv, Wo, dY, fwd_ws, dWqkv, dWo, dXi, b, s, heads_local, kv_heads_local=None,
                           d=128, causal=True, ws=None, stream=None):
    """Backward of the attention shard: dWqkv = X^T [dQ|dK|dV], dWo = O^T dY
    (float32, dense) and this shard's partial dXi (float32).  ``fwd_ws`` is
    the uint8 workspace tensor the forward call (tp_attn_heads_shard /
    tp_attn_gqa_shard with the same inputs) wrote; it must be passed to the
    forward explicitly so that it survives until here."""
    kvl = heads_local if kv_heads_local is None else kv_heads_local
    dt = _dtype_code(X)
    px, _, h, ldx = _mat(X, "X")
    pq, _, _, ldq = _mat(Wqkv, "Wqkv")
    po, _, _, ldo = _mat(Wo, "Wo")
    py, _, _, ldy = _mat(dY, "dY")
    pd, _, _, lddx = _mat(dXi, "dXi")
    for t, name in ((dWqkv, "dWqkv"), (dWo, "dWo")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be dense")
    need = tp_attn_shard_backward_workspace(dt, b, s, heads_local, kvl, d)
    st = _stream(stream, X)
    pws, nws = _workspace(ws, need, X.device, zeroed=False, stream=st)
    _check("tp_attn_shard_backward", lib().tp_attn_shard_backward(
        dt, b, s, h, heads_local, kvl, d, 1 if causal else 0, px, ldx, pq, ldq, po, ldo, py, ldy,
        fwd_ws.data_ptr(), fwd_ws.numel() * fwd_ws.element_size(), dWqkv.data_ptr(), dWo.data_ptr(), pd, lddx,
        pws, nws, _stream(stream, X)))
    return dWqkv, dWo, dXi


def tp_shard_sum(partials, Y, bias=None, stream=None):
    """Y = sum_i partials[i] (+ bias), partials float32 [M x N]."""
    n = len(partials)
    if n == 0:
        raise ValueError("need at least one partial")
    _, M, N, ldp = _mat(partials[0], "partials[0]")
    for p in partials[1:]:
        if tuple(p.shape) != (M, N) or (M > 1 and p.stride(0) != ldp):
            raise ValueError("all partials must share shape and row stride")
    arr = (ctypes.c_void_p * n)(*[p.data_ptr() for p in partials])
    py, _, _, ldy = _mat(Y, "Y")
    _check("tp_shard_sum", lib().tp_shard_sum(
        _dtype_code(Y), M, N, n, arr, ldp, _ptr(bias), py, ldy, _stream(stream, Y)))
    return Y


def tp_shard_reduce_scatter_layernorm(partials, gamma, beta, Y, eps=1e-5, bias=None, residual=None,
                                      Ysum=None, stream=None):
    """This rank's rows of LN(sum_i partials[i] (+ bias) (+ residual)).

    partials: float32 [rows x N] views at the rank's first row (e.g.
    P[r*T//n:(r+1)*T//n]); Y: [rows x N] bf16 or float32; Ysum: optional
    float32 [rows x N] for the pre-norm sum."""
    n = len(partials)
    if n == 0:
        raise ValueError("need at least one partial")
    _, rows, N, ldp = _mat(partials[0], "partials[0]")
    for p in partials[1:]:
        if tuple(p.shape) != (rows, N) or (rows > 1 and p.stride(0) != ldp):
            raise ValueError("all partials must share shape and row stride")
    arr = (ctypes.c_void_p * n)(*[p.data_ptr() for p in partials])
    py, _, _, ldy = _mat(Y, "Y")
    pr, _, _, ldr = _mat(residual, "residual")
    ps, _, _, lds = _mat(Ysum, "Ysum")
    _check("tp_shard_reduce_scatter_layernorm", lib().tp_shard_reduce_scatter_layernorm(
        _dtype_code(Y), rows, N, n, arr, ldp, _ptr(bias), pr, ldr, _ptr(gamma), _ptr(beta), float(eps),
        ps, lds, py, ldy, _stream(stream, Y)))
    return Y


def tp_vocab_ce_shard_stats(logits, stats, stream=None):
    """stats [T x 2] float32 = (row max, sum exp(z - max)) of this shard's logits."""
    pz, T, Vi, ldz = _mat(logits, "logits")
    _check("tp_vocab_ce_shard_stats", lib().tp_vocab_ce_shard_stats(
        _dtype_code(logits), T, Vi, pz, ldz, stats.data_ptr(), _stream(stream, logits)))
    return stats


def tp_vocab_ce_lse(stats, lse, stream=None):
    """lse [T] = log-sum-exp of each row over all shards from their stats."""
    n = len(stats)
    arr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in stats])
    _check("tp_vocab_ce_lse", lib().tp_vocab_ce_lse(lse.numel(), n, arr, lse.data_ptr(), _stream(stream, lse)))
    return lse


def tp_vocab_ce_shard_loss(logits, vocab_start, targets, lse, shard_loss, row_loss=None, stream=None):
    """shard_loss [1] = sum over rows whose target this shard holds of lse - z_target."""
    pz, T, Vi, ldz = _mat(logits, "logits")
    _check("tp_vocab_ce_shard_loss", lib().tp_vocab_ce_shard_loss(
        _dtype_code(logits), T, Vi, vocab_start, pz, ldz, targets.data_ptr(), lse.data_ptr(), _ptr(row_loss),
        shard_loss.data_ptr(), _stream(stream, logits)))
    return shard_loss


def tp_vocab_ce_total(shard_losses, total, stream=None):
    """total [1] = sum of the shards' losses, in shard order."""
    n = len(shard_losses)
    arr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in shard_losses])
    _check("tp_vocab_ce_total", lib().tp_vocab_ce_total(n, arr, total.data_ptr(), _stream(stream, total)))
    return total


def tp_mlp_shard_backward(X, W1, W2, dY, dW1, dW2, dXi, act="gelu", Wup=None, b1=None,
                          dWup=None, db1=None, ws=None, stream=None):
    """Shard backward of H = act(X W1) / SwiGLU, P = H W2 given dY."""
    dt = _dtype_code(X)
    a = _ACTS[act] if isinstance(act, str) else int(act)
    px, M, K, ldx = _mat(X, "X")
    pw1, _, Ni, ldw1 = _mat(W1, "W1")
    pu, _, _, ldu = _mat(Wup, "Wup")
    pw2, _, _, ldw2 = _mat(W2, "W2")
    pdy, _, _, lddy = _mat(dY, "dY")
    pdx, _, _, lddx = _mat(dXi, "dXi")
    need = tp_mlp_shard_backward_workspace(dt, a, M, Ni)
    st = _stream(stream, X)
    pws, nws = _workspace(ws, need, X.device, zeroed=False, stream=st)
    _check("tp_mlp_shard_backward", lib().tp_mlp_shard_backward(
        dt, a, M, K, Ni, px, ldx, pw1, ldw1, pu, ldu, _ptr(b1), pw2, ldw2, pdy, lddy,
        _ptr(dW1), _ptr(dWup), _ptr(dW2), _ptr(db1), pdx, lddx, pws, nws, _stream(stream, X)))
    return dXi


def tp_check_split(h, ffn, heads, n) -> int:
    return lib().tp_check_split(h, ffn, heads, n)


def tp_set_gemv_max_m(max_m: int) -> int:
    prev = lib().tp_set_gemv_max_m(max_m)
    if prev < 0:
        raise TpError("tp_set_gemv_max_m", prev, tp_last_error())
    return prev
