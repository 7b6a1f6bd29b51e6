"""Seeded synthetic inputs for the tensor-parallel shard workloads.

This module is shared by the fp64 oracle, the tests and the benchmark. It only
draws random numbers and rounds them to the storage precision; it holds none
of the method's arithmetic (no products, activations or reductions), so the
oracle and the HIP path stay independent of each other.

Drawing convention (one reading, since the pages fix no seed or generator):
  * NumPy PCG64 ``default_rng(seed)``, ``standard_normal(dtype=float32)``.
  * Draw order: X, then the FULL weight matrices in argument order
    (W1, W2 | Wg, Wu, Wd | Wq, Wk, Wv, Wo), then dY.  Full matrices are drawn
    first and split afterwards, so every shard sees slices of one unsharded
    model (the tensor-parallel result must equal the single-device one).
  * Weights are scaled by their standard deviation (0.02), activations and
    dY are N(0, 1).
  * bf16 workloads are rounded from the float32 draw with round-to-nearest-
    even; the float32 array returned holds exactly the bf16 values, and the
    ``bits`` view holds the 16-bit patterns that go to the device.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "round_to_bf16_bits", "bf16_bits_to_f32",
    "Tensor", "draw_normal", "make_mlp_inputs", "make_swiglu_inputs",
    "make_mha_inputs", "make_gqa_inputs", "column_shard", "row_shard", "qkv_shard",
    "gqa_qkv_shard", "gqa_kv_heads_of_shard", "out_shard", "make_sp_inputs", "make_ce_inputs",
]


# ---------------------------------------------------------------------------
# Workload table (shapes and distributions only)
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "mlp_gelu" | "mlp_swiglu" | "mha" | "decode_gelu"
    dtype: str           # "f32" | "bf16"
    b: int
    s: int
    h: int
    ffn: int = 0
    heads: int = 0
    kv_heads: int = 0    # grouped-query attention: key/value heads (0: = heads)
    n_shards: int = 1
    causal: bool = True
    backward: bool = False
    w_std: float = 0.02
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.b * self.s

    @property
    def ffn_shard(self) -> int:
        return self.ffn // self.n_shards

    @property
    def head_dim(self) -> int:
        return self.h // self.heads if self.heads else 0

    @property
    def heads_shard(self) -> int:
        return self.heads // self.n_shards if self.heads else 0


WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 MLP, two shards, forward and backward
    "tiny_mlp_f32": Workload("tiny_mlp_f32", "mlp_gelu", "f32", b=2, s=16, h=128,
                             ffn=512, n_shards=2, backward=True),
    # GPT-2-medium-shaped MLP shard, four shards on one device + shard sum
    "gpt2m_mlp_bf16": Workload("gpt2m_mlp_bf16", "mlp_gelu", "bf16", b=8, s=1024,
                               h=1024, ffn=4096, n_shards=4),
    # Llama-style SwiGLU MLP shard, forward and backward
    "llama_swiglu_bf16": Workload("llama_swiglu_bf16", "mlp_swiglu", "bf16", b=4,
                                  s=2048, h=4096, ffn=14336, n_shards=4, backward=True),
    # head-sharded causal MHA, 32 heads of 128, 8 heads per shard
    "mha_heads_bf16": Workload("mha_heads_bf16", "mha", "bf16", b=4, s=2048, h=4096,
                               heads=32, n_shards=4, causal=True),
    # grouped-query attention shard (Llama-3-8B-like 32 query / 8 key-value
    # heads of 128), 8 query heads and their 2 key/value heads per shard
    "gqa_heads_bf16": Workload("gqa_heads_bf16", "gqa", "bf16", b=4, s=2048, h=4096,
                               heads=32, kv_heads=8, n_shards=4, causal=True),
    # sequence-parallel end of the GPT-2-medium-shaped block: 4 fp32 partials
    # of [8192 x 1024] reduce-scattered over 4 ranks (2048 rows each), plus
    # bias, residual and LayerNorm
    "sp_ln_gpt2m": Workload("sp_ln_gpt2m", "sp_layernorm", "f32", b=8, s=1024, h=1024,
                            n_shards=4),
    # vocabulary-parallel cross-entropy, Llama-3 vocabulary (128256) over 4
    # shards of 32064 columns, 8192 token rows, bf16 logits
    "vocab_ce_bf16": Workload("vocab_ce_bf16", "vocab_ce", "bf16", b=4, s=2048, h=128256,
                              n_shards=4),
    # decode-phase MLP shard: 16 single-token requests, memory-bound GEMV
    "decode_mlp_bf16": Workload("decode_mlp_bf16", "decode_gelu", "bf16", b=16, s=1,
                                h=8192, ffn=28672, n_shards=8),
}


# ---------------------------------------------------------------------------
# Storage rounding
# ---------------------------------------------------------------------------
def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16) with round-to-nearest-even.

    Finite inputs only (the generators never produce inf/NaN)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Tensor:
    """A host tensor in its storage precision.

    ``f32`` holds the exact values (bf16-representable when dtype == "bf16");
    ``bits`` holds the uint16 patterns for bf16, else None."""
    f32: np.ndarray
    dtype: str
    bits: Optional[np.ndarray] = None

    @property
    def shape(self):
        return self.f32.shape

    def f64(self) -> np.ndarray:
        return self.f32.astype(np.float64)

    def device_array(self) -> np.ndarray:
        """Array whose raw bytes are what the device buffer must hold."""
        return self.bits if self.dtype == "bf16" else self.f32

    def slice_cols(self, c0: int, c1: int) -> "Tensor":
        return Tensor(np.ascontiguousarray(self.f32[:, c0:c1]), self.dtype,
                      None if self.bits is None else np.ascontiguousarray(self.bits[:, c0:c1]))

    def slice_rows(self, r0: int, r1: int) -> "Tensor":
        return Tensor(np.ascontiguousarray(self.f32[r0:r1]), self.dtype,
                      None if self.bits is None else np.ascontiguousarray(self.bits[r0:r1]))


def _finish(a32: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        bits = round_to_bf16_bits(a32)
        return Tensor(bf16_bits_to_f32(bits), dtype, bits)
    if dtype == "f32":
        return Tensor(np.ascontiguousarray(a32, dtype=np.float32), dtype, None)
    raise ValueError(f"unknown dtype {dtype!r}")


def draw_normal(rng: np.random.Generator, shape, std: float, dtype: str,
                row_block: int = 1 << 30) -> Tensor:
    """Draw N(0, std^2) in float32, in row blocks of the same stream (bounded
    temporary memory for very large matrices), then round to ``dtype``."""
    rows = shape[0]
    out = np.empty(shape, dtype=np.float32)
    for r0 in range(0, rows, row_block):
        r1 = min(rows, r0 + row_block)
        blk = rng.standard_normal((r1 - r0,) + tuple(shape[1:]), dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        out[r0:r1] = blk
    return _finish(out, dtype)


# ---------------------------------------------------------------------------
# Workload generators (full, unsharded matrices)
# ---------------------------------------------------------------------------
def make_mlp_inputs(T: int, h: int, ffn: int, dtype: str, seed: int = 0,
                    w_std: float = 0.02, with_dy: bool = False,
                    with_bias: bool = False, row_block: int = 1 << 30):
    """X[T,h], W1[h,ffn], W2[ffn,h] (+ b1[ffn], b2[h]) (+ dY[T,h])."""
    rng = np.random.default_rng(seed)
    d = {"X": draw_normal(rng, (T, h), 1.0, dtype, row_block),
         "W1": draw_normal(rng, (h, ffn), w_std, dtype, row_block),
         "W2": draw_normal(rng, (ffn, h), w_std, dtype, row_block)}
    if with_bias:
        d["b1"] = draw_normal(rng, (1, ffn), w_std, dtype)
        d["b2"] = draw_normal(rng, (1, h), w_std, "f32")
    if with_dy:
        d["dY"] = draw_normal(rng, (T, h), 1.0, dtype, row_block)
    return d


def make_swiglu_inputs(T: int, h: int, ffn: int, dtype: str, seed: int = 0,
                       w_std: float = 0.02, with_dy: bool = False,
                       row_block: int = 1 << 30):
    """X[T,h], Wg[h,ffn], Wu[h,ffn], Wd[ffn,h] (+ dY[T,h])."""
    rng = np.random.default_rng(seed)
    d = {"X": draw_normal(rng, (T, h), 1.0, dtype, row_block),
         "Wg": draw_normal(rng, (h, ffn), w_std, dtype, row_block),
         "Wu": draw_normal(rng, (h, ffn), w_std, dtype, row_block),
         "Wd": draw_normal(rng, (ffn, h), w_std, dtype, row_block)}
    if with_dy:
        d["dY"] = draw_normal(rng, (T, h), 1.0, dtype, row_block)
    return d


def make_mha_inputs(T: int, h: int, dtype: str, seed: int = 0, w_std: float = 0.02,
                    row_block: int = 1 << 30):
    """X[T,h], Wq, Wk, Wv [h,h], Wo [h,h]."""
    rng = np.random.default_rng(seed)
    d = {"X": draw_normal(rng, (T, h), 1.0, dtype, row_block)}
    for name in ("Wq", "Wk", "Wv", "Wo"):
        d[name] = draw_normal(rng, (h, h), w_std, dtype, row_block)
    return d


def make_gqa_inputs(T: int, h: int, heads: int, kv_heads: int, dtype: str, seed: int = 0,
                    w_std: float = 0.02, row_block: int = 1 << 30):
    """X[T,h], Wq [h,h], Wk, Wv [h, kv_heads*d], Wo [h,h] (d = h / heads)."""
    d = h // heads
    rng = np.random.default_rng(seed)
    out = {"X": draw_normal(rng, (T, h), 1.0, dtype, row_block)}
    for name, cols in (("Wq", h), ("Wk", kv_heads * d), ("Wv", kv_heads * d), ("Wo", h)):
        out[name] = draw_normal(rng, (h, cols), w_std, dtype, row_block)
    return out


def make_sp_inputs(T: int, N: int, n: int, seed: int = 0):
    """n fp32 partials [T,N] ~ N(0,1), bias [N] ~ N(0, 0.1^2), residual [T,N]
    ~ N(0,1), LayerNorm gamma [N] ~ N(1, 0.1^2) and beta [N] ~ N(0, 0.1^2),
    drawn in that order (float32)."""
    rng = np.random.default_rng(seed)
    out = {"P": [rng.standard_normal((T, N), dtype=np.float32) for _ in range(n)]}
    out["bias"] = (rng.standard_normal(N, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    out["residual"] = rng.standard_normal((T, N), dtype=np.float32)
    out["gamma"] = (np.float32(1.0) + rng.standard_normal(N, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    out["beta"] = (rng.standard_normal(N, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    return out


def make_ce_inputs(T: int, V: int, dtype: str, seed: int = 0, scale: float = 2.0,
                   row_block: int = 1 << 30):
    """Logits [T, V] ~ N(0, scale^2) and int32 target token ids uniform in
    [0, V), drawn in that order."""
    rng = np.random.default_rng(seed)
    logits = draw_normal(rng, (T, V), scale, dtype, row_block)
    targets = rng.integers(0, V, size=T).astype(np.int32)
    return {"logits": logits, "targets": targets}


# ---------------------------------------------------------------------------
# Shard slicing (index bookkeeping only): contiguous blocks in index order
# ---------------------------------------------------------------------------
def column_shard(W: Tensor, i: int, n: int) -> Tensor:
    w = W.shape[1] // n
    return W.slice_cols(i * w, (i + 1) * w)


def row_shard(W: Tensor, i: int, n: int) -> Tensor:
    w = W.shape[0] // n
    return W.slice_rows(i * w, (i + 1) * w)


def qkv_shard(Wq: Tensor, Wk: Tensor, Wv: Tensor, i: int, n: int, heads: int) -> Tensor:
    """Packed [Wq_i | Wk_i | Wv_i]: shard i holds global heads
    i*heads/n .. (i+1)*heads/n - 1, each block heads_local*d columns wide.
    Head t owns columns t*d .. (t+1)*d - 1 of Wq/Wk/Wv, so a head block is a
    contiguous column block."""
    if heads % n or Wq.shape[1] % heads:
        raise ValueError("heads must be a multiple of the shard count and divide h")
    parts = [column_shard(W, i, n) for W in (Wq, Wk, Wv)]
    f32 = np.ascontiguousarray(np.concatenate([p.f32 for p in parts], axis=1))
    bits = None
    if Wq.bits is not None:
        bits = np.ascontiguousarray(np.concatenate([p.bits for p in parts], axis=1))
    return Tensor(f32, Wq.dtype, bits)


def out_shard(Wo: Tensor, i: int, n: int) -> Tensor:
    return row_shard(Wo, i, n)


def gqa_kv_heads_of_shard(i: int, n: int, heads: int, kv_heads: int):
    """Global key/value heads that shard i's query heads i*heads/n ..
    (i+1)*heads/n - 1 read (query head t reads kv head t // (heads/kv_heads)):
    kv_heads/n of them when n <= kv_heads, else the one kv head of the group,
    replicated on n/kv_heads shards."""
    hl, g = heads // n, heads // kv_heads
    first, last = (i * hl) // g, (i * hl + hl - 1) // g
    return list(range(first, last + 1))


def gqa_qkv_shard(Wq: Tensor, Wk: Tensor, Wv: Tensor, i: int, n: int, heads: int,
                  kv_heads: int) -> Tensor:
    """Packed [Wq_i | Wk_i | Wv_i] of a grouped-query shard: the shard's
    heads/n query heads, then the key and value columns of the kv heads they
    read (``gqa_kv_heads_of_shard``)."""
    if heads % n or heads % kv_heads:
        raise ValueError("heads must be a multiple of the shard count and of kv_heads")
    if n > kv_heads and n % kv_heads:
        raise ValueError("with more shards than kv heads, kv_heads must divide the shard count")
    d = Wq.shape[1] // heads
    kv = gqa_kv_heads_of_shard(i, n, heads, kv_heads)
    q = column_shard(Wq, i, n)
    ks = [Wk.slice_cols(u * d, (u + 1) * d) for u in kv]
    vs = [Wv.slice_cols(u * d, (u + 1) * d) for u in kv]
    parts = [q] + ks + vs
    f32 = np.ascontiguousarray(np.concatenate([p.f32 for p in parts], axis=1))
    bits = None
    if Wq.bits is not None:
        bits = np.ascontiguousarray(np.concatenate([p.bits for p in parts], axis=1))
    return Tensor(f32, Wq.dtype, bits)
