"""NumPy float64 oracle of the unsharded block (test infrastructure only).

Notation follows the pages: X is the activation (tokens x h), W1/A the first
MLP weight, W2/B the second, H = GELU(X W1) the hidden activation, Y the
block output.  Weights are [in x out] and used as X @ W (the "张量并行" and
"Infra: Tensor Parallel" pages write X W; the nn.Linear [out x in] layout of
the "Megatron-LM 实战 04" code is the transpose of the same map).

Every input is cast to float64 first; inputs are expected to hold exactly the
values the device consumed (bf16-rounded where the workload is bf16).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

_SQRT2 = np.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / np.sqrt(2.0 * np.pi)


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Activations
# ---------------------------------------------------------------------------
def gelu(z):
    """Exact (erf) GELU: z * Phi(z) = z * 1/2 * [1 + erf(z / sqrt 2)].

    "张量并行", section MLP 层的并行化 (the GELU formula under Row -> Column)."""
    z = _f64(z)
    return z * 0.5 * (1.0 + erf(z / _SQRT2))


def gelu_grad(z):
    """d/dz [z Phi(z)] = Phi(z) + z phi(z), phi the standard normal density.
    (Chain rule on the GELU definition above; the pages do not print it.)"""
    z = _f64(z)
    return 0.5 * (1.0 + erf(z / _SQRT2)) + z * _INV_SQRT_2PI * np.exp(-0.5 * z * z)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    """SiLU(z) = z * sigmoid(z), the gate of the SwiGLU FFN whose W_gate and
    W_up are column-split (parallelism overview post, section 1 Tensor
    Parallelism); standard definition, not printed on the pages."""
    z = _f64(z)
    return z * _sigmoid(z)


def silu_grad(z):
    """d/dz [z sigmoid(z)] = sigmoid(z) * (1 + z (1 - sigmoid(z)))."""
    z = _f64(z)
    s = _sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def softmax_rows(S):
    """Row softmax, max-subtracted for range (exact up to rounding)."""
    S = _f64(S)
    m = np.max(S, axis=-1, keepdims=True)
    e = np.exp(S - m)
    return e / np.sum(e, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# Linear pieces
# ---------------------------------------------------------------------------
def linear(X, W, b=None):
    """Y = X W (+ b).  Column-linear shard i is the same map with W_i, the
    i-th column block (Infra: Tensor Parallel, Column-wise TP equation)."""
    Y = _f64(X) @ _f64(W)
    if b is not None:
        Y = Y + _f64(b).reshape(1, -1)
    return Y


def row_partial(Xi, Wi):
    """P_i = X_i W_i: one term of the row-wise sum  X W = sum_i X_i W_i
    ("张量并行", section 两个矩阵相乘, first step; Infra: Tensor Parallel,
    Row-wise TP equation).  No bias: the row bias is added once, after the
    sum, since sum_i (P_i + b) = X W + n b."""
    return _f64(Xi) @ _f64(Wi)


def shard_sum(partials, bias=None):
    """Y = sum_i P_i (+ b once): what the all-reduce of the row-parallel layer
    delivers ("张量并行", 行并行 / MLP 层的并行化: g's forward all-reduce)."""
    acc = np.zeros_like(_f64(partials[0]))
    for P in partials:
        acc = acc + _f64(P)
    if bias is not None:
        acc = acc + _f64(bias).reshape(1, -1)
    return acc


# ---------------------------------------------------------------------------
# MLP blocks
# ---------------------------------------------------------------------------
def mlp_gelu(X, W1, W2, b1=None, b2=None):
    """Y = GELU(X W1 + b1) W2 + b2.

    The Megatron MLP of "张量并行" (MLP 层的并行化, the A-column / B-row
    formula) and of "Infra: Tensor Parallel" (MLP section):
        Y = GELU(X [A_1 A_2]) [B_1; B_2] = sum_i GELU(X A_i) B_i.
    Returns dict(Z=pre-activation, H=hidden, Y=output)."""
    Z = linear(X, W1, b1)
    H = gelu(Z)
    Y = H @ _f64(W2)
    if b2 is not None:
        Y = Y + _f64(b2).reshape(1, -1)
    return {"Z": Z, "H": H, "Y": Y}


def mlp_swiglu(X, Wg, Wu, Wd):
    """Y = (SiLU(X Wg) * (X Wu)) Wd, '*' elementwise.  W_gate and W_up are
    column-split, the second layer row-split (parallelism overview post,
    section 1 Tensor Parallelism)."""
    Zg = linear(X, Wg)
    Zu = linear(X, Wu)
    H = silu(Zg) * Zu
    return {"Zg": Zg, "Zu": Zu, "H": H, "Y": H @ _f64(Wd)}


def mlp_gelu_backward(X, W1, W2, dY, b1=None):
    """Gradients of L = <Y, dY> for Y = GELU(X W1 + b1) W2.

    Row-wise layer (Infra: Tensor Parallel, Row-wise TP backward):
        dW2 = H^T dY,  dH = dY W2^T.
    Elementwise activation (chain rule): dZ = dH * GELU'(Z), db1 = sum_rows dZ.
    Column-wise layer (Infra: Tensor Parallel, Column-wise TP backward):
        dW1 = X^T dZ,  dX = dZ W1^T  (= sum_i dZ_i W1_i^T over column shards).
    """
    X, W1, W2, dY = _f64(X), _f64(W1), _f64(W2), _f64(dY)
    Z = linear(X, W1, b1)
    H = gelu(Z)
    dW2 = H.T @ dY
    dH = dY @ W2.T
    dZ = dH * gelu_grad(Z)
    return {"Z": Z, "H": H, "dH": dH, "dZ": dZ, "dW2": dW2, "dW1": X.T @ dZ,
            "db1": dZ.sum(axis=0), "dX": dZ @ W1.T}


def mlp_swiglu_backward(X, Wg, Wu, Wd, dY):
    """Gradients of L = <Y, dY> for Y = (SiLU(X Wg) * X Wu) Wd.

    dWd = H^T dY, dH = dY Wd^T (row-wise layer);
    dZu = dH * SiLU(Zg), dZg = dH * Zu * SiLU'(Zg) (chain rule);
    dWg = X^T dZg, dWu = X^T dZu, dX = dZg Wg^T + dZu Wu^T (column-wise)."""
    X, Wg, Wu, Wd, dY = _f64(X), _f64(Wg), _f64(Wu), _f64(Wd), _f64(dY)
    Zg = X @ Wg
    Zu = X @ Wu
    H = silu(Zg) * Zu
    dH = dY @ Wd.T
    dZu = dH * silu(Zg)
    dZg = dH * Zu * silu_grad(Zg)
    return {"Zg": Zg, "Zu": Zu, "H": H, "dH": dH, "dZg": dZg, "dZu": dZu,
            "dWd": H.T @ dY, "dWg": X.T @ dZg, "dWu": X.T @ dZu,
            "dX": dZg @ Wg.T + dZu @ Wu.T}


# ---------------------------------------------------------------------------
# Multi-head attention
# ---------------------------------------------------------------------------
def attention_heads(Q, K, V, causal):
    """O = softmax(Q K^T / sqrt(d) [+ causal mask]) V for ONE head of one
    sequence.  Q, K, V: [s, d].  Scores with key j > query i are excluded
    when causal (the diagonal is always kept, so no row is empty).

    Scaled dot-product as in "Megatron-LM 实战 04" (TPAttention.forward);
    causal masking is the workload's choice (decoder self-attention)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    d = Q.shape[1]
    S = (Q @ K.T) / np.sqrt(d)
    if causal:
        s = S.shape[0]
        mask = np.triu(np.ones((s, S.shape[1]), dtype=bool), k=1)
        S = np.where(mask, -np.inf, S)
    P = softmax_rows(S)
    return P @ V


def mha(X, Wq, Wk, Wv, Wo, heads, b, s, causal=True):
    """Unsharded multi-head attention block output Y and concatenated head
    outputs O (token-major [b*s, heads*d]).

    Head t uses columns t*d .. (t+1)*d - 1 of Wq/Wk/Wv with d = h / heads
    ("张量并行", Multi-Head Attention 的并行化: k_dim = v_dim = h // heads);
    O_t = Attention(X Wq^(t), X Wk^(t), X Wv^(t)) and Y = [O_1 ... O_H] Wo
    (Infra: Tensor Parallel, MHA equation).  Batch elements are independent.
    """
    X, Wq, Wk, Wv, Wo = _f64(X), _f64(Wq), _f64(Wk), _f64(Wv), _f64(Wo)
    h = X.shape[1]
    if h % heads:
        raise ValueError("hidden size must be a multiple of the head count")
    d = h // heads
    Q, K, V = X @ Wq, X @ Wk, X @ Wv
    O = np.zeros((b * s, Wq.shape[1]), dtype=np.float64)
    for bi in range(b):
        r = slice(bi * s, (bi + 1) * s)
        for t in range(Wq.shape[1] // d):
            c = slice(t * d, (t + 1) * d)
            O[r, c] = attention_heads(Q[r, c], K[r, c], V[r, c], causal)
    return {"Q": Q, "K": K, "V": V, "O": O, "Y": O @ Wo}


def mha_gqa(X, Wq, Wk, Wv, Wo, heads, kv_heads, b, s, causal=True):
    """Unsharded grouped-query attention block ("张量并行", 相关分析: GQA has
    num_attention_heads query heads but only num_kv_heads key/value heads,
    heads >= kv_heads).  Query head t reads key/value head t // g with
    g = heads / kv_heads, the grouping of consecutive query heads; with
    kv_heads == heads this is ``mha``.

    Wq, Wo: [h, h] (d = h / heads); Wk, Wv: [h, kv_heads * d], kv head u in
    columns u*d .. (u+1)*d - 1.  Returns Q, K, V, O (token-major) and Y."""
    X, Wq, Wk, Wv, Wo = _f64(X), _f64(Wq), _f64(Wk), _f64(Wv), _f64(Wo)
    h = X.shape[1]
    if h % heads or heads % kv_heads:
        raise ValueError("heads must divide h and be a multiple of kv_heads")
    d = h // heads
    g = heads // kv_heads
    if Wk.shape[1] != kv_heads * d or Wv.shape[1] != kv_heads * d:
        raise ValueError("Wk / Wv must have kv_heads * d columns")
    Q, K, V = X @ Wq, X @ Wk, X @ Wv
    O = np.zeros((b * s, heads * d), dtype=np.float64)
    for bi in range(b):
        r = slice(bi * s, (bi + 1) * s)
        for t in range(heads):
            u = t // g
            cq, ckv = slice(t * d, (t + 1) * d), slice(u * d, (u + 1) * d)
            O[r, cq] = attention_heads(Q[r, cq], K[r, ckv], V[r, ckv], causal)
    return {"Q": Q, "K": K, "V": V, "O": O, "Y": O @ Wo}


def attention_head_backward(Q, K, V, dO, causal):
    """Gradients of L = <O, dO> for one head, O = softmax(Q K^T / sqrt(d)
    [+ causal mask]) V.  The pages stop at the forward ("张量并行", Multi-Head
    Attention 的并行化: heads are independent, so a shard differentiates its
    own heads); the backward is the chain rule through the two products and
    the row softmax, whose Jacobian is diag(p) - p p^T:

        dV = P^T dO,   dP = dO V^T,
        dS = P * (dP - D),  D_i = sum_j P_ij dP_ij  (= sum_c dO_ic O_ic),
        dQ = dS K / sqrt(d),   dK = dS^T Q / sqrt(d).

    Masked entries have P = 0 and so dS = 0.  Also returns P, O, D and lse,
    the natural log of each row's softmax denominator sum_j exp(S_ij) of the
    scaled scores S = Q K^T / sqrt(d)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    d = Q.shape[1]
    S = (Q @ K.T) / np.sqrt(d)
    if causal:
        S = np.where(np.triu(np.ones(S.shape, dtype=bool), k=1), -np.inf, S)
    P = softmax_rows(S)
    m = S.max(axis=1)
    lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    O = P @ V
    dP = dO @ V.T
    D = (dP * P).sum(axis=1)
    dS = P * (dP - D[:, None])
    return {"P": P, "O": O, "lse": lse, "D": D, "dS": dS, "dV": P.T @ dO,
            "dQ": dS @ K / np.sqrt(d), "dK": dS.T @ Q / np.sqrt(d)}


def mha_backward(X, Wq, Wk, Wv, Wo, dY, heads, b, s, causal=True, kv_heads=None, head_dim=None):
    """Gradients of L = <Y, dY> for the unsharded (grouped-query) attention
    block Y = [O_1 ... O_H] Wo, O_t = Attention(X Wq^(t), X Wk^(u), X Wv^(u)),
    u = t // g, g = heads / kv_heads (kv_heads = heads: multi-head).

    Output projection, a row-wise layer (Infra: Tensor Parallel, Row-wise TP
    backward): dWo = O^T dY, dO = dY Wo^T.  Per head ``attention_head_backward``;
    a kv head read by g query heads receives the sum of their dK / dV.
    QKV projection, a column-wise layer (Infra: Tensor Parallel, Column-wise
    TP backward): dWq = X^T dQ, dWk = X^T dK, dWv = X^T dV,
    dX = dQ Wq^T + dK Wk^T + dV Wv^T.

    ``heads`` counts the query heads in Wq's columns; d = h / heads unless
    ``head_dim`` is given (a shard's subset of the heads: d = head_dim, Wq
    holding heads * d columns).  Token-major results ([b*s, ...]); lse and D
    are [b*s, heads]."""
    X, Wq, Wk, Wv, Wo, dY = (_f64(a) for a in (X, Wq, Wk, Wv, Wo, dY))
    kv_heads = heads if kv_heads is None else kv_heads
    h = X.shape[1]
    if (head_dim is None and h % heads) or heads % kv_heads:
        raise ValueError("heads must divide h and be a multiple of kv_heads")
    d = h // heads if head_dim is None else head_dim
    if Wq.shape[1] != heads * d or Wk.shape[1] != kv_heads * d or Wv.shape[1] != kv_heads * d:
        raise ValueError("Wq needs heads * d columns, Wk / Wv kv_heads * d")
    g = heads // kv_heads
    Q, K, V = X @ Wq, X @ Wk, X @ Wv
    O = np.zeros((b * s, heads * d))
    lse = np.zeros((b * s, heads))
    D = np.zeros((b * s, heads))
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    # O is needed before dO = dY Wo^T can be split per head; dO itself only
    # needs dY and Wo.
    dO = dY @ Wo.T
    for bi in range(b):
        r = slice(bi * s, (bi + 1) * s)
        for t in range(heads):
            u = t // g
            cq, ckv = slice(t * d, (t + 1) * d), slice(u * d, (u + 1) * d)
            gr = attention_head_backward(Q[r, cq], K[r, ckv], V[r, ckv], dO[r, cq], causal)
            O[r, cq] = gr["O"]
            lse[r, t] = gr["lse"]
            D[r, t] = gr["D"]
            dQ[r, cq] = gr["dQ"]
            dK[r, ckv] += gr["dK"]
            dV[r, ckv] += gr["dV"]
    return {"Q": Q, "K": K, "V": V, "O": O, "Y": O @ Wo, "lse": lse, "D": D, "dO": dO,
            "dQ": dQ, "dK": dK, "dV": dV, "dWo": O.T @ dY, "dWq": X.T @ dQ, "dWk": X.T @ dK,
            "dWv": X.T @ dV, "dX": dQ @ Wq.T + dK @ Wk.T + dV @ Wv.T}


def layernorm(x, gamma, beta, eps):
    """LN(x) = gamma * (x - mu(x)) / sqrt(sigma^2(x) + eps) + beta over the
    last (hidden) dimension, mu and sigma^2 the mean and the population
    variance of the full row ("张量并行", 相关分析: LayerNorm needs statistics
    over the complete hidden dimension, so it cannot run on a column shard)."""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return _f64(gamma) * (x - mu) / np.sqrt(var + eps) + _f64(beta)


def reduce_scatter_layernorm(partials, gamma, beta, eps, n, rank, bias=None, residual=None):
    """Sequence-parallel end of a tensor-parallel block (parallelism overview
    post, 5 Sequence Parallelism: the all-reduce splits into reduce-scatter +
    all-gather, and LayerNorm runs on each shard's 1/N of the tokens).

    The full sum Ysum = sum_i P_i (+ bias once) (+ residual) of the shards'
    partials, then rank's block of rows [rank*T/n, (rank+1)*T/n) of Ysum and
    of LN(Ysum).  Returns {"Ysum": block, "Y": LN(block)}."""
    full = shard_sum(partials, bias)
    if residual is not None:
        full = full + _f64(residual)
    T = full.shape[0]
    if T % n:
        raise ValueError("token count must be a multiple of the shard count")
    r = slice(rank * T // n, (rank + 1) * T // n)
    return {"Ysum": full[r], "Y": layernorm(full[r], gamma, beta, eps)}


def cross_entropy_rows(Z, targets):
    """Per-row softmax cross-entropy of logits Z [T, V] against target token
    ids: loss_t = log sum_j exp(Z[t, j]) - Z[t, target_t] ("张量并行",
    损失计算层的并行化: softmax over each row of the logits, then the
    cross-entropy with the true token).  The log-sum-exp is evaluated with
    the row max factored out (same value)."""
    Z = _f64(Z)
    m = Z.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(Z - m).sum(axis=1, keepdims=True)))[:, 0]
    t = np.asarray(targets, dtype=np.int64)
    return lse - Z[np.arange(Z.shape[0]), t]


def vocab_shard_stats(Zi):
    """Row statistics of one vocabulary shard's logits Zi [T, V/n]: the row
    max m_i and s_i = sum_j exp(Zi[t, j] - m_i)."""
    Zi = _f64(Zi)
    m = Zi.max(axis=1)
    return m, np.exp(Zi - m[:, None]).sum(axis=1)


def vocab_parallel_cross_entropy(Z, targets, n):
    """Vocabulary-parallel cross-entropy over n contiguous vocabulary shards
    ("张量并行", 损失计算层的并行化): per shard the row statistics; their
    combination over shards (a b*s-sized all-reduce) gives the softmax
    denominator lse_t = M_t + log sum_i s_i exp(m_i - M_t), M_t = max_i m_i;
    each shard's loss is the sum over the rows whose target token falls in
    its slice of (lse_t - Z[t, target_t]); the total is the sum of the n
    shard losses (an n-sized all-reduce).

    Returns {"stats": [(m_i, s_i)], "lse": [T], "shard_loss": [n], "total",
    "rows": per-row loss}."""
    Z = _f64(Z)
    T, V = Z.shape
    if V % n:
        raise ValueError("vocabulary size must be a multiple of the shard count")
    w = V // n
    t = np.asarray(targets, dtype=np.int64)
    stats = [vocab_shard_stats(Z[:, i * w:(i + 1) * w]) for i in range(n)]
    M = np.max(np.stack([m for m, _ in stats]), axis=0)
    lse = M + np.log(sum(s * np.exp(m - M) for m, s in stats))
    rows = lse - Z[np.arange(T), t]
    shard_loss = np.array([rows[(t >= i * w) & (t < (i + 1) * w)].sum() for i in range(n)])
    return {"stats": stats, "lse": lse, "shard_loss": shard_loss, "total": shard_loss.sum(), "rows": rows}
