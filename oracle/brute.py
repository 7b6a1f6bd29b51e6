"""Pure-Python-loop oracle for tiny inputs (test infrastructure only).

Written element by element from the same definitions as ``oracle.block``
(see there for the page citations) with ``math.erf`` / ``math.exp`` and no
NumPy arithmetic, so that a transposed operand, a dropped term or a wrong
index in the vectorised oracle shows up as a mismatch.  Inputs are nested
lists or arrays; outputs are lists of lists of Python floats.
"""
from __future__ import annotations

import math


def _rows(A):
    return [[float(v) for v in row] for row in A]


def matmul(A, B):
    A, B = _rows(A), _rows(B)
    n, k, m = len(A), len(B), len(B[0])
    assert all(len(r) == k for r in A)
    out = []
    for i in range(n):
        row = []
        for j in range(m):
            acc = 0.0
            for t in range(k):
                acc += A[i][t] * B[t][j]
            row.append(acc)
        out.append(row)
    return out


def transpose(A):
    A = _rows(A)
    return [[A[i][j] for i in range(len(A))] for j in range(len(A[0]))]


def gelu(x):
    return x * 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def gelu_grad(x):
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0))) + x * math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def silu(x):
    return x / (1.0 + math.exp(-x))


def silu_grad(x):
    s = 1.0 / (1.0 + math.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def _map(f, A):
    return [[f(v) for v in row] for row in A]


def _mul(A, B):
    return [[a * b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def _add(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def mlp_gelu(X, W1, W2, b1=None):
    Z = matmul(X, W1)
    if b1 is not None:
        b1 = [float(v) for v in b1]
        Z = [[z + b1[j] for j, z in enumerate(row)] for row in Z]
    H = _map(gelu, Z)
    return {"Z": Z, "H": H, "Y": matmul(H, W2)}


def mlp_swiglu(X, Wg, Wu, Wd):
    Zg, Zu = matmul(X, Wg), matmul(X, Wu)
    H = _mul(_map(silu, Zg), Zu)
    return {"H": H, "Y": matmul(H, Wd)}


def mlp_gelu_backward(X, W1, W2, dY):
    Z = matmul(X, W1)
    H = _map(gelu, Z)
    dH = matmul(dY, transpose(W2))
    dZ = _mul(dH, _map(gelu_grad, Z))
    return {"dW2": matmul(transpose(H), dY), "dW1": matmul(transpose(X), dZ),
            "dX": matmul(dZ, transpose(W1)),
            "db1": [sum(dZ[i][j] for i in range(len(dZ))) for j in range(len(dZ[0]))]}


def mlp_swiglu_backward(X, Wg, Wu, Wd, dY):
    Zg, Zu = matmul(X, Wg), matmul(X, Wu)
    H = _mul(_map(silu, Zg), Zu)
    dH = matmul(dY, transpose(Wd))
    dZu = _mul(dH, _map(silu, Zg))
    dZg = _mul(_mul(dH, Zu), _map(silu_grad, Zg))
    return {"dWd": matmul(transpose(H), dY), "dWg": matmul(transpose(X), dZg),
            "dWu": matmul(transpose(X), dZu),
            "dX": _add(matmul(dZg, transpose(Wg)), matmul(dZu, transpose(Wu)))}


def attention_head(Q, K, V, causal):
    """One head: for each query i, weights w_j = exp(q_i.k_j / sqrt d) over the
    allowed keys j (j <= i when causal), normalised, then sum_j w_j v_j."""
    Q, K, V = _rows(Q), _rows(K), _rows(V)
    d = len(Q[0])
    out = []
    for i in range(len(Q)):
        keys = range(i + 1) if causal else range(len(K))
        scores = [sum(Q[i][t] * K[j][t] for t in range(d)) / math.sqrt(d) for j in keys]
        m = max(scores)
        w = [math.exp(sc - m) for sc in scores]
        z = sum(w)
        out.append([sum(w[n] * V[j][c] for n, j in enumerate(keys)) / z for c in range(len(V[0]))])
    return out


def mha(X, Wq, Wk, Wv, Wo, heads, b, s, causal=True):
    X = _rows(X)
    h = len(X[0])
    d = h // heads
    Q, K, V = matmul(X, Wq), matmul(X, Wk), matmul(X, Wv)
    nh = len(Q[0]) // d
    O = [[0.0] * (nh * d) for _ in range(b * s)]
    for bi in range(b):
        for t in range(nh):
            sl = lambda M: [row[t * d:(t + 1) * d] for row in M[bi * s:(bi + 1) * s]]
            Ot = attention_head(sl(Q), sl(K), sl(V), causal)
            for i in range(s):
                O[bi * s + i][t * d:(t + 1) * d] = Ot[i]
    return {"O": O, "Y": matmul(O, Wo)}


def mha_gqa(X, Wq, Wk, Wv, Wo, heads, kv_heads, b, s, causal=True):
    """Grouped-query attention by loops: query head t attends with key/value
    head t // (heads // kv_heads)."""
    X = _rows(X)
    h = len(X[0])
    d = h // heads
    g = heads // kv_heads
    Q, K, V = matmul(X, Wq), matmul(X, Wk), matmul(X, Wv)
    O = [[0.0] * (heads * d) for _ in range(b * s)]
    for bi in range(b):
        for t in range(heads):
            u = t // g
            rows = range(bi * s, (bi + 1) * s)
            Qt = [Q[r][t * d:(t + 1) * d] for r in rows]
            Kt = [K[r][u * d:(u + 1) * d] for r in rows]
            Vt = [V[r][u * d:(u + 1) * d] for r in rows]
            Ot = attention_head(Qt, Kt, Vt, causal)
            for i in range(s):
                O[bi * s + i][t * d:(t + 1) * d] = Ot[i]
    return {"O": O, "Y": matmul(O, Wo)}


def layernorm(x, gamma, beta, eps):
    """Row by row: mean, population variance, normalise, scale and shift."""
    out = []
    for row in _rows(x):
        n = len(row)
        mu = sum(row) / n
        var = sum((v - mu) ** 2 for v in row) / n
        inv = 1.0 / math.sqrt(var + eps)
        out.append([float(gamma[j]) * (row[j] - mu) * inv + float(beta[j]) for j in range(n)])
    return out


def cross_entropy_rows(Z, targets):
    """Row by row: -log(exp(z_target) / sum_j exp(z_j)) with math.exp, the
    row max subtracted first."""
    out = []
    for row, t in zip(_rows(Z), targets):
        m = max(row)
        z = sum(math.exp(v - m) for v in row)
        out.append(-math.log(math.exp(row[int(t)] - m) / z))
    return out
