"""The pins are strong enough: plant a plausible mistake in the oracle (on the
CPU, via monkeypatch) and check that at least one pin test then fails."""
import numpy as np
import pytest
from scipy.special import erf

import oracle
import oracle.block as blk
import test_oracle_activations as T_act
import test_oracle_attention as T_att
import test_oracle_mlp as T_mlp


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(blk, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _gelu_tanh(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1 + np.tanh(np.sqrt(2 / np.pi) * (z + 0.044715 * z ** 3)))


def _gelu_grad_dropped_term(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * (1.0 + erf(z / np.sqrt(2.0)))


def _attention_unscaled(Q, K, V, causal):
    Q, K, V = (np.asarray(a, np.float64) for a in (Q, K, V))
    S = Q @ K.T
    if causal:
        S = np.where(np.triu(np.ones(S.shape, bool), 1), -np.inf, S)
    return blk.softmax_rows(S) @ V


def _attention_mask_diagonal(Q, K, V, causal):
    Q, K, V = (np.asarray(a, np.float64) for a in (Q, K, V))
    S = Q @ K.T / np.sqrt(Q.shape[1])
    if causal:
        S = np.where(np.triu(np.ones(S.shape, bool), 0), -np.inf, S)
    with np.errstate(invalid="ignore"):
        return blk.softmax_rows(S) @ V


def _shard_sum_drops_last(partials, bias=None):
    return _orig_shard_sum(partials[:-1], bias)


_orig_shard_sum = blk.shard_sum
_orig_backward = blk.mlp_gelu_backward


MUTATIONS = [
    ("gelu", _gelu_tanh, T_act.test_gelu_matches_printed_normal_cdf, ("block",)),
    ("gelu_grad", _gelu_grad_dropped_term, T_act.test_gelu_grad_closed_forms_and_finite_differences, ()),
    ("attention_heads", _attention_unscaled, T_att.test_attention_vs_torch_sdpa_float64, (True,)),
    ("attention_heads", _attention_mask_diagonal, T_att.test_attention_closed_forms, ()),
    ("shard_sum", _shard_sum_drops_last, T_mlp.test_row_split_sum_identity, ()),
]


@pytest.mark.parametrize("name,fn,pin,args", MUTATIONS,
                         ids=[f"{m[0]}-{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn, pin, args):
    _patch(monkeypatch, name, fn)
    with pytest.raises(AssertionError):
        pin(*args)


def test_backward_missing_activation_derivative_is_caught(monkeypatch):
    def wrong(X, W1, W2, dY, b1=None):
        g = dict(_orig_backward(X, W1, W2, dY, b1))
        g["dW1"] = np.asarray(X, np.float64).T @ g["dH"]   # forgot GELU'
        return g
    _patch(monkeypatch, "mlp_gelu_backward", wrong)
    with pytest.raises(AssertionError):
        T_mlp.test_mlp_gelu_backward_vs_torch_autograd()


def test_transposed_operand_is_caught(monkeypatch):
    # X W^T instead of X W (square weight so shapes still fit)
    def wrong_linear(X, W, b=None):
        Y = np.asarray(X, np.float64) @ np.asarray(W, np.float64).T
        return Y if b is None else Y + np.asarray(b, np.float64).reshape(1, -1)
    _patch(monkeypatch, "linear", wrong_linear)
    with pytest.raises(AssertionError):
        _square_linear_check()


def _square_linear_check():
    rng = np.random.default_rng(3)
    X = rng.integers(-2, 3, size=(9, 12)).astype(np.float32)
    Wm = rng.integers(-2, 3, size=(12, 12)).astype(np.float32)
    exact = (X.astype(np.int64) @ Wm.astype(np.int64)).astype(np.float64)
    assert np.array_equal(oracle.linear(X, Wm), exact)
