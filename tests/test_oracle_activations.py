"""Pins for the oracle's elementwise pieces: GELU, GELU', SiLU, SiLU', softmax.

Each check compares against something other than the oracle's own formula:
printed normal-CDF values, exact identities, finite differences, or the
pure-Python loop implementation.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "normal_cdf.txt")


def _load_phi():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        x, p = line.split()
        rows.append((float(x), float(p)))
    assert len(rows) >= 5
    return rows


@pytest.mark.parametrize("impl", ["block", "brute"])
def test_gelu_matches_printed_normal_cdf(impl):
    # GELU(x) = x Phi(x); GELU(-x) = -x (1 - Phi(x)).
    f = (lambda v: float(oracle.gelu(v))) if impl == "block" else brute.gelu
    for x, phi in _load_phi():
        assert abs(f(x) - x * phi) < 2e-15 * max(1.0, x)
        assert abs(f(-x) - (-x * (1.0 - phi))) < 2e-15 * max(1.0, x)


def test_gelu_identities():
    x = np.linspace(-6, 6, 1201)
    g = oracle.gelu(x)
    assert oracle.gelu(0.0) == 0.0
    # Phi(-x) = 1 - Phi(x)  =>  GELU(x) - GELU(-x) = x
    np.testing.assert_allclose(g - oracle.gelu(-x), x, rtol=0, atol=1e-14)
    # not additive (the pages' reason the row->column order needs an all-reduce first)
    assert abs(oracle.gelu(1.0) + oracle.gelu(1.0) - oracle.gelu(2.0)) > 0.1


def test_gelu_grad_closed_forms_and_finite_differences():
    # GELU'(0) = Phi(0) = 1/2 ; GELU'(1) = Phi(1) + phi(1)
    phi1 = dict(_load_phi())[1.0]
    assert abs(oracle.gelu_grad(0.0) - 0.5) < 1e-16
    assert abs(oracle.gelu_grad(1.0) - (phi1 + math.exp(-0.5) / math.sqrt(2 * math.pi))) < 1e-14
    x = np.linspace(-5, 5, 401)
    eps = 1e-5
    fd = (oracle.gelu(x + eps) - oracle.gelu(x - eps)) / (2 * eps)
    np.testing.assert_allclose(oracle.gelu_grad(x), fd, rtol=0, atol=1e-9)
    np.testing.assert_allclose(oracle.gelu_grad(x), [brute.gelu_grad(v) for v in x], rtol=0, atol=1e-15)


def test_silu_closed_forms():
    ln3 = math.log(3.0)
    # sigmoid(ln 3) = 3/4
    assert abs(oracle.silu(ln3) - 0.75 * ln3) < 1e-15
    assert abs(oracle.silu_grad(ln3) - 0.75 * (1.0 + ln3 * 0.25)) < 1e-15
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu_grad(0.0) - 0.5) < 1e-16
    x = np.linspace(-8, 8, 801)
    # sigmoid(-x) = 1 - sigmoid(x)  =>  SiLU(x) - SiLU(-x) = x
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=0, atol=1e-13)
    eps = 1e-5
    fd = (oracle.silu(x + eps) - oracle.silu(x - eps)) / (2 * eps)
    np.testing.assert_allclose(oracle.silu_grad(x), fd, rtol=0, atol=1e-9)
    np.testing.assert_allclose(oracle.silu(x), [brute.silu(v) for v in x], rtol=0, atol=1e-14)


def test_softmax_rows_closed_forms():
    # two entries: softmax([a, b]) = [sigmoid(a - b), sigmoid(b - a)]
    a, b = 0.3, -1.1
    p = oracle.softmax_rows(np.array([[a, b]]))[0]
    s = 1.0 / (1.0 + math.exp(-(a - b)))
    assert abs(p[0] - s) < 1e-16 and abs(p[1] - (1 - s)) < 1e-15
    rng = np.random.default_rng(1)
    S = rng.standard_normal((7, 13)) * 5
    P = oracle.softmax_rows(S)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    # shift invariance and uniform rows
    np.testing.assert_allclose(oracle.softmax_rows(S + 3.0), P, rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.softmax_rows(np.zeros((2, 4))), 0.25, rtol=0, atol=0)
