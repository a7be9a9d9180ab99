"""CPU pins of the oracle's elementwise steps either side of the core: SiLU,
per-head RMSNorm and the sigmoid gate (closed-form values, limits,
invariants)."""
import math

import numpy as np
import pytest

import oracle


def test_silu_values():
    assert oracle.silu(0.0) == 0.0
    # sigmoid(1) = e / (1 + e): silu(1) = e / (1 + e), silu(-1) = -1 / (1 + e)
    assert abs(oracle.silu(1.0) - math.e / (1 + math.e)) < 1e-15
    assert abs(oracle.silu(-1.0) + 1 / (1 + math.e)) < 1e-15
    # silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1)
    x = np.linspace(-7, 7, 57)
    assert np.allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=0, atol=1e-14)
    # limits: identity for large x, zero for very negative x
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12 and abs(oracle.silu(-40.0)) < 1e-15


def test_rmsnorm_heads_invariants():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((2, 3, 5, 16))
    y = oracle.rmsnorm_heads(o, eps=0.0)
    # unit RMS per token and head, and invariance under positive scaling
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0)
    assert np.allclose(oracle.rmsnorm_heads(7.5 * o, eps=0.0), y)
    # gamma scales each head's features
    gamma = rng.standard_normal((3, 16))
    assert np.allclose(oracle.rmsnorm_heads(o, gamma, eps=0.0), y * gamma[:, None, :])
    # a constant row c normalises to sign(c) / sqrt(1 + eps / c^2)
    c = np.full((1, 1, 1, 16), -0.5)
    assert np.allclose(oracle.rmsnorm_heads(c, eps=1e-5), -1.0 / math.sqrt(1 + 1e-5 / 0.25))
    # per token: normalising token by token gives the same rows
    for n in range(5):
        assert np.allclose(oracle.rmsnorm_heads(o[:, :, n:n + 1], gamma, eps=1e-5)[:, :, 0],
                           oracle.rmsnorm_heads(o, gamma, eps=1e-5)[:, :, n])


def test_sigmoid_gate_values():
    y = np.array([2.0, -3.0, 5.0])
    assert np.array_equal(oracle.sigmoid_gate(y, np.zeros(3)), y / 2)
    assert np.allclose(oracle.sigmoid_gate(y, np.full(3, 50.0)), y)
    assert np.allclose(oracle.sigmoid_gate(y, np.full(3, -50.0)), 0.0)
    assert abs(oracle.sigmoid_gate(1.0, 1.0) - math.e / (1 + math.e)) < 1e-15
