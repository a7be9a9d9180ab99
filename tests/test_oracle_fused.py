"""CPU pins of the oracle's elementwise steps either side of the core: SiLU,
per-head RMSNorm and the sigmoid gate (closed-form values, limits,
invariants), and planted mistakes in copies of them that the pins must catch.

Each RMSNorm check takes a function with the oracle's signature
rms(o, gamma=None, eps=1e-5) and raises AssertionError when it is wrong.
"""
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


def check_rms_unit(rms):
    """With eps = 0 every (token, head) row has unit RMS, and a positive scale
    of the input leaves the output unchanged."""
    o = np.random.default_rng(0).standard_normal((2, 3, 5, 16))
    y = rms(o, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12, atol=0)
    assert np.allclose(rms(7.5 * o, eps=0.0), y, rtol=1e-12, atol=0)


def check_rms_gamma(rms):
    """gamma [H, d] multiplies feature j of every token of head h by gamma[h, j]."""
    rng = np.random.default_rng(1)
    o = rng.standard_normal((2, 3, 5, 16))
    gamma = rng.standard_normal((3, 16))
    assert np.allclose(rms(o, gamma, eps=0.0), rms(o, eps=0.0) * gamma[:, None, :], rtol=1e-12, atol=1e-14)


def check_rms_constant_rows(rms):
    """A constant row c normalises to c / sqrt(c^2 + eps) exactly (mean(c^2) =
    c^2).  At c = 1e-3, eps = 1e-5 the eps term is ten times the mean square,
    so the value (0.3015...) is far from that of eps added outside the root
    (0.990...) or left out (1.0)."""
    for c, eps in ((-0.5, 1e-5), (1e-3, 1e-5), (2e-3, 1e-5), (4.0, 0.25)):
        row = np.full((1, 1, 1, 16), c)
        want = c / math.sqrt(c * c + eps)
        got = rms(row, eps=eps)
        assert np.allclose(got, want, rtol=1e-13, atol=0), (c, eps, float(got.reshape(-1)[0]), want)


def check_rms_per_token(rms):
    """Rows are normalised one token at a time (over the d features, not over
    tokens or heads)."""
    rng = np.random.default_rng(2)
    o = rng.standard_normal((2, 3, 5, 16)) * rng.uniform(0.1, 10.0, (2, 3, 5, 1))
    gamma = rng.standard_normal((3, 16))
    whole = rms(o, gamma, eps=1e-5)
    for n in range(5):
        assert np.allclose(rms(o[:, :, n:n + 1], gamma, eps=1e-5)[:, :, 0], whole[:, :, n], rtol=1e-12, atol=1e-14)
    # and one (token, head) row by hand: sum of squares over d features
    r = o[1, 2, 3]
    want = r / math.sqrt(float(np.sum(r * r)) / 16 + 1e-5) * gamma[2]
    assert np.allclose(whole[1, 2, 3], want, rtol=1e-12, atol=1e-14)


RMS_CHECKS = [check_rms_unit, check_rms_gamma, check_rms_constant_rows, check_rms_per_token]


@pytest.mark.parametrize("check", RMS_CHECKS, ids=lambda c: c.__name__)
def test_rmsnorm_heads_pins(check):
    check(oracle.rmsnorm_heads)


def _rms_copy(o, gamma=None, eps=1e-5, *, eps_outside=False, no_eps=False, sum_not_mean=False,
              over_tokens=False, gamma_per_token=False):
    o = np.asarray(o, dtype=np.float64)
    axis = -2 if over_tokens else -1
    ms = (np.sum if sum_not_mean else np.mean)(o * o, axis=axis, keepdims=True)
    if no_eps:
        den = np.sqrt(ms)
    elif eps_outside:
        den = np.sqrt(ms) + eps
    else:
        den = np.sqrt(ms + eps)
    y = o / den
    if gamma is not None:
        g = np.asarray(gamma, dtype=np.float64)
        y = y * (g[None, :, :] if gamma_per_token and g.shape[0] == o.shape[-2] else g[:, None, :])
    return y


RMS_MUTANTS = {
    "eps_outside_the_root": dict(eps_outside=True),
    "eps_dropped": dict(no_eps=True),
    "sum_instead_of_mean": dict(sum_not_mean=True),
    "normalised_over_tokens": dict(over_tokens=True),
}


def test_rms_copy_unmutated_passes():
    for check in RMS_CHECKS:
        check(_rms_copy)


@pytest.mark.parametrize("name", sorted(RMS_MUTANTS))
def test_rmsnorm_mutant_caught(name):
    kw = RMS_MUTANTS[name]
    caught = []
    for check in RMS_CHECKS:
        try:
            check(lambda o, gamma=None, eps=1e-5: _rms_copy(o, gamma, eps, **kw))
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"


def test_eps_placement_is_pinned_by_constant_rows():
    """The placement of eps inside the square root is caught by the
    constant-row pin on its own (the value it tests differs by 3x)."""
    with pytest.raises(AssertionError):
        check_rms_constant_rows(lambda o, gamma=None, eps=1e-5: _rms_copy(o, gamma, eps, eps_outside=True))


def test_sigmoid_gate_values():
    y = np.array([2.0, -3.0, 5.0])
    assert np.array_equal(oracle.sigmoid_gate(y, np.zeros(3)), y / 2)
    assert np.allclose(oracle.sigmoid_gate(y, np.full(3, 50.0)), y)
    assert np.allclose(oracle.sigmoid_gate(y, np.full(3, -50.0)), 0.0)
    assert abs(oracle.sigmoid_gate(1.0, 1.0) - math.e / (1 + math.e)) < 1e-15
    # sigmoid(g) + sigmoid(-g) = 1: the gate and its mirror add up to y
    g = np.linspace(-6, 6, 25)
    assert np.allclose(oracle.sigmoid_gate(1.5, g) + oracle.sigmoid_gate(1.5, -g), 1.5, rtol=0, atol=1e-14)
