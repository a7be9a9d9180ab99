"""CPU-only pins of the fp64 oracle (see tests/oracle_pins.py for what pins what)."""
import numpy as np
import pytest

import oracle
from oracle import crec
import oracle_pins as pins


class _Oracle:
    quadratic = staticmethod(oracle.quadratic)
    recurrent = staticmethod(oracle.recurrent)


class _COracle:
    """The plain-C recurrence, behind the same interface (quadratic stays NumPy)."""
    quadratic = staticmethod(oracle.quadratic)

    @staticmethod
    def recurrent(q, k, v, lam, s0=None):
        q = np.asarray(q, dtype=np.float64)
        if not np.array_equal(q.astype(np.float32).astype(np.float64), q):
            pytest.skip("C oracle takes float32 inputs")
        return crec.recurrent(q, k, v, lam, s0)


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pins(check):
    check(_Oracle)


@pytest.mark.parametrize("check", [pins.check_golden, pins.check_brute, pins.check_constant,
                                   ], ids=lambda f: f.__name__)
def test_c_oracle_pins(check):
    check(_COracle)


def test_c_oracle_matches_numpy_forms():
    r = np.random.default_rng(3)
    b, h, n, d = 2, 3, 300, 32
    q, k, v = (r.standard_normal((b, h, n, d)).astype(np.float32) for _ in range(3))
    lam = np.array([0.0, 0.95, 1.0], dtype=np.float32)
    s0 = r.standard_normal((b, h, d, d))
    oq, sq = oracle.quadratic(q, k, v, lam, s0)
    oc, sc = crec.recurrent(q, k, v, lam, s0, threads=2)
    assert np.abs(oq - oc).max() <= 1e-12 * np.abs(oq).max()
    assert np.abs(sq - sc).max() <= 1e-12 * np.abs(sq).max()
    # partial output range
    op, _ = crec.recurrent(q, k, v, lam, s0, o_range=(100, 140), want_state=False)
    assert np.array_equal(op, oc[..., 100:140, :])


def test_state_closed_form():
    r = np.random.default_rng(4)
    n, d = 200, 8
    k, v, q = (r.standard_normal((n, d)) for _ in range(3))
    s0 = r.standard_normal((d, d))
    for lam in (0.0, 0.5, 0.99, 1.0):
        for t in (0, 1, 63, 199):
            _, s_t = oracle.recurrent(q[: t + 1], k[: t + 1], v[: t + 1], lam, s0)
            st = oracle.state_at(k, v, lam, t, s0)
            assert np.allclose(st, s_t, rtol=1e-12, atol=1e-12), (lam, t)


def test_decode_step_is_recurrence_of_one_token():
    r = np.random.default_rng(5)
    B, H, d = 3, 4, 16
    q, k, v = (r.standard_normal((B, H, d)) for _ in range(3))
    s = r.standard_normal((B, H, d, d))
    lam = np.array([0.0, 0.5, 0.9, 1.0])
    o1, s1 = oracle.decode_step(q, k, v, lam, s)
    o2, s2 = oracle.recurrent(q[..., None, :], k[..., None, :], v[..., None, :], lam, s)
    assert np.allclose(o1, o2[..., 0, :], rtol=1e-13, atol=1e-13)
    assert np.allclose(s1, s2, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("lam", [0.0, 0.5, 0.9961, 1.0 - 2.0 ** -20, 1.0])
def test_decode_repeated_closed_form(lam):
    r = np.random.default_rng(6)
    d = 8
    q, k, v = (r.standard_normal(d) for _ in range(3))
    s0 = r.standard_normal((d, d))
    s = s0.copy()
    for _ in range(1000):
        _, s = oracle.decode_step(q, k, v, lam, s)
    ref = oracle.decode_repeated(s0, k, v, lam, 1000)
    assert np.allclose(s, ref, rtol=1e-11, atol=1e-11)
    if lam == 1.0:
        assert np.allclose(ref, s0 + 1000 * np.outer(k, v), rtol=1e-13)


def test_window_truncation_bound():
    r = np.random.default_rng(7)
    n, d, w = 600, 8, 200
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    for lam in (0.5, 0.9):
        o_full, _ = oracle.recurrent(q, k, v, lam)
        ow = oracle.window(q, k, v, lam, 400, 450, w)
        # the dropped prefix state has norm <= sum_j lam^(..)|k_j||v_j|; bound it crudely
        smax = np.abs(oracle.state_at(k, v, lam, 199)).sum()
        bound = lam ** (w + 1) * np.abs(q[400:450]).sum(axis=1).max() * smax
        assert np.abs(ow - o_full[400:450]).max() <= bound + 1e-12
    # at lam = 1 the window oracle is wrong by design: it must differ
    o1, _ = oracle.recurrent(q, k, v, 1.0)
    assert np.abs(oracle.window(q, k, v, 1.0, 400, 450, w) - o1[400:450]).max() > 1e-3
