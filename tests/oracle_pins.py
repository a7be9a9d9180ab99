"""Pins for the fp64 oracle: checks that tie it to something other than itself.

Each check takes an implementation object exposing `quadratic` and
`recurrent` (signature (q, k, v, lam, s0=None) -> (O, S_final)) and raises
AssertionError when the implementation is wrong.  tests/test_oracle.py runs
them on the oracle; tests/test_oracle_mutants.py runs them on copies of the
oracle with planted mistakes and requires every mistake to be caught.

What pins what (none of these re-types the oracle's own formula):
  * golden        -- dyadic values worked by hand (tests/golden/hand_small.json)
  * brute         -- the double sum over (i, j) written as pure-Python loops
  * lam_one       -- textbook causal linear attention tril(Q K^T) V and the
                     cumulative sum of outer products k_t^T v_t
  * lam_zero      -- o_t = (q_t . k_t) v_t
  * constant      -- the geometric series for q = k = v = c * ones
  * carry         -- splitting a sequence and passing the final state on
                     reproduces the unsplit output and state
  * linearity     -- O is linear in V and in Q, and in S0 jointly with V
  * forms_agree   -- the two forms agree (quadratic vs recurrence)
"""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_small.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _both(impl):
    return [("quadratic", impl.quadratic), ("recurrent", impl.recurrent)]


def check_golden(impl):
    g = json.load(open(GOLDEN))
    q, k, v, s0 = (np.array(g[x], dtype=np.float64) for x in ("q", "k", "v", "s0"))
    for case in g["cases"]:
        for name, fn in _both(impl):
            o, s = fn(q, k, v, case["lam"], s0)
            assert np.array_equal(o, np.array(case["o"], dtype=np.float64)), (name, case["lam"], o)
            assert np.array_equal(s, np.array(case["s_final"], dtype=np.float64)), (name, case["lam"], s)


def check_brute(impl):
    """o_i = sum_{j<=i} lam^(i-j) (sum_c q_ic k_jc) v_j + lam^(i+1) sum_c q_ic S0[c, :]."""
    r = _rng(11)
    n, d = 6, 3
    q, k, v = (r.integers(-3, 4, size=(n, d)).astype(np.float64) for _ in range(3))
    s0 = r.integers(-2, 3, size=(d, d)).astype(np.float64)
    for lam in (0.0, 0.5, 0.75, 1.0):
        ref = [[0.0] * d for _ in range(n)]
        for i in range(n):
            for j in range(i + 1):
                dot = sum(q[i][c] * k[j][c] for c in range(d))
                for e in range(d):
                    ref[i][e] += (lam ** (i - j)) * dot * v[j][e]
            for e in range(d):
                ref[i][e] += (lam ** (i + 1)) * sum(q[i][c] * s0[c][e] for c in range(d))
        sref = [[(lam ** n) * s0[a][b] for b in range(d)] for a in range(d)]
        for j in range(n):
            for a in range(d):
                for b in range(d):
                    sref[a][b] += (lam ** (n - 1 - j)) * k[j][a] * v[j][b]
        for name, fn in _both(impl):
            o, s = fn(q, k, v, lam, s0)
            assert np.allclose(o, np.array(ref), rtol=1e-13, atol=1e-12), (name, lam)
            assert np.allclose(s, np.array(sref), rtol=1e-13, atol=1e-12), (name, lam)


def check_lam_one(impl):
    r = _rng(12)
    b, h, n, d = 2, 2, 97, 8
    q, k, v = (r.standard_normal((b, h, n, d)) for _ in range(3))
    lam = np.ones(h)
    ref = np.tril(q @ np.swapaxes(k, -1, -2)) @ v
    outer = k[..., :, :, None] * v[..., :, None, :]
    cum = np.cumsum(outer, axis=-3)
    ref2 = np.einsum("bhti,bhtij->bhtj", q, cum)
    for name, fn in _both(impl):
        o, s = fn(q, k, v, lam)
        assert np.allclose(o, ref, rtol=1e-11, atol=1e-11), name
        assert np.allclose(o, ref2, rtol=1e-11, atol=1e-11), name
        assert np.allclose(s, np.swapaxes(k, -1, -2) @ v, rtol=1e-11, atol=1e-11), name


def check_lam_zero(impl):
    r = _rng(13)
    n, d = 40, 8
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    s0 = r.standard_normal((d, d))
    ref = np.sum(q * k, axis=1)[:, None] * v
    for name, fn in _both(impl):
        o, s = fn(q, k, v, 0.0, s0)
        assert np.allclose(o, ref, rtol=1e-12, atol=1e-12), name
        assert np.allclose(s, np.outer(k[-1], v[-1]), rtol=1e-12, atol=1e-12), name


def check_constant(impl):
    n, d, c = 50, 4, 0.5
    x = np.full((n, d), c)
    t = np.arange(n)
    for lam in (0.3, 0.9, 1.0):
        g = (t + 1.0) if lam == 1.0 else (1.0 - lam ** (t + 1)) / (1.0 - lam)
        ref = (d * c ** 3 * g)[:, None] * np.ones((1, d))
        for name, fn in _both(impl):
            o, _ = fn(x, x, x, lam)
            assert np.allclose(o, ref, rtol=1e-12, atol=1e-12), (name, lam)


def check_carry(impl):
    r = _rng(14)
    n, d = 130, 8
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    s0 = r.standard_normal((d, d))
    for lam in (0.4, 0.97, 1.0):
        for name, fn in _both(impl):
            o_full, s_full = fn(q, k, v, lam, s0)
            for t0 in (1, 64, 77, 129):
                o1, s1 = fn(q[:t0], k[:t0], v[:t0], lam, s0)
                o2, s2 = fn(q[t0:], k[t0:], v[t0:], lam, s1)
                assert np.allclose(np.concatenate([o1, o2]), o_full, rtol=1e-11, atol=1e-11), (name, lam, t0)
                assert np.allclose(s2, s_full, rtol=1e-11, atol=1e-11), (name, lam, t0)


def check_linearity(impl):
    r = _rng(15)
    n, d = 33, 6
    q, k, v, v2 = (r.standard_normal((n, d)) for _ in range(4))
    q2 = r.standard_normal((n, d))
    s0, s0b = r.standard_normal((d, d)), r.standard_normal((d, d))
    lam = 0.8
    for name, fn in _both(impl):
        a, sa = fn(q, k, v, lam, s0)
        b, sb = fn(q, k, v2, lam, s0b)
        c, sc = fn(q, k, 2.0 * v - 3.0 * v2, lam, 2.0 * s0 - 3.0 * s0b)
        assert np.allclose(c, 2.0 * a - 3.0 * b, rtol=1e-11, atol=1e-11), name
        assert np.allclose(sc, 2.0 * sa - 3.0 * sb, rtol=1e-11, atol=1e-11), name
        e, _ = fn(q2, k, v, lam, s0)
        f, _ = fn(0.5 * q - q2, k, v, lam, s0)
        assert np.allclose(f, 0.5 * a - e, rtol=1e-11, atol=1e-11), name


def check_forms_agree(impl):
    r = _rng(16)
    b, h, n, d = 1, 3, 257, 16
    q, k, v = (r.standard_normal((b, h, n, d)) for _ in range(3))
    s0 = r.standard_normal((b, h, d, d))
    lam = np.array([0.0, 0.6, 0.999])
    o1, s1 = impl.quadratic(q, k, v, lam, s0)
    o2, s2 = impl.recurrent(q, k, v, lam, s0)
    scale = max(np.abs(o1).max(), 1.0)
    assert np.abs(o1 - o2).max() <= 1e-12 * scale
    assert np.abs(s1 - s2).max() <= 1e-12 * max(np.abs(s1).max(), 1.0)


ALL_CHECKS = [
    check_golden,
    check_brute,
    check_lam_one,
    check_lam_zero,
    check_constant,
    check_carry,
    check_linearity,
    check_forms_agree,
]
