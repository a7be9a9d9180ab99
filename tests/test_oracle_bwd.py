"""CPU pins of the oracle's gradients (the backward pass).

Two derivations live in oracle/: the adjoint token recurrence in plain C
(crec.backward) and matrix calculus on the masked quadratic form
(lightning.backward_quadratic).  They are pinned to what does not depend on
either: a hand-worked example, central differences of the (separately
pinned) forward oracle, which are exact here because the loss is linear in
every single input entry, closed forms at lam = 0 and lam = 1, and the
split-sequence rule.  Planted mistakes in a copy of the matrix form must
fail the finite-difference pin."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import crec

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_backward.json")


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _loss(q, k, v, lam, g, s0, dsn):
    o, s = oracle.recurrent(q, k, v, lam, s0)
    return float(np.sum(g * o) + (0.0 if dsn is None else np.sum(dsn * s)))


def test_hand_worked_example():
    c = json.load(open(GOLDEN))
    args = [np.array(c[x], dtype=np.float64) for x in ("q", "k", "v")]
    g, s0, dsn = (np.array(c[x], dtype=np.float64) for x in ("dO", "s0", "dSN"))
    want = [np.array(c[x]) for x in ("dq", "dk", "dv", "ds0")]
    for got in (crec.backward(*args, c["lam"], g, s0, dsn), oracle.backward_quadratic(*args, c["lam"], g, s0, dsn)):
        for x, y in zip(got, want):
            assert np.array_equal(x, y), (x, y)


@pytest.mark.parametrize("lam", [0.0, 0.37, 0.9, 1.0])
@pytest.mark.parametrize("n", [0, 1, 2, 9, 40])
def test_two_forms_agree(lam, n):
    rng = np.random.default_rng(100 + n)
    B, H, d = 2, 2, 6
    q, k, v, g = (_rand((B, H, n, d), rng).astype(np.float32) for _ in range(4))
    s0, dsn = _rand((B, H, d, d), rng), _rand((B, H, d, d), rng)
    lamv = np.array([lam, 0.5])
    for s0x, dsnx in ((None, None), (s0, None), (None, dsn), (s0, dsn)):
        a = crec.backward(q, k, v, lamv, g, s0x, dsnx)
        b = oracle.backward_quadratic(q, k, v, lamv, g, s0x, dsnx)
        for x, y in zip(a, b):
            scale = max([1.0] + ([float(np.abs(y).max())] if y.size else []))
            assert np.allclose(x, y, rtol=1e-12, atol=1e-12 * scale)


def _fd_check(grad_fn, rng, lam, n=7, d=4, picks=12):
    """Central differences of the forward oracle at random coordinates of q,
    k, v and S0.  The loss is linear in each single entry, so the difference
    quotient is the derivative up to rounding."""
    # float32-exact values, so that the C oracle (float32 inputs) sees them as they are
    q, k, v, g = (_rand((n, d), rng).astype(np.float32).astype(np.float64) for _ in range(4))
    s0, dsn = _rand((d, d), rng), _rand((d, d), rng)
    dq, dk, dv, ds0 = grad_fn(q, k, v, lam, g, s0, dsn)
    h = 0.5
    worst = 0.0
    for name, x, gx in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("s0", s0, ds0)):
        for _ in range(picks):
            idx = tuple(rng.integers(0, s) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            argp = dict(q=q, k=k, v=v, s0=s0)
            argm = dict(q=q, k=k, v=v, s0=s0)
            argp[name], argm[name] = xp, xm
            fp = _loss(argp["q"], argp["k"], argp["v"], lam, g, argp["s0"], dsn)
            fm = _loss(argm["q"], argm["k"], argm["v"], lam, g, argm["s0"], dsn)
            fd = (fp - fm) / (2 * h)
            worst = max(worst, abs(fd - gx[idx]) / max(1.0, abs(fd)))
    return worst


@pytest.mark.parametrize("lam", [0.0, 0.5, 0.8, 1.0])
def test_finite_differences(lam):
    rng = np.random.default_rng(7)
    for fn in (oracle.backward_quadratic, crec.backward):
        assert _fd_check(fn, np.random.default_rng(7), lam) < 1e-9


def test_lambda_zero_closed_form():
    # lam = 0 keeps only the current token: o_t = (q_t.k_t) v_t, S_final = k_last^T v_last
    rng = np.random.default_rng(3)
    n, d = 6, 5
    q, k, v, g = (_rand((n, d), rng) for _ in range(4))
    s0, dsn = _rand((d, d), rng), _rand((d, d), rng)
    dq, dk, dv, ds0 = oracle.backward_quadratic(q, k, v, 0.0, g, s0, dsn)
    gv = np.sum(g * v, axis=1)[:, None]
    qk = np.sum(q * k, axis=1)[:, None]
    want_dk = gv * q
    want_dk[-1] += v[-1] @ dsn.T
    want_dv = qk * g
    want_dv[-1] += k[-1] @ dsn
    assert np.allclose(dq, gv * k) and np.allclose(dk, want_dk) and np.allclose(dv, want_dv)
    assert np.array_equal(ds0, np.zeros((d, d)))


def test_lambda_one_textbook():
    # lam = 1, no states: the gradients of causal linear attention tril(Q K^T) V
    rng = np.random.default_rng(4)
    n, d = 9, 4
    q, k, v, g = (_rand((n, d), rng) for _ in range(4))
    dq, dk, dv, _ = crec.backward(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), 1.0,
                                  g.astype(np.float32))
    q, k, v, g = (x.astype(np.float32).astype(np.float64) for x in (q, k, v, g))
    t = np.tril(np.ones((n, n)))
    assert np.allclose(dq, (t * (g @ v.T)) @ k)
    assert np.allclose(dk, (t * (g @ v.T)).T @ q)
    assert np.allclose(dv, (t * (q @ k.T)).T @ g)


def test_split_sequence_rule():
    # Backward of a split run: the second part's dS0 is the first part's dSN.
    rng = np.random.default_rng(5)
    n, d, t0, lam = 13, 4, 5, 0.7
    q, k, v, g = (_rand((n, d), rng).astype(np.float32) for _ in range(4))
    s0, dsn = _rand((d, d), rng), _rand((d, d), rng)
    full = crec.backward(q, k, v, lam, g, s0, dsn)
    _, s_mid = oracle.recurrent(q[:t0], k[:t0], v[:t0], lam, s0)
    b2 = crec.backward(q[t0:], k[t0:], v[t0:], lam, g[t0:], s_mid, dsn)
    b1 = crec.backward(q[:t0], k[:t0], v[:t0], lam, g[:t0], s0, b2[3])
    for i in range(3):
        assert np.allclose(np.concatenate([b1[i], b2[i]]), full[i], rtol=1e-12, atol=1e-12)
    assert np.allclose(b1[3], full[3], rtol=1e-12, atol=1e-12)


# --- planted mistakes: each must fail the finite-difference pin -------------

def _bwd_mutant(q, k, v, lam, g, s0, dsn, *, mut):
    n, d = q.shape
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    m = np.where(i >= j, lam ** np.maximum(i - j, 0).astype(float), 0.0)
    if mut == "noncausal":
        m = lam ** np.abs(i - j).astype(float)
    gv = (g @ v.T) * m
    qk = (q @ k.T) * m
    dq = gv @ k
    dk = (gv @ q) if mut == "dk_untransposed" else gv.T @ q
    dv = (qk @ g) if mut == "dv_untransposed" else qk.T @ g
    row = lam ** (np.arange(n) + (0 if mut == "s0_pow" else 1)).astype(float)
    dq = dq + row[:, None] * (g @ (s0 if mut == "s0_untransposed" else s0.T))
    w = lam ** (np.arange(n - 1, -1, -1) + (1 if mut == "dsn_pow" else 0)).astype(float)
    dk = dk + w[:, None] * (v @ (dsn if mut == "dsn_untransposed" else dsn.T))
    dv = dv + w[:, None] * (k @ dsn)
    ds0 = (row[:, None] * q).T @ g + (0.0 if mut == "ds0_no_dsn" else lam ** n) * dsn
    return dq, dk, dv, ds0


@pytest.mark.parametrize("mut", ["noncausal", "dk_untransposed", "dv_untransposed", "s0_pow", "s0_untransposed",
                                 "dsn_pow", "dsn_untransposed", "ds0_no_dsn"])
def test_mutants_are_caught(mut):
    rng = np.random.default_rng(11)
    fn = lambda q, k, v, lam, g, s0, dsn: _bwd_mutant(q, k, v, lam, g, s0, dsn, mut=mut)
    assert _fd_check(fn, rng, 0.6) > 1e-3
    rng = np.random.default_rng(11)
    ok = lambda q, k, v, lam, g, s0, dsn: _bwd_mutant(q, k, v, lam, g, s0, dsn, mut="none")
    assert _fd_check(ok, rng, 0.6) < 1e-9
