"""Plant mistakes in copies of the oracle (on the CPU) and require that the pins
in tests/oracle_pins.py catch every one of them."""
import numpy as np
import pytest

import oracle
import oracle_pins as pins


def _rec(q, k, v, lam, s0=None, *, first_undecayed=False, transpose_out=False,
         exclusive=False, decay_new=False, ignore_s0=False, swap_kv=False):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    lam_b = np.broadcast_to(np.asarray(lam, dtype=np.float64), lead)[..., None, None] if lead else float(lam)
    s = np.zeros(lead + (d, d)) if (s0 is None or ignore_s0) else np.asarray(s0, dtype=np.float64).copy()
    o = np.zeros(lead + (n, d))
    for t in range(n):
        kt, vt = (v[..., t, :], k[..., t, :]) if swap_kv else (k[..., t, :], v[..., t, :])
        new = kt[..., :, None] * vt[..., None, :]
        prev = s
        decay = 1.0 if (first_undecayed and t == 0) else lam_b
        s = decay * s + (lam_b * new if decay_new else new)
        use = prev if exclusive else s
        if transpose_out:
            use = np.swapaxes(use, -1, -2)
        o[..., t, :] = np.einsum("...i,...ij->...j", q[..., t, :], use)
    return o, s


def _quad(q, k, v, lam, s0=None, *, mask_shift=0, noncausal=False, s0_pow_shift=1,
          s0_transposed=False, w_shift=0, s0_final_undecayed=False, scores_transposed=False):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    assert q.ndim == 2, "mutants of the quadratic form are exercised on single heads"
    n, d = q.shape
    lam = float(np.asarray(lam).reshape(-1)[0]) if np.ndim(lam) else float(lam)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    diff = i - j
    m = lam ** (np.abs(diff) + mask_shift)
    if not noncausal:
        m = np.where(diff >= 0, m, 0.0)
    a = (k @ q.T) if scores_transposed else (q @ k.T)
    o = (a * m) @ v
    w = lam ** (np.arange(n - 1, -1, -1) + w_shift)
    s = (w[:, None] * k).T @ v
    if s0 is not None:
        s0 = np.asarray(s0, dtype=np.float64)
        s0u = s0.T if s0_transposed else s0
        o = o + (lam ** (np.arange(n) + s0_pow_shift))[:, None] * (q @ s0u)
        s = s + (1.0 if s0_final_undecayed else lam ** n) * s0
    return o, s


def _single_head_only(fn):
    """Pins that batch over heads see the mutant applied head by head."""
    def wrapped(q, k, v, lam, s0=None):
        q = np.asarray(q)
        if q.ndim == 2:
            return fn(q, k, v, lam, s0)
        lead = q.shape[:-2]
        lam_f = np.broadcast_to(np.asarray(lam, dtype=np.float64), lead)
        o = np.zeros(q.shape[:-1] + (np.asarray(v).shape[-1],))
        s = np.zeros(lead + (q.shape[-1], np.asarray(v).shape[-1]))
        for idx in np.ndindex(*lead):
            oi, si = fn(q[idx], np.asarray(k)[idx], np.asarray(v)[idx], lam_f[idx],
                        None if s0 is None else np.asarray(s0)[idx])
            o[idx], s[idx] = oi, si
        return o, s
    return wrapped


REC_MUTANTS = {
    "first_token_leaves_S0_undecayed": dict(first_undecayed=True),
    "output_uses_transposed_state": dict(transpose_out=True),
    "output_before_update": dict(exclusive=True),
    "new_term_decayed_once_more": dict(decay_new=True),
    "initial_state_dropped": dict(ignore_s0=True),
    "k_and_v_swapped": dict(swap_kv=True),
}

QUAD_MUTANTS = {
    "mask_exponent_off_by_one": dict(mask_shift=1),
    "mask_not_causal": dict(noncausal=True),
    "S0_row_power_off_by_one": dict(s0_pow_shift=0),
    "S0_transposed": dict(s0_transposed=True),
    "final_state_weights_off_by_one": dict(w_shift=1),
    "final_state_S0_undecayed": dict(s0_final_undecayed=True),
    "scores_transposed": dict(scores_transposed=True),
}


def _caught(impl):
    failures = []
    for check in pins.ALL_CHECKS:
        try:
            check(impl)
        except AssertionError:
            failures.append(check.__name__)
    return failures


@pytest.mark.parametrize("name", sorted(REC_MUTANTS))
def test_recurrence_mutant_caught(name):
    kw = REC_MUTANTS[name]

    class Impl:
        quadratic = staticmethod(oracle.quadratic)
        recurrent = staticmethod(lambda q, k, v, lam, s0=None: _rec(q, k, v, lam, s0, **kw))

    assert _caught(Impl), f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(QUAD_MUTANTS))
def test_quadratic_mutant_caught(name):
    kw = QUAD_MUTANTS[name]

    class Impl:
        quadratic = staticmethod(_single_head_only(lambda q, k, v, lam, s0=None: _quad(q, k, v, lam, s0, **kw)))
        recurrent = staticmethod(oracle.recurrent)

    assert _caught(Impl), f"mutant {name} passed every pin"


def test_unmutated_copies_pass():
    """The mutant scaffolding itself is faithful when no mistake is planted."""
    class Impl:
        quadratic = staticmethod(_single_head_only(lambda q, k, v, lam, s0=None: _quad(q, k, v, lam, s0)))
        recurrent = staticmethod(lambda q, k, v, lam, s0=None: _rec(q, k, v, lam, s0))

    assert _caught(Impl) == []
