"""fp64 CPU oracle for causal decayed linear attention (lightning attention).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library.

What is computed
----------------
The MiniMax-M1 fact sheet (archdb), in its "linear / SSM layer configuration"
field, describes the lightning layer as linear attention with a fixed
per-head exponential decay and a 128x128 state per head; its "positional
scheme" field says these layers carry no RoPE, only that decay.  The CocoLoop
explainer ("MiniMax-01 Lightning Attention", section "El enfoque de Lightning
Attention") places it among linear-attention variants that take the cost from
O(n^2) to about O(n).  The function fixed from that description, for one
(batch, head) pair with decay lambda in [0, 1] and an initial state S0, is

    quadratic form:  O = (Q K^T * M) V + diag(lambda^(i+1)) Q S0,
                     M[i, j] = lambda^(i-j) for i >= j, else 0   (M[i, i] = 1)
    recurrence:      S_t = lambda S_{t-1} + k_t^T v_t,  S_{-1} = S0,
                     o_t = q_t S_t

Readings taken where the pages are silent (each is pinned by a test):
  * lambda^0 = 1 on the diagonal, including lambda = 0.
  * The initial state is S_{-1}: the first token already decays it once, and
    the returned final state is S_{N-1}.  Splitting a sequence and feeding the
    final state of the first part as the initial state of the second part then
    reproduces the unsplit result exactly.
  * No 1/sqrt(d) scale and no normaliser; inputs arrive pre-scaled.
  * The state is indexed S[key_dim, value_dim] (S = sum of k^T v).

Gradients (the backward pass; the pages are silent on it, so it is the
derivative of the function above and nothing more): for a loss L with
dL/dO = dO and dL/dS_final = dSN,

    dQ  = ((dO V^T) * M) K     + diag(lambda^(t+1)) dO S0^T
    dK  = ((dO V^T) * M)^T Q   + diag(lambda^(N-1-s)) V dSN^T
    dV  = ((Q K^T) * M)^T dO   + diag(lambda^(N-1-s)) K dSN
    dS0 = Q^T diag(lambda^(t+1)) dO + lambda^N dSN

(`backward_quadratic`, matrix calculus on the quadratic form).

The steps either side of the core (the same field of the fact sheet: SiLU on
Q, K, V and an RMSNorm on the output; its "output gate" field: a sigmoid gate
on the lightning output after that norm, before the output projection):

    silu(x)        = x * sigmoid(x),   sigmoid(x) = 1 / (1 + exp(-x))
    rmsnorm_heads  y = o / sqrt(mean_d(o^2) + eps) * gamma[h]   (per head, over
                   the d features of one token; eps = 1e-5 as the block norms)
    gate           y * sigmoid(g)

The token form of the same gradients, an adjoint recurrence run from the last
token back, is in recurrence.c (`crec.backward`); the two are checked against
each other and against central finite differences of the forward oracle.

Every function works in float64 on whatever bits it is given: callers pass the
exact values a GPU consumed (bf16 or fp32, upcast), and lambda as the fp32
value the GPU received, upcast, never recomputed.

Shapes: q, k, v are [..., N, d] with arbitrary leading (batch, head) dims;
lam broadcasts against the leading dims (shape [...], e.g. [H] for [B, H]);
states are [..., d, d].
"""

import numpy as np

__all__ = [
    "decay_matrix",
    "quadratic",
    "recurrent",
    "state_at",
    "decode_step",
    "decode_repeated",
    "window",
    "backward_quadratic",
    "silu",
    "rmsnorm_heads",
    "sigmoid_gate",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _pow_int(lam, e):
    """lambda ** e elementwise for integer e >= 0, with 0 ** 0 = 1.

    numpy's float power already gives 0.0 ** 0 == 1.0; this helper only makes
    that convention explicit and keeps the exponent integral."""
    e = np.asarray(e)
    assert np.all(e >= 0)
    return np.power(_f64(lam), e.astype(np.float64))


def decay_matrix(lam, n):
    """M[i, j] = lam^(i-j) for i >= j, else 0, for a scalar lam (n x n)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    diff = i - j
    m = _pow_int(float(lam), np.maximum(diff, 0))
    return np.where(diff >= 0, m, 0.0)


def _lead(q):
    return q.shape[:-2]


def _iter_lead(shape):
    if len(shape) == 0:
        yield ()
        return
    for idx in np.ndindex(*shape):
        yield idx


def _lam_at(lam, lead_shape, idx):
    lam = _f64(lam)
    lam_full = np.broadcast_to(lam, lead_shape) if lead_shape else lam
    return float(lam_full[idx]) if lead_shape else float(lam)


def quadratic(q, k, v, lam, s0=None):
    """Quadratic masked form, per (batch, head): brute force, small N only.

    Returns (O [..., N, d], S_final [..., d, d])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = _lead(q)
    n, d = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    o = np.zeros(lead + (n, dv))
    s_out = np.zeros(lead + (d, dv))
    for idx in _iter_lead(lead):
        lm = _lam_at(lam, lead, idx)
        qi, ki, vi = q[idx], k[idx], v[idx]
        a = qi @ ki.T
        o[idx] = (a * decay_matrix(lm, n)) @ vi
        w = _pow_int(lm, np.arange(n - 1, -1, -1))          # lam^(N-1-j)
        s_fin = (w[:, None] * ki).T @ vi
        if s0 is not None:
            s0i = _f64(s0)[idx]
            row = _pow_int(lm, np.arange(1, n + 1))          # lam^(i+1)
            o[idx] += row[:, None] * (qi @ s0i)
            s_fin = s_fin + (lm ** n) * s0i
        s_out[idx] = s_fin
    return o, s_out


def recurrent(q, k, v, lam, s0=None):
    """Token-by-token recurrence S_t = lam S_{t-1} + k_t^T v_t, o_t = q_t S_t.

    Loops over tokens; vectorised only across the independent leading
    (batch, head) pairs.  Returns (O, S_final)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = _lead(q)
    n, d = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    lam_b = np.broadcast_to(_f64(lam), lead)[..., None, None] if lead else _f64(lam)
    s = np.zeros(lead + (d, dv)) if s0 is None else _f64(s0).copy()
    o = np.zeros(lead + (n, dv))
    for t in range(n):
        s = lam_b * s + k[..., t, :, None] * v[..., t, None, :]
        o[..., t, :] = np.einsum("...i,...ij->...j", q[..., t, :], s)
    return o, s


def state_at(k, v, lam, t, s0=None):
    """Closed-form state after token t (inclusive), one GEMM, no token loop:

        S_t = lam^(t+1) S0 + (w * K[0..t])^T V[0..t],   w_j = lam^(t-j)."""
    k, v = _f64(k), _f64(v)
    lead = _lead(k)
    d, dv = k.shape[-1], v.shape[-1]
    out = np.zeros(lead + (d, dv))
    for idx in _iter_lead(lead):
        lm = _lam_at(lam, lead, idx)
        w = _pow_int(lm, np.arange(t, -1, -1))
        st = (w[:, None] * k[idx][: t + 1]).T @ v[idx][: t + 1]
        if s0 is not None:
            st = st + (lm ** (t + 1)) * _f64(s0)[idx]
        out[idx] = st
    return out


def decode_step(q, k, v, lam, s):
    """One decode step: S <- lam S + k^T v, then o = q S.

    q, k, v are [..., d]; s is [..., d, d].  Returns (o, S_new)."""
    q, k, v, s = _f64(q), _f64(k), _f64(v), _f64(s)
    lead = q.shape[:-1]
    lam_b = np.broadcast_to(_f64(lam), lead)[..., None, None] if lead else _f64(lam)
    s_new = lam_b * s + k[..., :, None] * v[..., None, :]
    o = np.einsum("...i,...ij->...j", q, s_new)
    return o, s_new


def decode_repeated(s0, k, v, lam, n):
    """State after n decode steps that all see the same (k, v):

        S_n = lam^n S0 + g_n k^T v,  g_n = (1 - lam^n) / (1 - lam)  (= n at lam = 1).

    The geometric sum is evaluated as sum_{j<n} lam^j when lam is within
    1e-6 of 1, where the quotient loses digits."""
    s0, k, v = _f64(s0), _f64(k), _f64(v)
    lead = k.shape[:-1]
    lam_full = np.broadcast_to(_f64(lam), lead)
    g = np.empty(lead)
    for idx in _iter_lead(lead):
        lm = float(lam_full[idx]) if lead else float(lam_full)
        if abs(1.0 - lm) < 1e-6:
            g[idx] = float(np.sum(_pow_int(lm, np.arange(n))))
        else:
            g[idx] = (1.0 - lm ** n) / (1.0 - lm)
    lam_n = np.power(lam_full, n)
    return lam_n[..., None, None] * s0 + g[..., None, None] * (k[..., :, None] * v[..., None, :])


def window(q, k, v, lam, t0, t1, w, s0=None):
    """Outputs o_t for t in [t0, t1), from the recurrence started at token
    max(0, t0 - w) with zero state (or s0 if that start is token 0).

    The dropped prefix contributes lam^(w+1) * q_t S_{t0-w-1} ... at most
    lam^(w+1+(t-t0)) |q_t| |S|, so for lam^w tiny the result equals the exact
    one up to that bound."""
    start = max(0, t0 - w)
    init = s0 if (start == 0) else None
    o, _ = recurrent(q[..., start:t1, :], k[..., start:t1, :], v[..., start:t1, :], lam, init)
    return o[..., t0 - start:, :]


def backward_quadratic(q, k, v, lam, dout, s0=None, dsn=None):
    """Gradients of L with dL/dO = dout and dL/dS_final = dsn, from the masked
    matrix form (matrix calculus; brute force, small N only):

        dQ  = ((dO V^T) * M) K   + diag(lam^(t+1)) dO S0^T
        dK  = ((dO V^T) * M)^T Q + diag(lam^(N-1-s)) V dSN^T
        dV  = ((Q K^T) * M)^T dO + diag(lam^(N-1-s)) K dSN
        dS0 = Q^T diag(lam^(t+1)) dO + lam^N dSN

    Returns (dQ, dK, dV [..., N, d], dS0 [..., d, d])."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    lead = _lead(q)
    n, d = q.shape[-2], q.shape[-1]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    ds0 = np.zeros(lead + (d, d))
    for idx in _iter_lead(lead):
        lm = _lam_at(lam, lead, idx)
        qi, ki, vi, gi = q[idx], k[idx], v[idx], g[idx]
        m = decay_matrix(lm, n)
        gv = (gi @ vi.T) * m          # (dO V^T) * M
        qk = (qi @ ki.T) * m          # (Q K^T) * M
        dq[idx] = gv @ ki
        dk[idx] = gv.T @ qi
        dv[idx] = qk.T @ gi
        row = _pow_int(lm, np.arange(1, n + 1))              # lam^(t+1)
        ds = (row[:, None] * qi).T @ gi
        if s0 is not None:
            dq[idx] += row[:, None] * (gi @ _f64(s0)[idx].T)
        if dsn is not None:
            dsi = _f64(dsn)[idx]
            w = _pow_int(lm, np.arange(n - 1, -1, -1))       # lam^(N-1-s)
            dk[idx] += w[:, None] * (vi @ dsi.T)
            dv[idx] += w[:, None] * (ki @ dsi)
            ds = ds + (lm ** n) * dsi
        ds0[idx] = ds
    return dq, dk, dv, ds0


def _sigmoid(x):
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    """x * sigmoid(x), elementwise, float64."""
    x = _f64(x)
    return x * _sigmoid(x)


def rmsnorm_heads(o, gamma=None, eps=1e-5):
    """Per-head RMSNorm over the feature axis of o [..., H, N, d]:
    o / sqrt(mean(o^2) + eps), times gamma [H, d] (the same for every token)
    when given.  One token per head is o[..., H, 1, d]."""
    o = _f64(o)
    y = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    if gamma is not None:
        y = y * _f64(gamma)[:, None, :]
    return y


def sigmoid_gate(y, g):
    """y * sigmoid(g), elementwise, float64."""
    return _f64(y) * _sigmoid(g)
