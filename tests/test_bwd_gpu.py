"""GPU parity of the backward pass (lightning_attn_bwd) against the fp64
gradient oracle (adjoint recurrence in plain C), through the C ABI.

The gradients are three prefill-shaped passes over the forward kernels at
block 64 (dK and dV with the tokens last first), so the cases mix heads that
take the warm-start path with heads that take the three-pass path, ragged
tails, initial states and final-state gradients.  Each head is held to the
tolerance on its own RMS."""
import math

import numpy as np
import pytest
import torch

import long_context_decayed_amd as la
from long_context_decayed_amd.inputs import decay_lambdas, qkv_device, state_device
from oracle import crec
import tolerances as tol
from gpu_helpers import host, oracle, oracle_threads, require_gpu, say

pytestmark = pytest.mark.gpu

MIXED_LAMS = np.array([0.0, 1e-3, 0.3, 0.7, 0.9, 0.97, 0.999, 1.0], dtype=np.float32)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _grad_oracle(q, k, v, lam, g, s0, dsn):
    return crec.backward(host(q), host(k), host(v), np.asarray(lam, np.float32).astype(np.float64), host(g),
                         None if s0 is None else host(s0).astype(np.float64),
                         None if dsn is None else host(dsn).astype(np.float64), threads=oracle_threads())


def _check_heads(got, ref, what, H):
    got = host(got)
    for h in range(H):
        tol.assert_bf16_f32out(got[:, h], ref[:, h], "%s head %d" % (what, h))


@pytest.mark.parametrize("states", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 63, 700, 3000 + 37])
def test_bwd_mixed_decays(dev, n, d, states):
    B, H = 2, 8
    say("bwd mixed decays B2 H8 N", n, "d", d, "states", states)
    q, k, v, g = qkv_device(B, H, n, d, seed=80 + n, device=dev) + qkv_device(B, H, n, d, seed=90 + n, device=dev)[:1]
    s0 = state_device(B, H, d, seed=80 + n, device=dev) if states else None
    dsn = state_device(B, H, d, seed=90 + n, device=dev) if states else None
    lam_t = torch.from_numpy(MIXED_LAMS).to(dev)
    dq, dk, dv, ds0 = la.bwd(q, k, v, lam_t, g, kv_in=s0, dkv_out=dsn, out_dtype=torch.float32, dkv_in=True)
    dq16, dk16, dv16, ds016 = la.bwd(q, k, v, lam_t, g, kv_in=s0, dkv_out=dsn, dkv_in=True)
    torch.cuda.synchronize()
    rq, rk, rv, rs = _grad_oracle(q, k, v, MIXED_LAMS, g, s0, dsn)
    _check_heads(dq, rq, "dQ", H)
    _check_heads(dk, rk, "dK", H)
    _check_heads(dv, rv, "dV", H)
    ds_h = host(ds0)
    for h in range(H):
        tol.assert_state(ds_h[:, h], rs[:, h], "dS0 head %d" % h)
    for a, b in ((dq, dq16), (dk, dk16), (dv, dv16)):
        assert torch.equal(a.to(torch.bfloat16), b), "bf16 gradients must be RNE(fp32 gradients)"
    assert torch.equal(ds0, ds016)


def test_bwd_layer_8k(dev):
    # one layer shaped like the 64-head model
    say("bwd B1 H64 N8192 d128 (inputs + oracle)")
    B, H, N, d = 1, 64, 8192, 128
    q, k, v = qkv_device(B, H, N, d, seed=81, device=dev)
    g = qkv_device(B, H, N, d, seed=82, device=dev)[0]
    lam = decay_lambdas(H)
    dq, dk, dv, _ = la.bwd(q, k, v, torch.from_numpy(lam).to(dev), g, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rq, rk, rv, _ = _grad_oracle(q, k, v, lam, g, None, None)
    e = [tol.assert_bf16_f32out(host(x), r, name) for x, r, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV"))]
    print("max|err|/RMS dQ %.3e dK %.3e dV %.3e" % tuple(e))


def test_bwd_split_sequence(dev):
    # Gradients of a run split at t0: the second half starts from the forward's
    # state at t0, its dS0 is the first half's dkv_out; the pieces must match
    # the unsplit backward.
    say("bwd split B1 H8 N2000 at 700, mixed decays")
    B, H, N, d, t0 = 1, 8, 2000, 128, 700
    q, k, v = qkv_device(B, H, N, d, seed=83, device=dev)
    g = qkv_device(B, H, N, d, seed=84, device=dev)[0]
    s0 = state_device(B, H, d, seed=83, device=dev)
    dsn = state_device(B, H, d, seed=84, device=dev)
    lam_t = torch.from_numpy(MIXED_LAMS).to(dev)
    cut = lambda x, a, b: x[:, :, a:b].contiguous()
    kv_mid = torch.empty_like(s0)
    la.fwd(cut(q, 0, t0), cut(k, 0, t0), cut(v, 0, t0), lam_t, kv_in=s0, kv_out=kv_mid, block=64)
    full = la.bwd(q, k, v, lam_t, g, kv_in=s0, dkv_out=dsn, out_dtype=torch.float32, dkv_in=True)
    b2 = la.bwd(cut(q, t0, N), cut(k, t0, N), cut(v, t0, N), lam_t, cut(g, t0, N), kv_in=kv_mid, dkv_out=dsn,
                out_dtype=torch.float32, dkv_in=True)
    b1 = la.bwd(cut(q, 0, t0), cut(k, 0, t0), cut(v, 0, t0), lam_t, cut(g, 0, t0), kv_in=s0, dkv_out=b2[3],
                out_dtype=torch.float32, dkv_in=True)
    torch.cuda.synchronize()
    for i, name in enumerate(("dQ", "dK", "dV")):
        split = torch.cat([b1[i], b2[i]], dim=2)
        for h in range(H):
            tol.assert_bf16_f32out(host(split)[:, h], host(full[i])[:, h].astype(np.float64), "%s head %d" % (name, h))
    rs = _grad_oracle(q, k, v, MIXED_LAMS, g, s0, dsn)[3]
    for h in range(H):
        tol.assert_state(host(b1[3])[:, h], rs[:, h], "dS0 head %d" % h)


def test_bwd_dkv_in_place(dev):
    say("bwd dkv_in is dkv_out, B1 H8 N1500 d64")
    B, H, N, d = 1, 8, 1500, 64
    q, k, v = qkv_device(B, H, N, d, seed=85, device=dev)
    g = qkv_device(B, H, N, d, seed=86, device=dev)[0]
    dsn = state_device(B, H, d, seed=85, device=dev)
    dsn_h = host(dsn).astype(np.float64)
    lam_t = torch.from_numpy(MIXED_LAMS).to(dev)
    _, _, _, out = la.bwd(q, k, v, lam_t, g, dkv_out=dsn, out_dtype=torch.float32, dkv_in=dsn)
    torch.cuda.synchronize()
    rs = crec.backward(host(q), host(k), host(v), MIXED_LAMS.astype(np.float64), host(g), None, dsn_h,
                       threads=oracle_threads())[3]
    for h in range(H):
        tol.assert_state(host(dsn)[:, h], rs[:, h], "dS0 head %d" % h)


# --- fp32 inputs: the general kernels, reversed for dK and dV ----------------

def test_bwd_fp32_tiny_workload(dev):
    say("bwd fp32 B1 H2 N1024 d64 (the tiny fp32 workload, seed 0)")
    from long_context_decayed_amd.inputs import qkv_cpu
    q, k, v = (t.to(dev) for t in qkv_cpu(1, 2, 1024, 64, seed=0))
    g = qkv_cpu(1, 2, 1024, 64, seed=1)[0].to(dev)
    lam = decay_lambdas(2)
    dq, dk, dv, ds0 = la.bwd(q, k, v, torch.from_numpy(lam).to(dev), g, dkv_in=True)
    torch.cuda.synchronize()
    assert dq.dtype == torch.float32
    rq, rk, rv, rs = _grad_oracle(q, k, v, lam, g, None, None)
    for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        tol.assert_fp32(host(got), ref, name)
    tol.assert_fp32(host(ds0), rs, "dS0")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_fp32_mixed_decays_with_states(dev, d):
    say("bwd fp32 mixed decays B2 H8 N777 d", d, "with states")
    B, H, n = 2, 8, 777
    from long_context_decayed_amd.inputs import qkv_cpu
    q, k, v = (t.to(dev) for t in qkv_cpu(B, H, n, d, seed=40 + d))
    g = qkv_cpu(B, H, n, d, seed=50 + d)[0].to(dev)
    s0 = state_device(B, H, d, seed=40 + d, device=dev)
    dsn = state_device(B, H, d, seed=50 + d, device=dev)
    dq, dk, dv, ds0 = la.bwd(q, k, v, torch.from_numpy(MIXED_LAMS).to(dev), g, kv_in=s0, dkv_out=dsn, dkv_in=True)
    torch.cuda.synchronize()
    rq, rk, rv, rs = _grad_oracle(q, k, v, MIXED_LAMS, g, s0, dsn)
    for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        got_h = host(got)
        for h in range(H):
            tol.assert_fp32(got_h[:, h], ref[:, h], "%s head %d" % (name, h))
    for h in range(H):
        tol.assert_fp32(host(ds0)[:, h], rs[:, h], "dS0 head %d" % h)


def test_bwd_exact_flag(dev):
    say("bwd exact flag, mixed decays B1 H8 N2100 d64 with states")
    B, H, N, d = 1, 8, 2100, 64
    q, k, v = qkv_device(B, H, N, d, seed=160, device=dev)
    g = qkv_device(B, H, N, d, seed=161, device=dev)[0]
    s0 = state_device(B, H, d, seed=160, device=dev)
    dsn = state_device(B, H, d, seed=161, device=dev)
    dq, dk, dv, ds0 = la.bwd(q, k, v, torch.from_numpy(MIXED_LAMS).to(dev), g, kv_in=s0, dkv_out=dsn,
                             out_dtype=torch.float32, dkv_in=True, exact=True)
    torch.cuda.synchronize()
    rq, rk, rv, rs = _grad_oracle(q, k, v, MIXED_LAMS, g, s0, dsn)
    _check_heads(dq, rq, "dQ", H)
    _check_heads(dk, rk, "dK", H)
    _check_heads(dv, rv, "dV", H)
    for h in range(H):
        tol.assert_state(host(ds0)[:, h], rs[:, h], "dS0 head %d" % h)


@pytest.mark.parametrize("in_place", [False, True])
def test_bwd_warm_chunk_longer_than_scan_chunk(dev, in_place):
    """At B16 H4 N16384 the backward's scan chunk is 1024 tokens and its
    warm-start chunk 2048, so the paired dK / dV launch runs warm-start chunks
    of one length beside pass-C chunks of another, and hands the reverse-time
    warm start's final state on as dS0.  Decays: 0, one with a carry span of
    832 (warm start only at the longer chunk), one just below 1, and 1; initial
    state and final-state gradient given, dS0 written over dS_N (in place) or
    apart."""
    B, H, n, d = 16, 4, 16384, 64
    assert la.chunk_for(B, H, n, 64) == 1024 and la.warm_chunk_for(B, H, n, 64) == 2048
    lams = np.array([0.0, 0.975, 0.9995, 1.0], dtype=np.float32)
    span = int(math.ceil(30 * math.log(2) / -math.log(float(lams[1]))))
    span = (span + 63) // 64 * 64
    assert 1024 < 2 * span <= 2048, span
    say("bwd warm chunk 2048 > scan chunk 1024, B16 H4 N16384 d64, in place", in_place)
    q, k, v = qkv_device(B, H, n, d, seed=170, device=dev)
    g = qkv_device(B, H, n, d, seed=171, device=dev)[0]
    s0 = state_device(B, H, d, seed=172, device=dev)
    dsn = state_device(B, H, d, seed=173, device=dev)
    dsn_host = dsn.clone()
    ds_out = dsn if in_place else True
    dq, dk, dv, ds0 = la.bwd(q, k, v, torch.from_numpy(lams).to(dev), g, kv_in=s0, dkv_out=dsn,
                             out_dtype=torch.float32, dkv_in=ds_out)
    torch.cuda.synchronize()
    if in_place:
        assert ds0.data_ptr() == dsn.data_ptr()
    rq, rk, rv, rs = _grad_oracle(q, k, v, lams, g, s0, dsn_host)
    _check_heads(dq, rq, "dQ", H)
    _check_heads(dk, rk, "dK", H)
    _check_heads(dv, rv, "dV", H)
    ds_h = host(ds0)
    for h in range(H):
        tol.assert_state(ds_h[:, h], rs[:, h], "dS0 head %d" % h)


def test_bwd_gradient_burst_before_a_reverse_warm_up_window(dev):
    """The dK and dV passes run the tokens last first; with lam = 0.7 at
    chunk 256 (carry span 64) the reverse pass's second chunk starts at row
    255 and its warm-up window covers rows 256-319.  A burst in dO (and q) at
    row 321, just past that window in reverse order, makes the adjoint state
    the window leaves out ~1e10 times the window's own: the check flags the
    head in both passes and they are computed on the exact path, so dk, dv
    and dS0 match the oracle (as with LA_FLAG_EXACT)."""
    say("bwd: burst in dO and q at row 321, B1 H2 N512 d128 chunk 256, lam 0.7 / 0.3")
    B, H, n, d = 1, 2, 512, 128
    q, k, v = qkv_device(B, H, n, d, seed=180, device=dev)
    g = qkv_device(B, H, n, d, seed=181, device=dev)[0]
    g[:, :, 321] *= 1e5
    q[:, :, 321] *= 1e5
    lams = np.array([0.7, 0.3], dtype=np.float32)
    assert la.chunk_for(B, H, n, 64) == 256
    lam_t = torch.from_numpy(lams).to(dev)
    dq, dk, dv, ds0 = la.bwd(q, k, v, lam_t, g, out_dtype=torch.float32, dkv_in=True)
    xq, xk, xv, xs = la.bwd(q, k, v, lam_t, g, out_dtype=torch.float32, dkv_in=True, exact=True)
    torch.cuda.synchronize()
    rq, rk, rv, rs = _grad_oracle(q, k, v, lams, g, None, None)
    _check_heads(dq, rq, "dQ", H)
    _check_heads(dk, rk, "dK", H)
    _check_heads(dv, rv, "dV", H)
    for h in range(H):
        tol.assert_state(host(ds0)[:, h], rs[:, h], "dS0 head %d" % h)
    # head 0 was flagged in both reverse passes and ran the exact path's
    # kernels; head 1 (lam^64 ~ 3e-34) left out nothing that mattered
    assert torch.equal(dk[:, 0], xk[:, 0]) and torch.equal(dv[:, 0], xv[:, 0]) and torch.equal(ds0[:, 0], xs[:, 0])
