"""GPU parity at the full workload sizes, on samples the oracle can compute.

* Batched long prefill: B=4, H=64, N=65536, d=128, bf16, initial state
  N(0, 0.1^2) per (b, h): all outputs and final states of 16 seeded (b, h)
  pairs, plus the first 4096 tokens of every pair (where the initial state is
  still visible: lam_max^4096 = e^-16).
* Million-token layer: B=1, H=64, N=1,048,576: a seeded interior 8192-token
  slice and the final slice, each checked against (a) the oracle run from the
  GPU's own state at the slice start (kv_out of a GPU call on the prefix) and
  (b) a window oracle that starts 8192 tokens earlier from zero state, whose
  truncation error is at most lam_max^8193 = e^-32 of the state.
* Long-range carries: lam = 1 over 2^20 tokens (nothing decays, so every
  chunk's contribution reaches the end).
* The longest sequence the library takes, N = 2^24 (N * d = 2^31 at d = 128):
  a warm-start head and a lam = 1 head, final slice and state from the GPU's
  own prefix state.
* Backward of the million-token layer: the interior and the final slice of
  dq, dk, dv against the gradient oracle (prefix state from the GPU forward,
  a future window for the adjoint).
"""
import numpy as np
import pytest
import torch

import long_context_decayed_amd as la
import oracle as ora
from long_context_decayed_amd.inputs import decay_lambdas, qkv_device, state_device
import tolerances as tol
from gpu_helpers import host, lam_for, oracle, oracle_threads, require_gpu, say
from oracle import crec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _sample_pairs(b, h, n, seed):
    rng = np.random.default_rng(seed)
    flat = rng.choice(b * h, size=n, replace=False)
    return sorted((int(i // h), int(i % h)) for i in flat)


@pytest.mark.parametrize("block", [64, 256])
def test_batched_long_prefill(dev, block):
    B, H, N, d = 4, 64, 65536, 128
    say("batched prefill B4 H64 N65536 block", block)
    q, k, v = qkv_device(B, H, N, d, seed=2, device=dev, slice_tokens=16384)
    lam = decay_lambdas(H)
    s0 = state_device(B, H, d, seed=2, std=0.1, device=dev)
    kv = torch.empty_like(s0)
    out = la.fwd(q, k, v, torch.from_numpy(lam).to(dev), kv_in=s0, kv_out=kv, block=block,
                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    s0h = host(s0).astype(np.float64)
    # 16 whole (b, h) pairs
    pairs = _sample_pairs(B, H, 16, seed=2)
    qs = np.stack([host(q[b, h]) for b, h in pairs])
    ks = np.stack([host(k[b, h]) for b, h in pairs])
    vs = np.stack([host(v[b, h]) for b, h in pairs])
    lam_s = np.array([lam[h] for _, h in pairs], dtype=np.float32)
    s0_s = np.stack([s0h[b, h] for b, h in pairs])
    o_ref, s_ref = oracle(qs, ks, vs, lam_s, s0_s)
    o_gpu = np.stack([host(out[b, h]) for b, h in pairs])
    e = tol.assert_bf16_f32out(o_gpu, o_ref, "O (16 pairs)")
    es = tol.assert_state(np.stack([host(kv[b, h]) for b, h in pairs]), s_ref, "kv_out (16 pairs)")
    # early tokens of every pair: the initial state's contribution is visible there
    t1 = 4096
    o_e, _ = oracle(host(q[:, :, :t1]), host(k[:, :, :t1]), host(v[:, :, :t1]), lam, s0h, want_state=False)
    e2 = tol.assert_bf16_f32out(host(out[:, :, :t1]), o_e, "O (first 4096 tokens, all pairs)")
    # the initial state matters there: dropping it changes the result far beyond the tolerance
    o_z, _ = oracle(host(q[:, :, :64]), host(k[:, :, :64]), host(v[:, :, :64]), lam, None, want_state=False)
    assert tol.bf16_rms_error(o_z, o_e[:, :, :64], tol.rms(o_e)) > 10 * tol.BF16_RMS
    print("max|err|/RMS: pairs %.3e, early %.3e; state rel %.3e" % (e, e2, es))


@pytest.fixture(scope="module")
def million(dev):
    B, H, N, d = 1, 64, 1 << 20, 128
    say("million-token layer: inputs")
    q, k, v = qkv_device(B, H, N, d, seed=3, device=dev, slice_tokens=65536)
    lam = decay_lambdas(H)
    rng = np.random.default_rng(3)
    t0 = int(rng.integers(8192 // 64, (N - 8192) // 64)) * 64
    return q, k, v, lam, t0


def _slice_checks(q, k, v, lam, dev, out, t0, t1, block, w=8192):
    """Oracle over [t0, t1) from the GPU prefix state and from a zero-state window."""
    lam_t = torch.from_numpy(lam).to(dev)
    B, H, N, d = q.shape
    kv_pre = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    la.fwd(q[:, :, :t0].contiguous(), k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous(), lam_t, kv_out=kv_pre,
           block=block)
    torch.cuda.synchronize()
    qs, ks, vs = host(q[:, :, t0:t1]), host(k[:, :, t0:t1]), host(v[:, :, t0:t1])
    o_pref, s_pref = oracle(qs, ks, vs, lam, host(kv_pre).astype(np.float64))
    lo = max(0, t0 - w)
    o_win, s_win = oracle(host(q[:, :, lo:t1]), host(k[:, :, lo:t1]), host(v[:, :, lo:t1]), lam,
                          o_range=(t0 - lo, t1 - lo))
    o_gpu = host(out[:, :, t0:t1])
    e1 = tol.assert_bf16_f32out(o_gpu, o_pref, "slice vs oracle from GPU prefix state")
    e2 = tol.assert_bf16_f32out(o_gpu, o_win, "slice vs window oracle")
    # the two oracles agree far inside the tolerance (window truncation <= e^-32)
    assert tol.bf16_rms_error(o_pref, o_win, tol.rms(o_win)) < 1e-3
    return e1, e2, s_pref, s_win


@pytest.mark.parametrize("block", [64, 256])
def test_million_token_slices(dev, million, block):
    q, k, v, lam, t0 = million
    say("million-token layer block", block, "interior slice at", t0)
    N = q.shape[2]
    lam_t = torch.from_numpy(lam).to(dev)
    kv = torch.empty((1, 64, 128, 128), device=dev, dtype=torch.float32)
    out = la.fwd(q, k, v, lam_t, kv_out=kv, block=block, out_dtype=torch.float32)
    torch.cuda.synchronize()
    e1, e2, _, _ = _slice_checks(q, k, v, lam, dev, out, t0, t0 + 8192, block)
    # A slice across a chunk start: the rows whose outputs still depend on
    # the chunk's start state (up to about 5400 for the slowest head here).
    # At block 64 every head here takes the warm start, whose chunks are the
    # warm-start chunk length.
    L = la.warm_chunk_for(1, 64, N, block) if block == 64 else la.chunk_for(1, 64, N, block)
    tb = 5 * L - 2048
    say("million-token layer block", block, "chunk", L, "slice across the chunk start", 5 * L)
    g1, g2, _, _ = _slice_checks(q, k, v, lam, dev, out, tb, tb + 8192, block)
    say("million-token layer block", block, "final slice")
    f1, f2, s_pref, s_win = _slice_checks(q, k, v, lam, dev, out, N - 8192, N, block)
    tol.assert_state(host(kv), s_pref, "kv_out vs oracle from GPU prefix state")
    tol.assert_state(host(kv), s_win, "kv_out vs window oracle")
    # bf16 output of the same kernels is RNE of the fp32 output (interior slice)
    o16 = la.fwd(q, k, v, lam_t, block=block)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, t0:t0 + 8192].to(torch.bfloat16), o16[:, :, t0:t0 + 8192])
    print("interior %.3e / %.3e, chunk start %.3e / %.3e, final %.3e / %.3e (max|err|/RMS)" % (
        e1, e2, g1, g2, f1, f2))


def test_lambda_one_million_tokens(dev):
    say("lam = 1, B1 H2 N2^20")
    B, H, N, d = 1, 2, 1 << 20, 128
    q, k, v = qkv_device(B, H, N, d, seed=41, device=dev, slice_tokens=65536)
    lam = lam_for(H, "one")
    kv = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    out = la.fwd(q, k, v, torch.from_numpy(lam).to(dev), kv_out=kv, block=64, out_dtype=torch.float32)
    torch.cuda.synchronize()
    t0 = N - 4096
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam, o_range=(t0, N))
    tol.assert_bf16_f32out(host(out[:, :, t0:]), o_ref, "last 4096 rows")
    tol.assert_state(host(kv), s_ref)
    # closed-form state at the end (one GEMM, no recurrence): K^T V
    kh, vh = host(k).astype(np.float64), host(v).astype(np.float64)
    st = np.matmul(np.swapaxes(kh, -1, -2), vh)
    tol.assert_state(host(kv), st, "kv_out vs K^T V")


def test_max_sequence_length(dev):
    B, H, N, d = 1, 2, 1 << 24, 128
    say("longest sequence: B1 H2 N2^24 d128 (warm-start head and lam = 1 head)")
    q, k, v = qkv_device(B, H, N, d, seed=44, device=dev, slice_tokens=1 << 20)
    # head 0 (lam = 0.99610, carry span 5376 tokens) takes the warm start at
    # the 65536-token warm-start chunk of this shape; head 1 (lam = 1) the
    # exact path's lam = 1 kernels
    lam = np.array([decay_lambdas(64)[63], 1.0], dtype=np.float32)
    lam_t = torch.from_numpy(lam).to(dev)
    assert la.warm_chunk_for(B, H, N, 64) == 65536
    kv = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    out = la.fwd(q, k, v, lam_t, kv_out=kv, block=64, out_dtype=torch.float32)
    torch.cuda.synchronize()
    t0 = N - 8192
    kv_pre = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    la.fwd(q[:, :, :t0].contiguous(), k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous(), lam_t, kv_out=kv_pre,
           block=64)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle(host(q[:, :, t0:]), host(k[:, :, t0:]), host(v[:, :, t0:]), lam,
                          host(kv_pre).astype(np.float64))
    e = tol.assert_bf16_f32out(host(out[:, :, t0:]), o_ref, "last 8192 rows vs oracle from GPU prefix state")
    es = tol.assert_state(host(kv), s_ref, "kv_out")
    print("N = 2^24: last rows max|err|/RMS %.3e, state %.3e" % (e, es))


def test_million_token_backward_slices(dev, million):
    """Backward at the million-token size, on slices the oracle can compute.

    dq on [t0, t0+w) needs the forward state at t0: the oracle starts from the
    GPU forward's kv_out of the prefix.  dk and dv on the slice need the adjoint
    state from the future: the oracle runs the slice plus the next w tokens
    with a zero final-state gradient, whose truncation is at most lam_max^w =
    e^-32 of that state.  The last slice is exact (the sequence ends there)."""
    q, k, v, lam, t0 = million
    B, H, N, d = q.shape
    w = 8192
    lam_t = torch.from_numpy(lam).to(dev)
    g = qkv_device(B, H, N, d, seed=30, device=dev, slice_tokens=65536)[0]
    dq, dk, dv, _ = la.bwd(q, k, v, lam_t, g, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for a in (t0, N - w):
        say("million-token backward: slice at", a)
        kv_pre = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
        la.fwd(q[:, :, :a].contiguous(), k[:, :, :a].contiguous(), v[:, :, :a].contiguous(), lam_t, kv_out=kv_pre,
               block=64)
        torch.cuda.synchronize()
        b = min(N, a + 2 * w)
        sl = lambda x: host(x[:, :, a:b])
        rq, rk, rv, _ = crec.backward(sl(q), sl(k), sl(v), lam.astype(np.float64), sl(g),
                                      host(kv_pre).astype(np.float64), None, threads=oracle_threads())
        for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
            e = tol.assert_bf16_f32out(host(got[:, :, a:a + w]), ref[:, :, :w], "%s slice %d" % (name, a))
            print("%s slice at %d: max|err|/RMS %.3e" % (name, a, e))


def test_million_token_silu_fused_is_silu_pass_then_prefill(dev, million):
    """At the million-token size, in the bench's launch configuration (block
    64, default chunk): the prefill with SiLU fused into its tile loads equals,
    bit for bit, the SiLU pass over q, k, v followed by the plain prefill (the
    plain prefill is checked against the oracle on slices above)."""
    q, k, v, lam, _ = million
    B, H, N, d = q.shape
    lam_t = torch.from_numpy(lam).to(dev)
    say("million-token prefill: fused SiLU vs SiLU pass + prefill")
    kv1, kv2 = (torch.empty((B, H, d, d), device=dev, dtype=torch.float32) for _ in range(2))
    o1 = la.fwd(q, k, v, lam_t, kv_out=kv1, block=64, silu=True)
    acts = [la.silu_(t.clone()) for t in (q, k, v)]
    o2 = la.fwd(*acts, lam_t, kv_out=kv2, block=64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(kv1, kv2)
    del acts, o1, o2
    torch.cuda.empty_cache()
