"""GPU parity of the decode step against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import long_context_decayed_amd as la
import oracle as ora
from long_context_decayed_amd.inputs import decay_lambdas, qkv_device, state_device
import tolerances as tol
from gpu_helpers import host, lam_for, oracle, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _tokens(b, h, d, seed, dev):
    q, k, v = qkv_device(b, h, 1, d, seed=seed, device=dev)
    return q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), v[:, :, 0].contiguous()


def test_decode_large_batch(dev):
    """4096 sequences x 64 heads (16 GiB of fp32 state, 262,144 pairs) in one
    in-place step: 64 seeded (sequence, head) pairs against the oracle."""
    B, H, d = 4096, 64, 128
    say("decode large batch B4096 H64 d128")
    q, k, v = _tokens(B, H, d, 91, dev)
    lam = decay_lambdas(H)
    s = state_device(B, H, d, seed=91, device=dev)
    rng = np.random.default_rng(91)
    pick = rng.choice(B * H, size=64, replace=False)
    bs, hs = pick // H, pick % H
    s0 = np.stack([host(s[b, h]) for b, h in zip(bs, hs)]).astype(np.float64)
    o = la.decode_step(q, k, v, torch.from_numpy(lam).to(dev), s, s)
    torch.cuda.synchronize()
    sel = lambda x: np.stack([host(x[b, h]) for b, h in zip(bs, hs)])
    o_ref, s_ref = ora.decode_step(sel(q), sel(k), sel(v), lam[hs].astype(np.float64), s0)
    tol.assert_bf16_out(sel(o), o_ref)
    tol.assert_state(sel(s), s_ref)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_one_step(dev, d):
    say("decode one step B256 H64 d", d)
    B, H = 256, 64
    q, k, v = _tokens(B, H, d, 4, dev)
    lam = decay_lambdas(H)
    s0 = state_device(B, H, d, seed=4, device=dev)
    s_in = host(s0).astype(np.float64)
    kv = torch.empty_like(s0)
    o = la.decode_step(q, k, v, torch.from_numpy(lam).to(dev), kv_in=s0, kv_out=kv)
    torch.cuda.synchronize()
    o_ref, s_ref = ora.decode_step(host(q), host(k), host(v), lam.astype(np.float64), s_in)
    tol.assert_state(host(kv), s_ref)
    tol.assert_bf16_out(host(o), o_ref)
    # k_i v_j of two bf16 values is exact in fp32: the only state rounding is
    # lam*S + kv in fp32, so the state is far inside the tolerance
    assert tol.state_error(host(kv), s_ref) < 1e-6


def test_decode_1000_steps_closed_form(dev):
    say("decode 1000 steps in place B256 H64 d128")
    B, H, d = 256, 64, 128
    q, k, v = _tokens(B, H, d, 5, dev)
    lam = decay_lambdas(H)
    s = state_device(B, H, d, seed=5, device=dev)
    s_in = host(s).astype(np.float64)
    lam_t = torch.from_numpy(lam).to(dev)
    for _ in range(1000):
        o = la.decode_step(q, k, v, lam_t, kv_in=s, kv_out=s)
    torch.cuda.synchronize()
    s_ref = ora.decode_repeated(s_in, host(k), host(v), lam.astype(np.float64), 1000)
    tol.assert_state(host(s), s_ref)
    o_ref = np.einsum("bhi,bhij->bhj", host(q).astype(np.float64), s_ref)
    tol.assert_bf16_out(host(o), o_ref)


@pytest.mark.parametrize("mode", ["one", "near_one"])
def test_decode_many_steps_lam_one(dev, mode):
    say("decode 300 steps lam", mode)
    B, H, d = 4, 8, 128
    q, k, v = _tokens(B, H, d, 6, dev)
    lam = lam_for(H, mode)
    s = state_device(B, H, d, seed=6, device=dev)
    s_in = host(s).astype(np.float64)
    lam_t = torch.from_numpy(lam).to(dev)
    for _ in range(300):
        la.decode_step(q, k, v, lam_t, kv_in=s, kv_out=s)
    torch.cuda.synchronize()
    tol.assert_state(host(s), ora.decode_repeated(s_in, host(k), host(v), lam.astype(np.float64), 300))


def test_decode_zero_state_and_no_kv_out(dev):
    say("decode kv_in=None kv_out=None")
    B, H, d = 3, 5, 64
    q, k, v = _tokens(B, H, d, 7, dev)
    lam = decay_lambdas(H)
    o = la.decode_step(q, k, v, torch.from_numpy(lam).to(dev))
    torch.cuda.synchronize()
    o_ref, _ = ora.decode_step(host(q), host(k), host(v), lam.astype(np.float64), np.zeros((B, H, d, d)))
    tol.assert_bf16_out(host(o), o_ref)


def test_prefill_then_decode_matches_longer_prefill(dev):
    say("fwd(N) + decode == fwd(N+1) B2 H4 N513 d128")
    B, H, d, n = 2, 4, 128, 513
    q, k, v = qkv_device(B, H, n + 1, d, seed=8, device=dev)
    lam = decay_lambdas(H)
    lam_t = torch.from_numpy(lam).to(dev)
    kv = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    la.fwd(q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous(), lam_t, kv_out=kv,
           block=64)
    o_dec = la.decode_step(q[:, :, n].contiguous(), k[:, :, n].contiguous(), v[:, :, n].contiguous(), lam_t,
                           kv_in=kv, kv_out=kv)
    kv_full = torch.empty_like(kv)
    o_full = la.fwd(q, k, v, lam_t, kv_out=kv_full, block=64, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam)
    tol.assert_bf16_out(host(o_dec), o_ref[:, :, n], ref_rms=tol.rms(o_ref))
    tol.assert_bf16_f32out(host(o_full), o_ref)
    tol.assert_state(host(kv), s_ref)
    tol.assert_state(host(kv_full), s_ref)
    # decode == fwd with N = 1 (both against the oracle)
    o1 = la.fwd(q[:, :, :1].contiguous(), k[:, :, :1].contiguous(), v[:, :, :1].contiguous(), lam_t,
                kv_in=kv_full, block=64, out_dtype=torch.float32)
    o2 = la.decode_step(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), v[:, :, 0].contiguous(), lam_t,
                        kv_in=kv_full)
    torch.cuda.synchronize()
    r1, _ = ora.decode_step(host(q[:, :, 0]), host(k[:, :, 0]), host(v[:, :, 0]), lam.astype(np.float64),
                            host(kv_full).astype(np.float64))
    tol.assert_bf16_f32out(host(o1)[:, :, 0], r1)
    tol.assert_bf16_out(host(o2), r1)


# --- serving form: a pool of states addressed through a slot table ---------

@pytest.mark.parametrize("d", [64, 128])
def test_decode_slots_against_oracle(dev, d):
    say("decode over a slot table, pool 12 x H8 d", d)
    H, P = 8, 12
    slots_h = np.array([5, 0, -1, 11, 3, 12, 7], dtype=np.int32)  # -1 and 12: idle rows
    B = len(slots_h)
    q, k, v = _tokens(B, H, d, 6, dev)
    lam = lam_for(H, "spec")
    pool = state_device(P, H, d, seed=6, device=dev)
    pool0 = host(pool).astype(np.float64)
    slots = torch.from_numpy(slots_h).to(dev)
    o = la.decode_slots(q, k, v, torch.from_numpy(lam).to(dev), pool, slots)
    torch.cuda.synchronize()
    active = [(b, int(s)) for b, s in enumerate(slots_h) if 0 <= s < P]
    rows = np.array([b for b, _ in active])
    sl = np.array([s for _, s in active])
    o_ref, s_ref = ora.decode_step(host(q)[rows], host(k)[rows], host(v)[rows], lam.astype(np.float64), pool0[sl])
    tol.assert_bf16_out(host(o)[rows], o_ref)
    pool1 = host(pool).astype(np.float64)
    tol.assert_state(pool1[sl], s_ref)
    idle = [b for b in range(B) if b not in rows]
    assert np.all(host(o)[idle] == 0.0), "idle rows must be zero"
    untouched = [s for s in range(P) if s not in sl]
    assert np.array_equal(pool1[untouched], pool0[untouched]), "slots not named must not change"


def test_decode_slots_identity_matches_decode_step(dev):
    say("decode_slots with slots = 0..B-1 vs decode_step, B64 H64 d128")
    B, H, d = 64, 64, 128
    q, k, v = _tokens(B, H, d, 7, dev)
    lam_t = torch.from_numpy(decay_lambdas(H)).to(dev)
    s0 = state_device(B, H, d, seed=7, device=dev)
    pool = s0.clone()
    kv = torch.empty_like(s0)
    o1 = la.decode_step(q, k, v, lam_t, kv_in=s0, kv_out=kv)
    o2 = la.decode_slots(q, k, v, lam_t, pool, torch.arange(B, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(kv, pool)


def test_decode_slots_interleaved_requests(dev):
    # Three steps with different request sets: each slot's state must follow
    # the recurrence over exactly the tokens its rows brought, in order.
    say("decode_slots: 3 steps of interleaved requests, pool 6 x H4 d64")
    H, P, d = 4, 6, 64
    lam = lam_for(H, "spec")
    lam_t = torch.from_numpy(lam).to(dev)
    pool = state_device(P, H, d, seed=8, device=dev)
    ref = host(pool).astype(np.float64)
    tables = [np.array([0, 2, 4], np.int32), np.array([4, 1, -1, 0], np.int32), np.array([3, 4], np.int32)]
    for step, tab in enumerate(tables):
        q, k, v = _tokens(len(tab), H, d, 20 + step, dev)
        o = la.decode_slots(q, k, v, lam_t, pool, torch.from_numpy(tab).to(dev))
        torch.cuda.synchronize()
        for b, s in enumerate(tab):
            if s < 0:
                assert np.all(host(o)[b] == 0.0)
                continue
            o_ref, s_new = ora.decode_step(host(q)[b:b + 1], host(k)[b:b + 1], host(v)[b:b + 1],
                                           lam.astype(np.float64), ref[s:s + 1])
            ref[s] = s_new[0]
            tol.assert_bf16_out(host(o)[b:b + 1], o_ref)
    tol.assert_state(host(pool), ref)
