"""GPU parity of the prefill path against the fp64 oracle, through the C ABI.

Sizes run in seconds, span several tiles, blocks and chunks, and include
ragged tails.  Each case prints its name before touching the GPU."""
import math

import numpy as np
import pytest
import torch

import long_context_decayed_amd as la
from long_context_decayed_amd.inputs import (decay_lambdas, decay_lambdas_depth, qkv_cpu, qkv_device, state_device,
                                             ternary_device)
import tolerances as tol
from gpu_helpers import host, lam_for, oracle, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _run(q, k, v, lam_np, dev, block, out_dtype=None, kv_in=None, chunk=0, want_kv=True):
    lam = torch.from_numpy(lam_np).to(dev)
    B, H, N, d = q.shape
    kv_out = torch.empty((B, H, d, d), device=dev, dtype=torch.float32) if want_kv else None
    out = la.fwd(q, k, v, lam, kv_in=kv_in, kv_out=kv_out, block=block, out_dtype=out_dtype, chunk=chunk)
    torch.cuda.synchronize()
    return out, kv_out


# --- fp32 workload: B=1, H=2, N=1024, d=64, block 64, seed 0 ---------------

@pytest.mark.parametrize("chunk", [0, 64, 1024])
def test_fp32_tiny_workload(dev, chunk):
    say("fp32 B1 H2 N1024 d64 block64 chunk", chunk)
    q, k, v = (t.to(dev) for t in qkv_cpu(1, 2, 1024, 64, seed=0))
    lam = decay_lambdas(2)
    out, kv = _run(q, k, v, lam, dev, 64, chunk=chunk)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam)
    tol.assert_fp32(host(out), o_ref)
    tol.assert_fp32(host(kv), s_ref, "kv_out")


@pytest.mark.parametrize("block", [64, 128, 256])
def test_fp32_d64_blocks_with_state(dev, block):
    say("fp32 B2 H3 N777 d64 block", block)
    q, k, v = (t.to(dev) for t in qkv_cpu(2, 3, 777, 64, seed=5))
    lam = np.array([0.5, 0.9, 0.999], dtype=np.float32)
    s0 = state_device(2, 3, 64, seed=5, device=dev)
    out, kv = _run(q, k, v, lam, dev, block, kv_in=s0, chunk=2 * block)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam, host(s0).astype(np.float64))
    tol.assert_fp32(host(out), o_ref)
    tol.assert_fp32(host(kv), s_ref, "kv_out")


def test_fp32_d128(dev):
    say("fp32 B1 H2 N600 d128 block64")
    q, k, v = (t.to(dev) for t in qkv_cpu(1, 2, 600, 128, seed=6))
    lam = np.array([0.7, 0.99], dtype=np.float32)
    out, kv = _run(q, k, v, lam, dev, 64, chunk=128)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam)
    tol.assert_fp32(host(out), o_ref)
    tol.assert_fp32(host(kv), s_ref, "kv_out")


# --- integer-exact check: lam = 1, entries in {-1, 0, 1} ---------------------
# Every partial sum is an integer below 2^24 in magnitude, so fp32 arithmetic
# (and the bf16 hi/lo splits of integers below 2^16) is exact.

def test_ternary_exact_fp32(dev):
    say("ternary fp32 lam=1 B1 H2 N1024 d64")
    q, k, v = ternary_device(1, 2, 1024, 64, seed=1, device=dev, dtype=torch.float32)
    lam = lam_for(2, "one")
    out, kv = _run(q, k, v, lam, dev, 64, chunk=256)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam)
    assert np.array_equal(host(out).astype(np.float64), o_ref)
    assert np.array_equal(host(kv).astype(np.float64), s_ref)


@pytest.mark.parametrize("lams", ["one", "zero_one"])
@pytest.mark.parametrize("block", [64, 128, 256])
def test_ternary_exact_bf16_f32out(dev, block, lams):
    # lam = 0 keeps only the diagonal term q_r.k_r v_r (0^0 = 1), still exact;
    # with block 64 that head takes the warm-start pass with no warm-up.
    say("ternary bf16->f32 lam", lams, "B1 H2 N1024 d128 block", block)
    q, k, v = ternary_device(1, 2, 1024, 128, seed=2, device=dev, dtype=torch.bfloat16)
    lam = lam_for(2, "one") if lams == "one" else np.array([0.0, 1.0], dtype=np.float32)
    out, kv = _run(q, k, v, lam, dev, block, out_dtype=torch.float32, chunk=256 if block < 256 else 512)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam)
    assert np.array_equal(host(out).astype(np.float64), o_ref)
    assert np.array_equal(host(kv).astype(np.float64), s_ref)


# --- bf16: one layer shaped like the 64-head model, N = 8192 ---------------

@pytest.fixture(scope="module")
def layer_8k(dev):
    say("bf16 B1 H64 N8192 d128 block256 (inputs + oracle)")
    q, k, v = qkv_device(1, 64, 8192, 128, seed=1, device=dev)
    lam = decay_lambdas(64)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam)
    return q, k, v, lam, o_ref, s_ref


def test_bf16_layer_8k(dev, layer_8k):
    q, k, v, lam, o_ref, s_ref = layer_8k
    say("bf16 B1 H64 N8192 block256: fp32-out and bf16-out")
    o32, kv32 = _run(q, k, v, lam, dev, 256, out_dtype=torch.float32)
    o16, kv16 = _run(q, k, v, lam, dev, 256, out_dtype=torch.bfloat16)
    e = tol.assert_bf16_f32out(host(o32), o_ref)
    tol.assert_bf16_out(host(o16), o_ref)
    assert torch.equal(o32.to(torch.bfloat16), o16), "bf16 out must be RNE(fp32 out)"
    es = tol.assert_state(host(kv32), s_ref, "kv_out")
    assert torch.equal(kv32, kv16)
    print("max|err|/RMS = %.4e  (bf16 out: %.4e)  state rel = %.3e" % (
        e, tol.bf16_rms_error(host(o16), o_ref), es))


@pytest.mark.parametrize("block,chunk", [(64, 64), (64, 1024), (128, 512), (256, 256), (256, 2048)])
def test_bf16_layer_8k_block_chunk_invariance(dev, layer_8k, block, chunk):
    q, k, v, lam, o_ref, s_ref = layer_8k
    say("bf16 B1 H64 N8192 block", block, "chunk", chunk)
    o32, kv = _run(q, k, v, lam, dev, block, out_dtype=torch.float32, chunk=chunk)
    tol.assert_bf16_f32out(host(o32), o_ref)
    tol.assert_state(host(kv), s_ref, "kv_out")


def test_bf16_deterministic(dev, layer_8k):
    q, k, v, lam, _, _ = layer_8k
    say("bf16 determinism")
    a, ka = _run(q, k, v, lam, dev, 256)
    b, kb = _run(q, k, v, lam, dev, 256)
    assert torch.equal(a, b) and torch.equal(ka, kb)


# --- ragged tails, initial state, state carry, in-place state ----------------

@pytest.mark.parametrize("block,d", [(128, 128), (64, 128), (64, 64)])
@pytest.mark.parametrize("n", [1, 63, 65, 1000, 4097 + 13])
def test_bf16_tails_with_state(dev, n, block, d):
    say("bf16 tails B2 H4 N", n, "d", d, "block", block)
    q, k, v = qkv_device(2, 4, n, d, seed=10 + n, device=dev)
    lam = decay_lambdas(4)
    s0 = state_device(2, 4, d, seed=10 + n, device=dev)
    o32, kv = _run(q, k, v, lam, dev, block, out_dtype=torch.float32, kv_in=s0, chunk=256)
    o16, kv16 = _run(q, k, v, lam, dev, block, out_dtype=torch.bfloat16, kv_in=s0, chunk=256)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam, host(s0).astype(np.float64))
    tol.assert_bf16_f32out(host(o32), o_ref)
    tol.assert_state(host(kv), s_ref, "kv_out")
    assert torch.equal(o32.to(torch.bfloat16), o16), "bf16 out must be RNE(fp32 out)"
    assert torch.equal(kv, kv16)


def test_bf16_many_heads_short_sequences(dev):
    """32,768 (batch, head) pairs of 200 tokens in one call (one chunk each;
    the decays of the 64-head workload, so fast heads take the warm start and
    the slowest the exact path), with initial and final states: 64 seeded
    pairs against the oracle."""
    B, H, n, d = 512, 64, 200, 128
    say("many heads: B512 H64 N200 d128 with states")
    q, k, v = qkv_device(B, H, n, d, seed=77, device=dev)
    lam = decay_lambdas(H)
    s0 = state_device(B, H, d, seed=77, device=dev)
    o32, kv = _run(q, k, v, lam, dev, 64, out_dtype=torch.float32, kv_in=s0)
    rng = np.random.default_rng(77)
    pick = rng.choice(B * H, size=64, replace=False)
    bs, hs = pick // H, pick % H
    sel = lambda x: np.stack([host(x[b, h]) for b, h in zip(bs, hs)])
    o_ref, s_ref = oracle(sel(q), sel(k), sel(v), lam[hs], sel(s0).astype(np.float64))
    tol.assert_bf16_f32out(sel(o32), o_ref)
    tol.assert_state(sel(kv), s_ref, "kv_out")


@pytest.mark.parametrize("t0", [512, 700])
def test_bf16_state_carry(dev, t0):
    say("bf16 state carry B1 H4 N2048 split", t0)
    n = 2048
    q, k, v = qkv_device(1, 4, n, 128, seed=20, device=dev)
    lam = lam_for(4, "near_one")
    s0 = state_device(1, 4, 128, seed=20, device=dev)
    full, kv_full = _run(q, k, v, lam, dev, 64, out_dtype=torch.float32, kv_in=s0)
    a, kv_a = _run(q[:, :, :t0].contiguous(), k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous(), lam, dev, 64,
                   out_dtype=torch.float32, kv_in=s0)
    b, kv_b = _run(q[:, :, t0:].contiguous(), k[:, :, t0:].contiguous(), v[:, :, t0:].contiguous(), lam, dev, 64,
                   out_dtype=torch.float32, kv_in=kv_a)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam, host(s0).astype(np.float64))
    split = np.concatenate([host(a), host(b)], axis=2)
    tol.assert_bf16_f32out(split, o_ref)
    tol.assert_bf16_f32out(host(full), o_ref)
    tol.assert_state(host(kv_b), s_ref)
    tol.assert_state(host(kv_full), s_ref)


def test_bf16_state_in_place(dev):
    say("bf16 kv_in is kv_out")
    q, k, v = qkv_device(1, 4, 1500, 64, seed=30, device=dev)
    lam = decay_lambdas(4)
    s0 = state_device(1, 4, 64, seed=30, device=dev)
    s_host = host(s0).astype(np.float64)
    out = la.fwd(q, k, v, torch.from_numpy(lam).to(dev), kv_in=s0, kv_out=s0, block=64, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam, s_host)
    tol.assert_bf16_f32out(host(out), o_ref)
    tol.assert_state(host(s0), s_ref)


# --- heads that decay within a chunk, next to heads that do not --------------
# Chunk 1024, block 64, bf16 inputs.  A head whose start-state weight lam^(r+1)
# falls below 2^-30 within half a chunk (here lam <= 0.9) is computed per
# chunk from the state that the preceding carry-span tokens build from zero;
# the others take the three-pass path.  Each head is held to the tolerance on
# its own RMS, so the fast-decaying heads are not hidden behind the large
# outputs of the lam ~ 1 heads.

MIXED_LAMS = np.array([0.0, 1e-3, 0.3, 0.7, 0.9, 0.97, 0.999, 1.0], dtype=np.float32)


@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 63, 700, 2048, 2048 + 100, 3000 + 37])
def test_bf16_mixed_decays(dev, n, d, with_state):
    B, H = 2, 8
    say("bf16 mixed decays B2 H8 N", n, "d", d, "kv_in", with_state, "chunk 1024 block 64")
    q, k, v = qkv_device(B, H, n, d, seed=50 + n, device=dev)
    s0 = state_device(B, H, d, seed=50 + n, device=dev) if with_state else None
    o32, kv = _run(q, k, v, MIXED_LAMS, dev, 64, out_dtype=torch.float32, kv_in=s0, chunk=1024)
    o16, kv16 = _run(q, k, v, MIXED_LAMS, dev, 64, out_dtype=torch.bfloat16, kv_in=s0, chunk=1024)
    o_ref, s_ref = oracle(host(q), host(k), host(v), MIXED_LAMS, None if s0 is None else host(s0).astype(np.float64))
    o_h, kv_h = host(o32), host(kv)
    for h in range(H):
        tol.assert_bf16_f32out(o_h[:, h], o_ref[:, h], "O head %d (lam %g)" % (h, MIXED_LAMS[h]))
        tol.assert_state(kv_h[:, h], s_ref[:, h], "kv_out head %d (lam %g)" % (h, MIXED_LAMS[h]))
    assert torch.equal(o32.to(torch.bfloat16), o16), "bf16 out must be RNE(fp32 out)"
    assert torch.equal(kv, kv16)


def test_bf16_mixed_decays_state_in_place(dev):
    # kv_in is kv_out: the first chunk of a fast head reads kv_in, and its final
    # state reaches kv_out only after every chunk is done.
    say("bf16 mixed decays in place B2 H8 N4100 d128 chunk 1024")
    q, k, v = qkv_device(2, 8, 4100, 128, seed=70, device=dev)
    s0 = state_device(2, 8, 128, seed=70, device=dev)
    s_host = host(s0).astype(np.float64)
    out = la.fwd(q, k, v, torch.from_numpy(MIXED_LAMS).to(dev), kv_in=s0, kv_out=s0, block=64,
                 out_dtype=torch.float32, chunk=1024)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle(host(q), host(k), host(v), MIXED_LAMS, s_host)
    o_h, s_h = host(out), host(s0)
    for h in range(8):
        tol.assert_bf16_f32out(o_h[:, h], o_ref[:, h], "O head %d" % h)
        tol.assert_state(s_h[:, h], s_ref[:, h], "kv head %d" % h)


def test_bf16_mixed_decays_chunk_invariance(dev):
    # The split between the two paths moves with the chunk size; the results
    # must not (up to rounding).
    say("bf16 mixed decays B1 H8 N5000 d128: chunk 256 / 1024 / 4096")
    q, k, v = qkv_device(1, 8, 5000, 128, seed=60, device=dev)
    s0 = state_device(1, 8, 128, seed=60, device=dev)
    o_ref, s_ref = oracle(host(q), host(k), host(v), MIXED_LAMS, host(s0).astype(np.float64))
    for chunk in (256, 1024, 4096):
        o32, kv = _run(q, k, v, MIXED_LAMS, dev, 64, out_dtype=torch.float32, kv_in=s0, chunk=chunk)
        o_h, kv_h = host(o32), host(kv)
        for h in range(8):
            tol.assert_bf16_f32out(o_h[:, h], o_ref[:, h], "O chunk %d head %d" % (chunk, h))
            tol.assert_state(kv_h[:, h], s_ref[:, h], "kv_out chunk %d head %d" % (chunk, h))


# --- long-range carries: lam = 1 and just below 1 -----------------------------

@pytest.mark.parametrize("mode", ["one", "near_one"])
def test_bf16_long_range_carry(dev, mode):
    say("bf16 long range lam", mode, "B1 H2 N65536+100")
    n = 65536 + 100
    q, k, v = qkv_device(1, 2, n, 128, seed=40, device=dev)
    lam = lam_for(2, mode)
    o32, kv = _run(q, k, v, lam, dev, 256, out_dtype=torch.float32, chunk=4096)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam)
    tol.assert_bf16_f32out(host(o32), o_ref)
    tol.assert_state(host(kv), s_ref)


# --- prefill into a pool of states (serving) ----------------------------------

@pytest.mark.parametrize("block,n", [(64, 100), (64, 2048 + 37), (256, 700)])
def test_fwd_slots_against_oracle(dev, block, n):
    say("prefill into a state pool: pool 10 x H8, rows -> slots [7, 2, -1, 9], N", n, "block", block)
    H, P, d = 8, 10, 64
    slots_h = np.array([7, 2, -1, 9], dtype=np.int32)
    B = len(slots_h)
    q, k, v = qkv_device(B, H, n, d, seed=100 + n, device=dev)
    pool = state_device(P, H, d, seed=100 + n, device=dev)
    pool0 = host(pool).astype(np.float64)
    o = la.fwd_slots(q, k, v, torch.from_numpy(MIXED_LAMS).to(dev), pool, torch.from_numpy(slots_h).to(dev),
                     block=block, out_dtype=torch.float32)
    torch.cuda.synchronize()
    pool1 = host(pool).astype(np.float64)
    for b, s in enumerate(slots_h):
        s0 = pool0[s] if 0 <= s < P else None
        o_ref, s_ref = oracle(host(q)[b], host(k)[b], host(v)[b], MIXED_LAMS, s0)
        for h in range(H):
            tol.assert_bf16_f32out(host(o)[b, h], o_ref[h], "row %d head %d" % (b, h))
            if 0 <= s < P:
                tol.assert_state(pool1[s, h], s_ref[h], "slot %d head %d" % (s, h))
    untouched = [s for s in range(P) if s not in slots_h]
    assert np.array_equal(pool1[untouched], pool0[untouched]), "slots not named must not change"


def test_fwd_slots_identity_matches_fwd(dev):
    say("fwd_slots with slots = 0..B-1 vs fwd with kv_in = kv_out, B3 H8 N3000")
    B, H, n, d = 3, 8, 3000, 128
    q, k, v = qkv_device(B, H, n, d, seed=110, device=dev)
    lam_t = torch.from_numpy(MIXED_LAMS).to(dev)
    s0 = state_device(B, H, d, seed=110, device=dev)
    pool = s0.clone()
    o1 = la.fwd(q, k, v, lam_t, kv_in=s0, kv_out=s0, block=64)
    o2 = la.fwd_slots(q, k, v, lam_t, pool, torch.arange(B, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s0, pool)


# --- decays of a 70-layer stack, scaled down linearly with depth ---------------

@pytest.mark.parametrize("chunk", [0, 4096])
@pytest.mark.parametrize("layer", [0, 23, 46, 69])
def test_bf16_depth_scaled_decays(dev, layer, chunk):
    # The slopes shrink with depth, so deeper layers move heads from the
    # warm-start path to the three-pass path; the last layer has lam = 1.
    say("bf16 depth-scaled decays layer", layer, "of 70, B1 H64 N4133 d128 chunk", chunk)
    lam = decay_lambdas_depth(64, layer, 70)
    q, k, v = qkv_device(1, 64, 4133, 128, seed=120 + layer, device=dev)
    s0 = state_device(1, 64, 128, seed=120 + layer, device=dev)
    o32, kv = _run(q, k, v, lam, dev, 64, out_dtype=torch.float32, kv_in=s0, chunk=chunk)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam, host(s0).astype(np.float64))
    o_h, kv_h = host(o32), host(kv)
    for h in range(0, 64, 9):
        tol.assert_bf16_f32out(o_h[:, h], o_ref[:, h], "O head %d" % h)
    tol.assert_bf16_f32out(o_h, o_ref)
    tol.assert_state(kv_h, s_ref, "kv_out")


def test_bf16_classification_boundary(dev):
    # At chunk 1024 a head takes the warm-start path when its carry span (30 ln 2
    # / -ln lam rounded up to 64) is at most 512: lam with 30 ln 2 / -ln lam =
    # 511.5 and 512 sit on the warm-start side, 512.5 just past it (span 576).
    lams = np.array([math.exp(-30 * math.log(2) / t) for t in (448.2, 511.5, 512.0, 512.5)], dtype=np.float32)
    say("bf16 decays at the warm-start boundary, chunk 1024, B2 H4 N5000 d128, with state")
    q, k, v = qkv_device(2, 4, 5000, 128, seed=130, device=dev)
    s0 = state_device(2, 4, 128, seed=130, device=dev)
    o32, kv = _run(q, k, v, lams, dev, 64, out_dtype=torch.float32, kv_in=s0, chunk=1024)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lams, host(s0).astype(np.float64))
    o_h, kv_h = host(o32), host(kv)
    for h in range(4):
        tol.assert_bf16_f32out(o_h[:, h], o_ref[:, h], "O head %d (lam %.7f)" % (h, lams[h]))
        tol.assert_state(kv_h[:, h], s_ref[:, h], "kv_out head %d" % h)


# --- the exact path on demand --------------------------------------------------

def _warm_flags(ws, B, H):
    """The warm-start check's per-(b, h) flags: the last B*H int32 of the
    workspace (its documented layout)."""
    return ws[ws.numel() - 4 * B * H:].view(torch.int32).cpu().numpy()


def test_spike_before_the_warm_up_window_is_caught(dev):
    # lam = 0.7 at chunk 256 takes the warm start (carry span 64): chunk 1
    # starts from zero at token 192.  A token at 190 whose k and v are 1e5
    # times the others still weighs lam^66 * 1e10 ~ 0.6 of a typical term on
    # the first rows of chunk 1.  The warm-start check sees the left-out state
    # far above 2^-24 of the window's own, flags the head and runs it on the
    # exact path: the default entry point matches the oracle there, as the
    # exact flag does.
    say("spike before the warm-up window, B1 H1 N512 d128 chunk 256: default and exact flag")
    q, k, v = qkv_device(1, 1, 512, 128, seed=140, device=dev)
    k[:, :, 190] *= 1e5
    v[:, :, 190] *= 1e5
    lam = np.array([0.7], dtype=np.float32)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam)
    lam_d = torch.from_numpy(lam).to(dev)
    ws = torch.empty(la.workspace_bytes(1, 1, 512, 128, 64, 256), device=dev, dtype=torch.uint8)
    kv = torch.empty((1, 1, 128, 128), device=dev, dtype=torch.float32)
    default = la.fwd(q, k, v, lam_d, kv_out=kv, block=64, chunk=256, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    flags = _warm_flags(ws, 1, 1)
    exact = la.fwd(q, k, v, lam_d, block=64, chunk=256, out_dtype=torch.float32, exact=True)
    torch.cuda.synchronize()
    assert flags.tolist() == [1], flags
    rows = slice(256, 320)
    for name, o in (("default", default), ("exact", exact)):
        tol.assert_bf16_f32out(host(o)[:, :, rows], o_ref[:, :, rows], "%s, rows 256-319" % name)
        tol.assert_bf16_f32out(host(o), o_ref, name)
    tol.assert_state(host(kv), s_ref, "kv_out")
    # the flagged head ran the exact path: the same kernels as the exact flag
    assert torch.equal(default, exact)


def test_warm_up_window_of_zeros_is_caught(dev):
    # Keys of zero over chunk 1's whole warm-up window [192, 256): the window
    # builds no state at all, so any earlier state is not negligible against
    # it and the head runs on the exact path.
    say("zero keys over the warm-up window, B1 H2 N700 d64 chunk 256, with state")
    q, k, v = qkv_device(1, 2, 700, 64, seed=141, device=dev)
    k[:, :, 192:256] = 0
    lam = np.array([0.7, 0.3], dtype=np.float32)
    s0 = state_device(1, 2, 64, seed=141, device=dev)
    ws = torch.empty(la.workspace_bytes(1, 2, 700, 64, 64, 256), device=dev, dtype=torch.uint8)
    kv = torch.empty_like(s0)
    o = la.fwd(q, k, v, torch.from_numpy(lam).to(dev), kv_in=s0, kv_out=kv, block=64, chunk=256,
               out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    flags = _warm_flags(ws, 1, 2)
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam, host(s0).astype(np.float64))
    assert flags.tolist() == [1, 1], flags
    for h in range(2):
        tol.assert_bf16_f32out(host(o)[:, h], o_ref[:, h], "O head %d" % h)
        tol.assert_state(host(kv)[:, h], s_ref[:, h], "kv_out head %d" % h)


def test_nan_input_reaches_every_later_row(dev):
    # A NaN in one key entry of head 0 at token 100: in the exact function
    # the state's row for that feature is NaN from then on (lam^n NaN = NaN),
    # so every later output row of the head is NaN.  The warm start of the
    # chunks after it would start from finite windows; the check sees the
    # NaN in the state those windows leave out and sends the head to the
    # exact path, so no later row comes out finite.  Rows of the NaN's own
    # 64-token sub-tile before it are not specified: the blocked products
    # meet the NaN there (0 * NaN), as any blocked attention kernel does.
    # Head 1 has no NaN and stays on the warm start.
    say("NaN key at token 100 of head 0, B1 H2 N700 d64 chunk 256")
    q, k, v = qkv_device(1, 2, 700, 64, seed=151, device=dev)
    k[0, 0, 100, 5] = float("nan")
    lam = np.array([0.7, 0.7], dtype=np.float32)
    lam_d = torch.from_numpy(lam).to(dev)
    ws = torch.empty(la.workspace_bytes(1, 2, 700, 64, 64, 256), device=dev, dtype=torch.uint8)
    kv = torch.empty((1, 2, 64, 64), device=dev, dtype=torch.float32)
    o = la.fwd(q, k, v, lam_d, kv_out=kv, block=64, chunk=256, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    flags = _warm_flags(ws, 1, 2)
    kvx = torch.empty_like(kv)
    exact = la.fwd(q, k, v, lam_d, kv_out=kvx, block=64, chunk=256, out_dtype=torch.float32, exact=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam)
    assert flags.tolist() == [1, 0], flags
    og, kg = host(o), host(kv)
    assert np.isnan(o_ref[0, 0, 100:]).all() and np.isnan(og[0, 0, 100:]).all()
    tol.assert_bf16_f32out(og[0, 0, :64], o_ref[0, 0, :64], "head 0 before the NaN's sub-tile")
    tol.assert_bf16_f32out(og[0, 1], o_ref[0, 1], "head 1")
    assert np.array_equal(np.isnan(kg), np.isnan(s_ref)) and np.isnan(kg[0, 0, 5]).all()
    fin = ~np.isnan(s_ref)
    tol.assert_state(kg[fin], s_ref[fin], "finite state entries")
    # the flagged head ran the exact path: bit for bit the exact flag's result
    assert torch.equal(o[:, 0].view(torch.int32), exact[:, 0].view(torch.int32))
    assert torch.equal(kv[:, 0].view(torch.int32), kvx[:, 0].view(torch.int32))


def test_warm_start_check_passes_the_workloads(dev):
    """On the workloads' Gaussian inputs no head is flagged (the left-out
    state is about lam^span <= 2^-30 of the window's), at the 64-head
    8192-token layer and with the decays of deeper layers."""
    B, H, N, d = 1, 64, 8192, 128
    q, k, v = qkv_device(B, H, N, d, seed=1, device=dev)
    ws = torch.empty(la.workspace_bytes(B, H, N, d, 64), device=dev, dtype=torch.uint8)
    for layer in (0, 23, 46, 60):
        say("warm-start check on the B1 H64 N8192 d128 layer, decays of layer", layer, "of 70")
        lam = torch.from_numpy(decay_lambdas_depth(H, layer, 70)).to(dev)
        la.fwd(q, k, v, lam, block=64, workspace=ws)
        torch.cuda.synchronize()
        assert not _warm_flags(ws, B, H).any(), layer


def test_exact_flag_matches_oracle_on_mixed_decays(dev):
    say("exact flag: mixed decays B2 H8 N3037 d128 chunk 1024, with state")
    q, k, v = qkv_device(2, 8, 3037, 128, seed=150, device=dev)
    s0 = state_device(2, 8, 128, seed=150, device=dev)
    kv = torch.empty_like(s0)
    o = la.fwd(q, k, v, torch.from_numpy(MIXED_LAMS).to(dev), kv_in=s0, kv_out=kv, block=64, chunk=1024,
               out_dtype=torch.float32, exact=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle(host(q), host(k), host(v), MIXED_LAMS, host(s0).astype(np.float64))
    for h in range(8):
        tol.assert_bf16_f32out(host(o)[:, h], o_ref[:, h], "O head %d" % h)
        tol.assert_state(host(kv)[:, h], s_ref[:, h], "kv_out head %d" % h)


# decays whose carry spans (64, 128, 256, 448, 704, 1408, 4160 tokens, then none)
# put heads on either path as the warm-start chunk grows
SPAN_LAMS = np.array([0.3, 0.85, 0.9, 0.95, 0.97, 0.985, 0.995, 1.0], dtype=np.float32)


@pytest.mark.parametrize("warm_chunk", [512, 1024, 4096])
@pytest.mark.parametrize("in_place", [False, True])
def test_bf16_warm_chunk_longer_than_scan_chunk(dev, warm_chunk, in_place):
    """The warm-start pass on chunks of warm_chunk tokens, the other heads'
    scan and output passes on chunks of 256: every kernel must judge the heads
    alike and the warm-start pass must leave its final states where the scan
    looks for them (also with kv_in = kv_out)."""
    B, H, n, d = 2, 8, 5000, 128
    say("bf16 scan chunk 256, warm-start chunk", warm_chunk, "B2 H8 N5000 d128, in place", in_place)
    q, k, v = qkv_device(B, H, n, d, seed=80, device=dev)
    s0 = state_device(B, H, d, seed=80, device=dev)
    s_host = host(s0).astype(np.float64)
    kv = s0 if in_place else torch.empty_like(s0)
    out = la.fwd(q, k, v, torch.from_numpy(SPAN_LAMS).to(dev), kv_in=s0, kv_out=kv, block=64,
                 out_dtype=torch.float32, chunk=256, warm_chunk=warm_chunk)
    torch.cuda.synchronize()
    assert la.warm_chunk_for(B, H, n, 64, 256, warm_chunk) == warm_chunk
    o_ref, s_ref = oracle(host(q), host(k), host(v), SPAN_LAMS, s_host)
    o_h, s_h = host(out), host(kv)
    for h in range(H):
        tol.assert_bf16_f32out(o_h[:, h], o_ref[:, h], "O head %d (lam %g)" % (h, SPAN_LAMS[h]))
        tol.assert_state(s_h[:, h], s_ref[:, h], "kv head %d (lam %g)" % (h, SPAN_LAMS[h]))
