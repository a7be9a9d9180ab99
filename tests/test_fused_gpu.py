"""GPU parity of the elementwise steps either side of the core (SiLU on
Q, K, V; per-head RMSNorm and sigmoid gate of the output) against the fp64
oracle: fused into the decode step, and as the prefill's own passes."""
import numpy as np
import pytest
import torch

import long_context_decayed_amd as la
import oracle as ora
from long_context_decayed_amd.inputs import decay_lambdas, qkv_device, state_device
import tolerances as tol
from gpu_helpers import host, oracle, require_gpu, say

pytestmark = pytest.mark.gpu
LAMS8 = np.array([0.0, 1e-3, 0.3, 0.7, 0.9, 0.97, 0.999, 1.0], dtype=np.float32)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _tok(b, h, d, seed, dev, scale=3.0):
    # pre-activation values: a wider spread than the core's inputs, so that
    # SiLU's bend near zero and its linear tail are both exercised
    q, k, v = qkv_device(b, h, 1, d, seed=seed, device=dev)
    return tuple((t[:, :, 0] * scale * d ** 0.5 / 4).to(torch.bfloat16).contiguous() for t in (q, k, v))


def _gamma(h, d, seed, dev):
    g = torch.Generator().manual_seed(seed)
    return (1.0 + 0.25 * torch.randn((h, d), generator=g)).to(torch.float32).to(dev)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_fused_against_oracle(dev, d):
    say("decode fused (silu, norm, gate) over a slot table, pool 9 x H8 d", d)
    H, P = 8, 9
    slots_h = np.array([4, -1, 0, 8, 2, 9, 6], dtype=np.int32)
    B = len(slots_h)
    q, k, v = _tok(B, H, d, 140 + d, dev)
    gate = _tok(B, H, d, 150 + d, dev)[0]
    gamma = _gamma(H, d, 160 + d, dev)
    pool = state_device(P, H, d, seed=140 + d, device=dev)
    pool0 = host(pool).astype(np.float64)
    o = la.decode_fused(q, k, v, torch.from_numpy(LAMS8).to(dev), pool, torch.from_numpy(slots_h).to(dev),
                        silu=True, gamma=gamma, gate=gate, eps=1e-5)
    torch.cuda.synchronize()
    act = [(b, int(s)) for b, s in enumerate(slots_h) if 0 <= s < P]
    rows = np.array([b for b, _ in act])
    sl = np.array([s for _, s in act])
    qs, ks, vs = (ora.silu(host(t)[rows]) for t in (q, k, v))
    o_core, s_ref = ora.decode_step(qs, ks, vs, LAMS8.astype(np.float64), pool0[sl])
    y = ora.rmsnorm_heads(o_core[:, :, None, :], host(gamma), eps=1e-5)[:, :, 0, :]
    y = ora.sigmoid_gate(y, host(gate)[rows])
    tol.assert_bf16_out(host(o)[rows], y)
    tol.assert_state(host(pool).astype(np.float64)[sl], s_ref)
    idle = [b for b in range(B) if b not in rows]
    assert np.all(host(o)[idle] == 0.0)


def test_decode_fused_without_steps_is_decode_slots(dev):
    say("decode fused with every step off vs decode_slots, B32 H64 d128")
    B, H, d = 32, 64, 128
    q, k, v = _tok(B, H, d, 170, dev, scale=1.0)
    lam_t = torch.from_numpy(decay_lambdas(H)).to(dev)
    pool_a = state_device(B, H, d, seed=170, device=dev)
    pool_b = pool_a.clone()
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    o1 = la.decode_slots(q, k, v, lam_t, pool_a, slots)
    o2 = la.decode_fused(q, k, v, lam_t, pool_b, None, silu=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(pool_a, pool_b)


@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_norm_gate_against_oracle(dev, d, odt):
    say("prefill norm + gate B2 H4 N1001 d", d, "o", odt)
    B, H, N = 2, 4, 1001
    o = qkv_device(B, H, N, d, seed=180 + d, device=dev, dtype=torch.float32)[0].to(odt) * 7.0
    gate = qkv_device(B, H, N, d, seed=190 + d, device=dev)[0] * 8.0
    gamma = _gamma(H, d, 200 + d, dev)
    y = la.norm_gate(o, gamma=gamma, gate=gate, eps=1e-5)
    torch.cuda.synchronize()
    ref = ora.sigmoid_gate(ora.rmsnorm_heads(host(o), host(gamma), eps=1e-5), host(gate))
    tol.assert_bf16_out(host(y), ref)
    # only the final rounding to bf16 (and fp32 arithmetic) separates them
    err = np.abs(host(y).astype(np.float64) - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max())
    # the norm alone, in place
    o2 = o.to(torch.bfloat16).contiguous()
    ref2 = ora.rmsnorm_heads(host(o2), host(gamma), eps=1e-5)
    la.norm_gate(o2, gamma=gamma, out=o2)
    torch.cuda.synchronize()
    assert np.all(np.abs(host(o2) - ref2) <= 2.0 ** -8 * np.abs(ref2) + 1e-6 * np.abs(ref2).max())


@pytest.mark.parametrize("n", [8, 13, 100003])
def test_silu_against_oracle(dev, n):
    say("silu in place, n", n)
    g = torch.Generator(device=dev).manual_seed(n)
    x = (torch.randn(n, device=dev, generator=g) * 4).to(torch.bfloat16)
    ref = ora.silu(host(x))
    la.silu_(x)
    torch.cuda.synchronize()
    assert np.all(np.abs(host(x) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


def test_layer_core_pipeline(dev):
    # pre-activations -> SiLU -> lightning prefill -> per-head norm and gate,
    # against the same chain in the oracle
    say("layer core pipeline B1 H8 N2000 d128: silu -> fwd -> norm_gate")
    B, H, N, d = 1, 8, 2000, 128
    q, k, v = (t * 2.0 for t in qkv_device(B, H, N, d, seed=210, device=dev))
    q, k, v = (t.contiguous() for t in (q, k, v))
    gate = qkv_device(B, H, N, d, seed=211, device=dev)[0] * 8.0
    gamma = _gamma(H, d, 212, dev)
    qa, ka, va = (la.silu_(t.clone()) for t in (q, k, v))
    o = la.fwd(qa, ka, va, torch.from_numpy(LAMS8).to(dev), block=64, out_dtype=torch.float32)
    y = la.norm_gate(o, gamma=gamma, gate=gate, eps=1e-5)
    torch.cuda.synchronize()
    # the oracle takes the GPU's bf16 SiLU outputs (the prefill's inputs) and
    # checks that step on its own
    for a, raw in ((qa, q), (ka, k), (va, v)):
        ref = ora.silu(host(raw))
        assert np.all(np.abs(host(a) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    o_ref, _ = oracle(host(qa), host(ka), host(va), LAMS8)
    y_ref = ora.sigmoid_gate(ora.rmsnorm_heads(o_ref, host(gamma), eps=1e-5), host(gate))
    for h in range(H):
        tol.assert_bf16_out(host(y)[:, h], y_ref[:, h], "head %d" % h)


def _preact(B, H, N, d, seed, dev, scale=2.5):
    # pre-activation projections: a wider spread than the core's inputs so
    # that SiLU's bend and both of its tails are exercised
    return tuple((t * scale).contiguous() for t in qkv_device(B, H, N, d, seed=seed, device=dev))


@pytest.mark.parametrize("d,N,odt,exact", [(128, 2500, torch.bfloat16, False), (128, 2500, torch.float32, False),
                                          (64, 1100, torch.float32, False), (128, 700, torch.float32, True),
                                          (128, 63, torch.bfloat16, False)])
def test_prefill_silu_fused_is_silu_pass_then_prefill(dev, d, N, odt, exact):
    """SiLU on the tiles as they load == the SiLU pass over q, k, v first, bit
    for bit (outputs and final state), on decays that take both the warm-start
    and the chunked paths (so the chunk-aggregate kernel's SiLU is covered),
    with an initial state and a ragged last tile; q, k, v are left unchanged."""
    say("prefill + fused SiLU vs SiLU pass + prefill: B2 H8 N", N, "d", d, odt, "exact", exact)
    B, H = 2, 8
    q, k, v = _preact(B, H, N, d, 300 + d + N, dev)
    keep = [t.clone() for t in (q, k, v)]
    s0 = state_device(B, H, d, seed=301, device=dev)
    lam = torch.from_numpy(LAMS8).to(dev)
    kv1, kv2 = (torch.empty((B, H, d, d), device=dev, dtype=torch.float32) for _ in range(2))
    o1 = la.fwd(q, k, v, lam, kv_in=s0, kv_out=kv1, block=64, chunk=256, out_dtype=odt, exact=exact, silu=True)
    qa, ka, va = (la.silu_(t.clone()) for t in (q, k, v))
    o2 = la.fwd(qa, ka, va, lam, kv_in=s0, kv_out=kv2, block=64, chunk=256, out_dtype=odt, exact=exact)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(kv1, kv2)
    for a, b in zip((q, k, v), keep):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_silu_fused_against_oracle(dev, d):
    """The fused path against the oracle chain: SiLU in fp64 (rounded to bf16,
    as the activations are stored), then the fp64 recurrence."""
    say("prefill + fused SiLU vs oracle: B1 H8 N1500 d", d)
    B, H, N = 1, 8, 1500
    q, k, v = _preact(B, H, N, d, 320 + d, dev)
    s0 = state_device(B, H, d, seed=321, device=dev)
    kv = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    o = la.fwd(q, k, v, torch.from_numpy(LAMS8).to(dev), kv_in=s0, kv_out=kv, block=64, chunk=512,
               out_dtype=torch.float32, silu=True)
    torch.cuda.synchronize()
    act = [torch.from_numpy(ora.silu(host(t))).to(torch.bfloat16).to(torch.float32).numpy() for t in (q, k, v)]
    o_ref, s_ref = oracle(*act, LAMS8, host(s0).astype(np.float64))
    for h in range(H):
        tol.assert_bf16_f32out(host(o)[:, h], o_ref[:, h], "O head %d" % h)
        tol.assert_state(host(kv)[:, h], s_ref[:, h], "state head %d" % h)


def test_pooled_prefill_silu_fused(dev):
    say("pooled prefill + fused SiLU vs SiLU pass + pooled prefill: pool 6, B4 H4 N900 d128")
    B, H, N, d, P = 4, 4, 900, 128, 6
    q, k, v = _preact(B, H, N, d, 330, dev)
    slots = torch.tensor([3, -1, 0, 5], dtype=torch.int32, device=dev)
    lam = torch.from_numpy(LAMS8[[0, 3, 6, 7]].copy()).to(dev)
    pool1 = state_device(P, H, d, seed=331, device=dev)
    pool2 = pool1.clone()
    o1 = la.fwd_slots(q, k, v, lam, pool1, slots, out_dtype=torch.float32, silu=True)
    qa, ka, va = (la.silu_(t.clone()) for t in (q, k, v))
    o2 = la.fwd_slots(qa, ka, va, lam, pool2, slots, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(pool1, pool2)


# --- the per-head RMSNorm and sigmoid gate fused into the prefill ----------------

def _epilogue_ref(o_ref, gamma, gate, eps=1e-5):
    y = o_ref if gamma is None else ora.rmsnorm_heads(o_ref, host(gamma), eps=eps)
    return y if gate is None else ora.sigmoid_gate(y, host(gate))


@pytest.mark.parametrize("d,N,silu,exact", [(128, 1500, False, False), (128, 1500, True, False),
                                            (64, 1037, True, False), (128, 700, False, True),
                                            (64, 63, False, False)])
def test_prefill_norm_gate_fused_against_oracle(dev, d, N, silu, exact):
    """out = RMSNorm_head(o) * gamma * sigmoid(gate) from the output kernels,
    against the oracle chain (SiLU in fp64 rounded to bf16 when asked, the
    fp64 recurrence, the fp64 norm and gate), per head, on decays that take
    both the warm-start and the chunked paths, with an initial state and a
    ragged last tile; fp32 out at the RMS rule, bf16 out = RNE(fp32 out)."""
    B, H = 2, 8
    say("prefill + fused norm/gate vs oracle: B2 H8 N", N, "d", d, "silu", silu, "exact", exact)
    q, k, v = _preact(B, H, N, d, 400 + d + N, dev) if silu else qkv_device(B, H, N, d, seed=400 + d + N, device=dev)
    gate = qkv_device(B, H, N, d, seed=401 + N, device=dev)[0] * 8.0
    gamma = _gamma(H, d, 402, dev)
    s0 = state_device(B, H, d, seed=403, device=dev)
    lam = torch.from_numpy(LAMS8).to(dev)
    kv = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    kw = dict(kv_in=s0, chunk=256, silu=silu, exact=exact)
    y32 = la.fwd_fused(q, k, v, lam, gamma=gamma, gate=gate, kv_out=kv, out_dtype=torch.float32, **kw)
    y16 = la.fwd_fused(q, k, v, lam, gamma=gamma, gate=gate, out_dtype=torch.bfloat16, **kw)
    kv_plain = torch.empty_like(kv)
    la.fwd(q, k, v, lam, kv_out=kv_plain, block=64, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), y16), "bf16 out must be RNE(fp32 out)"
    assert torch.equal(kv, kv_plain), "the epilogue must leave the final state alone"
    if silu:
        act = [torch.from_numpy(ora.silu(host(t))).to(torch.bfloat16).to(torch.float32).numpy() for t in (q, k, v)]
    else:
        act = [host(t) for t in (q, k, v)]
    o_ref, s_ref = oracle(*act, LAMS8, host(s0).astype(np.float64))
    y_ref = _epilogue_ref(o_ref, gamma, gate)
    for h in range(H):
        tol.assert_bf16_f32out(host(y32)[:, h], y_ref[:, h], "y head %d" % h)
        tol.assert_bf16_out(host(y16)[:, h], y_ref[:, h], "y bf16 head %d" % h)
        tol.assert_state(host(kv)[:, h], s_ref[:, h], "state head %d" % h)


@pytest.mark.parametrize("which", ["norm", "gate", "neither"])
def test_prefill_fused_optional_steps(dev, which):
    """Either factor alone, or neither (then the plain prefill, bit for bit)."""
    B, H, N, d = 1, 8, 900, 128
    say("prefill + fused", which, "B1 H8 N900 d128")
    q, k, v = qkv_device(B, H, N, d, seed=410, device=dev)
    gate = qkv_device(B, H, N, d, seed=411, device=dev)[0] * 8.0 if which == "gate" else None
    gamma = _gamma(H, d, 412, dev) if which == "norm" else None
    lam = torch.from_numpy(LAMS8).to(dev)
    y = la.fwd_fused(q, k, v, lam, gamma=gamma, gate=gate, out_dtype=torch.float32, chunk=256)
    o = la.fwd(q, k, v, lam, block=64, out_dtype=torch.float32, chunk=256)
    torch.cuda.synchronize()
    if which == "neither":
        assert torch.equal(y, o)
        return
    o_ref, _ = oracle(host(q), host(k), host(v), LAMS8)
    y_ref = _epilogue_ref(o_ref, gamma, gate)
    for h in range(H):
        tol.assert_bf16_f32out(host(y)[:, h], y_ref[:, h], "y head %d" % h)


def test_prefill_fused_matches_the_separate_pass(dev):
    """The fused epilogue against the prefill followed by the norm/gate pass
    on its fp32 output: the same function, differing only in the order the
    sums of squares are added (a few ulps)."""
    B, H, N, d = 1, 8, 2000, 128
    say("prefill + fused norm/gate vs prefill then norm_gate pass: B1 H8 N2000 d128")
    q, k, v = qkv_device(B, H, N, d, seed=420, device=dev)
    gate = qkv_device(B, H, N, d, seed=421, device=dev)[0] * 8.0
    gamma = _gamma(H, d, 422, dev)
    lam = torch.from_numpy(LAMS8).to(dev)
    y = la.fwd_fused(q, k, v, lam, gamma=gamma, gate=gate, out_dtype=torch.float32)
    o = la.fwd(q, k, v, lam, block=64, out_dtype=torch.float32)
    y2 = la.norm_gate(o, gamma=gamma, gate=gate, eps=1e-5, out=torch.empty_like(o, dtype=torch.bfloat16))
    torch.cuda.synchronize()
    yf, y2f = host(y), host(y2)
    # the pass stores bf16: agreement to within its rounding plus a few fp32 ulps
    assert np.all(np.abs(yf - y2f) <= 2.0 ** -8 * np.abs(yf) + 1e-6 * np.abs(yf).max())


def test_prefill_fused_with_a_flagged_head(dev):
    """A head that fails the warm-start check is run again on the exact path
    with the epilogue: the result still matches the oracle chain."""
    say("prefill + fused norm/gate with a spike before a warm-up window, B1 H2 N512 d128 chunk 256")
    q, k, v = qkv_device(1, 2, 512, 128, seed=430, device=dev)
    k[:, 0, 190] *= 1e5
    v[:, 0, 190] *= 1e5
    lam = np.array([0.7, 0.3], dtype=np.float32)
    gate = qkv_device(1, 2, 512, 128, seed=431, device=dev)[0] * 8.0
    gamma = _gamma(2, 128, 432, dev)
    ws = torch.empty(la.workspace_bytes(1, 2, 512, 128, 64, 256), device=dev, dtype=torch.uint8)
    y = la.fwd_fused(q, k, v, torch.from_numpy(lam).to(dev), gamma=gamma, gate=gate, out_dtype=torch.float32,
                     chunk=256, workspace=ws)
    torch.cuda.synchronize()
    assert ws[ws.numel() - 8:].view(torch.int32).cpu().tolist() == [1, 0]
    o_ref, _ = oracle(host(q), host(k), host(v), lam)
    y_ref = _epilogue_ref(o_ref, gamma, gate)
    for h in range(2):
        tol.assert_bf16_f32out(host(y)[:, h], y_ref[:, h], "y head %d" % h)
