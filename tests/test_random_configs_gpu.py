"""Seeded random configurations against the oracle: the prefill (every dtype,
block, chunk and flag the library takes, ragged lengths, initial states,
decays drawn across the warm-start / three-pass boundary), the pooled
prefill and the backward.  Sizes stay small so the oracle finishes in
seconds; each case prints its parameters before touching the GPU."""
import numpy as np
import pytest
import torch

import long_context_decayed_amd as la
from long_context_decayed_amd.inputs import qkv_cpu, qkv_device, state_device
from oracle import crec
import tolerances as tol
from gpu_helpers import host, oracle, oracle_threads, require_gpu, say

pytestmark = pytest.mark.gpu
N_CASES = 64


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _decays(rng, h):
    # a mix: exactly 0 and 1, fast decays, slow decays, and values near 1
    kinds = rng.integers(0, 5, size=h)
    out = []
    for kd in kinds:
        if kd == 0:
            out.append(rng.choice([0.0, 1.0]))
        elif kd == 1:
            out.append(rng.uniform(0.0, 0.8))
        elif kd == 2:
            out.append(rng.uniform(0.8, 0.99))
        elif kd == 3:
            out.append(1.0 - 10.0 ** rng.uniform(-7, -2))
        else:
            out.append(np.exp(-2.0 ** rng.uniform(-9, 0)))
    return np.asarray(out, dtype=np.float32)


def _case(i):
    rng = np.random.default_rng(1000 + i)
    c = dict(
        B=int(rng.integers(1, 4)), H=int(rng.integers(1, 6)), N=int(rng.integers(1, 2600)),
        d=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "bf16", "f32out", "fp32"])),
        state=bool(rng.integers(0, 2)), exact=bool(rng.integers(0, 4) == 0),
    )
    blocks = [64, 128, 256] if (c["dtype"] != "fp32" or c["d"] == 64) else [64]
    c["block"] = int(rng.choice(blocks))
    c["chunk"] = int(rng.choice([0, c["block"], 2 * c["block"], 1024 if c["block"] <= 256 else 0]))
    if c["chunk"] % c["block"]:
        c["chunk"] = 0
    c["lam"] = _decays(rng, c["H"])
    c["seed"] = 2000 + i
    return c


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_prefill(dev, i):
    c = _case(i)
    say("random prefill", i, {k: v for k, v in c.items() if k != "lam"}, "lam", np.round(c["lam"], 5).tolist())
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    if c["dtype"] == "fp32":
        q, k, v = (t.to(dev) for t in qkv_cpu(B, H, N, d, seed=c["seed"]))
        odt = torch.float32
    else:
        q, k, v = qkv_device(B, H, N, d, seed=c["seed"], device=dev)
        odt = torch.float32 if c["dtype"] == "f32out" else torch.bfloat16
    s0 = state_device(B, H, d, seed=c["seed"], device=dev) if c["state"] else None
    kv = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    o = la.fwd(q, k, v, torch.from_numpy(c["lam"]).to(dev), kv_in=s0, kv_out=kv, block=c["block"], chunk=c["chunk"],
               out_dtype=odt, exact=c["exact"])
    torch.cuda.synchronize()
    o_ref, s_ref = oracle(host(q), host(k), host(v), c["lam"], None if s0 is None else host(s0).astype(np.float64))
    o_h, kv_h = host(o), host(kv)
    for h in range(H):
        if c["dtype"] == "fp32":
            tol.assert_fp32(o_h[:, h], o_ref[:, h], "O head %d" % h)
            tol.assert_fp32(kv_h[:, h], s_ref[:, h], "kv head %d" % h)
        elif c["dtype"] == "f32out":
            tol.assert_bf16_f32out(o_h[:, h], o_ref[:, h], "O head %d" % h)
            tol.assert_state(kv_h[:, h], s_ref[:, h], "kv head %d" % h)
        else:
            tol.assert_bf16_out(o_h[:, h], o_ref[:, h], "O head %d" % h)
            tol.assert_state(kv_h[:, h], s_ref[:, h], "kv head %d" % h)


@pytest.mark.parametrize("i", range(24))
def test_random_backward(dev, i):
    rng = np.random.default_rng(3000 + i)
    B, H, N, d = int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.integers(1, 1800)), int(rng.choice([64, 128]))
    fp32 = bool(rng.integers(0, 4) == 0)
    states, exact = bool(rng.integers(0, 2)), bool(rng.integers(0, 4) == 0)
    lam = _decays(rng, H)
    say("random backward", i, dict(B=B, H=H, N=N, d=d, fp32=fp32, states=states, exact=exact),
        "lam", np.round(lam, 5).tolist())
    if fp32:
        q, k, v = (t.to(dev) for t in qkv_cpu(B, H, N, d, seed=4000 + i))
        g = qkv_cpu(B, H, N, d, seed=5000 + i)[0].to(dev)
    else:
        q, k, v = qkv_device(B, H, N, d, seed=4000 + i, device=dev)
        g = qkv_device(B, H, N, d, seed=5000 + i, device=dev)[0]
    s0 = state_device(B, H, d, seed=4000 + i, device=dev) if states else None
    dsn = state_device(B, H, d, seed=5000 + i, device=dev) if states else None
    dq, dk, dv, ds0 = la.bwd(q, k, v, torch.from_numpy(lam).to(dev), g, kv_in=s0, dkv_out=dsn,
                             out_dtype=torch.float32, dkv_in=True, exact=exact)
    torch.cuda.synchronize()
    refs = crec.backward(host(q), host(k), host(v), lam.astype(np.float64), host(g),
                         None if s0 is None else host(s0).astype(np.float64),
                         None if dsn is None else host(dsn).astype(np.float64), threads=oracle_threads())
    chk = tol.assert_fp32 if fp32 else tol.assert_bf16_f32out
    for got, ref, name in zip((dq, dk, dv), refs[:3], ("dQ", "dK", "dV")):
        for h in range(H):
            chk(host(got)[:, h], ref[:, h], "%s head %d" % (name, h))
    for h in range(H):
        (tol.assert_fp32 if fp32 else tol.assert_state)(host(ds0)[:, h], refs[3][:, h], "dS0 head %d" % h)


@pytest.mark.parametrize("i", range(12))
def test_random_pooled_prefill(dev, i):
    rng = np.random.default_rng(6000 + i)
    H, P, N, d = int(rng.integers(1, 5)), int(rng.integers(2, 9)), int(rng.integers(1, 2000)), int(rng.choice([64, 128]))
    B = int(rng.integers(1, P + 1))
    slots_h = rng.permutation(P)[:B].astype(np.int32)
    if B > 1 and rng.integers(0, 2):
        slots_h[int(rng.integers(0, B))] = -1 if rng.integers(0, 2) else P + 3
    lam = _decays(rng, H)
    block = int(rng.choice([64, 256]))
    say("random pooled prefill", i, dict(H=H, P=P, N=N, d=d, block=block, slots=slots_h.tolist()))
    q, k, v = qkv_device(B, H, N, d, seed=7000 + i, device=dev)
    pool = state_device(P, H, d, seed=7000 + i, device=dev)
    pool0 = host(pool).astype(np.float64)
    o = la.fwd_slots(q, k, v, torch.from_numpy(lam).to(dev), pool, torch.from_numpy(slots_h).to(dev), block=block,
                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    pool1 = host(pool).astype(np.float64)
    for b, s in enumerate(slots_h):
        ok = 0 <= s < P
        o_ref, s_ref = oracle(host(q)[b], host(k)[b], host(v)[b], lam, pool0[s] if ok else None)
        for h in range(H):
            tol.assert_bf16_f32out(host(o)[b, h], o_ref[h], "row %d head %d" % (b, h))
            if ok:
                tol.assert_state(pool1[s, h], s_ref[h], "slot %d head %d" % (s, h))
    untouched = [s for s in range(P) if s not in slots_h]
    assert np.array_equal(pool1[untouched], pool0[untouched])


@pytest.mark.parametrize("i", range(16))
def test_random_decode(dev, i):
    import oracle as ora
    rng = np.random.default_rng(8000 + i)
    H, d = int(rng.integers(1, 9)), int(rng.choice([64, 128]))
    P = int(rng.integers(1, 40))
    pooled, silu = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    use_gamma, use_gate = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    if pooled:
        B = int(rng.integers(1, P + 3))
        slots_h = rng.integers(-2, P + 2, size=B).astype(np.int32)
        # no two rows on one slot: repeats become idle rows
        seen = set()
        for b, s in enumerate(slots_h):
            if 0 <= s < P and s in seen:
                slots_h[b] = -1
            seen.add(int(s))
    else:
        B = P
        slots_h = np.arange(B, dtype=np.int32)
    lam = _decays(rng, H)
    say("random decode", i, dict(B=B, H=H, d=d, P=P, pooled=pooled, silu=silu, gamma=use_gamma, gate=use_gate))
    q, k, v = (t[:, :, 0].mul(float(rng.uniform(1, 6))).contiguous()
               for t in qkv_device(B, H, 1, d, seed=9000 + i, device=dev))
    gate = qkv_device(B, H, 1, d, seed=9100 + i, device=dev)[0][:, :, 0].mul(8.0).contiguous() if use_gate else None
    gen = torch.Generator().manual_seed(9200 + i)
    gamma = (1.0 + 0.3 * torch.randn((H, d), generator=gen)).to(dev) if use_gamma else None
    pool = state_device(P, H, d, seed=9300 + i, device=dev)
    pool0 = host(pool).astype(np.float64)
    o = la.decode_fused(q, k, v, torch.from_numpy(lam).to(dev), pool,
                        torch.from_numpy(slots_h).to(dev) if pooled else None,
                        silu=silu, gamma=gamma, gate=gate, eps=1e-5)
    torch.cuda.synchronize()
    act = [(b, int(s)) for b, s in enumerate(slots_h) if 0 <= s < P]
    rows = np.array([b for b, _ in act], dtype=np.int64)
    sl = np.array([s for _, s in act], dtype=np.int64)
    pool1 = host(pool).astype(np.float64)
    if len(act):
        qs, ks, vs = (host(t)[rows] for t in (q, k, v))
        if silu:
            qs, ks, vs = ora.silu(qs), ora.silu(ks), ora.silu(vs)
        y, s_ref = ora.decode_step(qs, ks, vs, lam.astype(np.float64), pool0[sl])
        if use_gamma:
            y = ora.rmsnorm_heads(y[:, :, None, :], host(gamma), eps=1e-5)[:, :, 0, :]
        if use_gate:
            y = ora.sigmoid_gate(y, host(gate)[rows])
        for h in range(H):
            tol.assert_bf16_out(host(o)[rows][:, h], y[:, h], "o head %d" % h)
            tol.assert_state(pool1[sl][:, h], s_ref[:, h], "state head %d" % h)
    idle = [b for b in range(B) if b not in set(rows.tolist())]
    assert np.all(host(o)[idle] == 0.0)
    untouched = [s for s in range(P) if s not in set(sl.tolist())]
    assert np.array_equal(pool1[untouched], pool0[untouched])


@pytest.mark.parametrize("i", range(24))
def test_random_prefill_warm_chunk_and_silu(dev, i):
    """bf16, block 64: random scan and warm-start chunk lengths, SiLU on the
    tiles or not, against the oracle (fed the bf16-rounded fp64 SiLU when on)."""
    import oracle as ora
    rng = np.random.default_rng(11000 + i)
    B, H, N, d = int(rng.integers(1, 3)), int(rng.integers(1, 7)), int(rng.integers(1, 4000)), int(rng.choice([64, 128]))
    chunk = int(rng.choice([0, 64, 128, 256, 512]))
    warm_chunk = 0 if chunk == 0 or rng.integers(0, 3) == 0 else chunk * int(rng.choice([1, 2, 4, 8]))
    silu, state, exact = bool(rng.integers(0, 2)), bool(rng.integers(0, 2)), bool(rng.integers(0, 5) == 0)
    odt = torch.float32 if rng.integers(0, 2) else torch.bfloat16
    lam = _decays(rng, H)
    say("random prefill, chunks and SiLU", i, dict(B=B, H=H, N=N, d=d, chunk=chunk, warm_chunk=warm_chunk, silu=silu,
                                                   state=state, exact=exact, out=str(odt)),
        "lam", np.round(lam, 5).tolist())
    scale = 2.5 if silu else 1.0
    q, k, v = (t * scale for t in qkv_device(B, H, N, d, seed=12000 + i, device=dev))
    q, k, v = (t.contiguous() for t in (q, k, v))
    s0 = state_device(B, H, d, seed=12000 + i, device=dev) if state else None
    kv = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    o = la.fwd(q, k, v, torch.from_numpy(lam).to(dev), kv_in=s0, kv_out=kv, block=64, chunk=chunk,
               warm_chunk=warm_chunk, out_dtype=odt, exact=exact, silu=silu)
    torch.cuda.synchronize()
    if silu:
        ins = [torch.from_numpy(ora.silu(host(t))).to(torch.bfloat16).to(torch.float32).numpy() for t in (q, k, v)]
    else:
        ins = [host(t) for t in (q, k, v)]
    o_ref, s_ref = oracle(*ins, lam, None if s0 is None else host(s0).astype(np.float64))
    o_h, kv_h = host(o), host(kv)
    for h in range(H):
        if odt == torch.float32:
            tol.assert_bf16_f32out(o_h[:, h], o_ref[:, h], "O head %d" % h)
        else:
            tol.assert_bf16_out(o_h[:, h], o_ref[:, h], "O head %d" % h)
        tol.assert_state(kv_h[:, h], s_ref[:, h], "kv head %d" % h)


@pytest.mark.parametrize("i", range(20))
def test_random_prefill_fused_norm_gate(dev, i):
    """The prefill with the per-head RMSNorm and the gate in its output
    kernels: random sizes, chunks, SiLU, exact flag, either factor or both,
    against the oracle chain; bf16 out = RNE(fp32 out)."""
    import oracle as ora
    rng = np.random.default_rng(13000 + i)
    B, H, N, d = int(rng.integers(1, 3)), int(rng.integers(1, 7)), int(rng.integers(1, 3000)), int(rng.choice([64, 128]))
    chunk = int(rng.choice([0, 64, 256, 512]))
    warm_chunk = 0 if chunk == 0 or rng.integers(0, 2) else chunk * int(rng.choice([1, 2, 4]))
    silu, state, exact = bool(rng.integers(0, 2)), bool(rng.integers(0, 2)), bool(rng.integers(0, 5) == 0)
    use_gamma, use_gate = [(True, True), (True, False), (False, True)][int(rng.integers(0, 3))]
    eps = float(rng.choice([1e-5, 1e-3]))
    lam = _decays(rng, H)
    say("random fused prefill", i, dict(B=B, H=H, N=N, d=d, chunk=chunk, warm_chunk=warm_chunk, silu=silu,
                                        state=state, exact=exact, gamma=use_gamma, gate=use_gate, eps=eps),
        "lam", np.round(lam, 5).tolist())
    scale = 2.5 if silu else 1.0
    q, k, v = (t * scale for t in qkv_device(B, H, N, d, seed=14000 + i, device=dev))
    q, k, v = (t.contiguous() for t in (q, k, v))
    gate = (qkv_device(B, H, N, d, seed=14100 + i, device=dev)[0] * 8.0).contiguous() if use_gate else None
    gen = torch.Generator().manual_seed(14200 + i)
    gamma = (1.0 + 0.3 * torch.randn((H, d), generator=gen)).to(dev) if use_gamma else None
    s0 = state_device(B, H, d, seed=14300 + i, device=dev) if state else None
    lam_d = torch.from_numpy(lam).to(dev)
    kw = dict(gamma=gamma, gate=gate, eps=eps, kv_in=s0, chunk=chunk, warm_chunk=warm_chunk, exact=exact, silu=silu)
    y32 = la.fwd_fused(q, k, v, lam_d, out_dtype=torch.float32, **kw)
    y16 = la.fwd_fused(q, k, v, lam_d, out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), y16)
    if silu:
        ins = [torch.from_numpy(ora.silu(host(t))).to(torch.bfloat16).to(torch.float32).numpy() for t in (q, k, v)]
    else:
        ins = [host(t) for t in (q, k, v)]
    o_ref, _ = oracle(*ins, lam, None if s0 is None else host(s0).astype(np.float64), want_state=False)
    y_ref = o_ref if gamma is None else ora.rmsnorm_heads(o_ref, host(gamma), eps=eps)
    y_ref = y_ref if gate is None else ora.sigmoid_gate(y_ref, host(gate))
    for h in range(H):
        tol.assert_bf16_f32out(host(y32)[:, h], y_ref[:, h], "y head %d" % h)


@pytest.mark.parametrize("i", range(12))
def test_random_decode_layers(dev, i):
    """One launch over several layers' pools: random layer counts, sizes,
    slot tables (idle rows included) and fusion flags, per layer against the
    oracle."""
    import oracle as ora
    rng = np.random.default_rng(15000 + i)
    L, H, d, P = int(rng.integers(1, 6)), int(rng.integers(1, 9)), int(rng.choice([64, 128])), int(rng.integers(1, 12))
    pooled, silu = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    use_gamma, use_gate = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    B = int(rng.integers(1, P + 3)) if pooled else P
    tables = np.empty((L, B), dtype=np.int32)
    for l in range(L):
        if pooled:
            t = rng.integers(-2, P + 2, size=B)
            seen = set()
            for b in range(B):  # no two rows of a layer on one slot
                if 0 <= t[b] < P and t[b] in seen:
                    t[b] = -1
                seen.add(int(t[b]))
            tables[l] = t
        else:
            tables[l] = np.arange(B)
    lam = np.stack([_decays(rng, H) for _ in range(L)])
    say("random decode layers", i, dict(L=L, B=B, H=H, d=d, P=P, pooled=pooled, silu=silu, gamma=use_gamma,
                                        gate=use_gate))
    q, k, v = (t.reshape(L, B, H, d).mul(float(rng.uniform(1, 6))).contiguous()
               for t in qkv_device(L * B, H, 1, d, seed=15100 + i, device=dev))
    gate = (qkv_device(L * B, H, 1, d, seed=15200 + i, device=dev)[0].reshape(L, B, H, d) * 8.0).contiguous() \
        if use_gate else None
    gen = torch.Generator().manual_seed(15300 + i)
    gamma = (1.0 + 0.3 * torch.randn((L, H, d), generator=gen)).to(dev) if use_gamma else None
    pool = torch.stack([state_device(P, H, d, seed=15400 + 10 * i + l, device=dev) for l in range(L)]).contiguous()
    pool0 = host(pool).astype(np.float64)
    o = la.decode_layers(q, k, v, torch.from_numpy(lam).to(dev), pool,
                         torch.from_numpy(tables).to(dev) if pooled else None, silu=silu, gamma=gamma, gate=gate)
    torch.cuda.synchronize()
    o_h, pool1 = host(o), host(pool).astype(np.float64)
    for l in range(L):
        rows = np.array([b for b in range(B) if 0 <= tables[l, b] < P], dtype=np.int64)
        sl = tables[l, rows].astype(np.int64)
        if len(rows):
            qs, ks, vs = (host(t)[l, rows] for t in (q, k, v))
            if silu:
                qs, ks, vs = ora.silu(qs), ora.silu(ks), ora.silu(vs)
            y, s_ref = ora.decode_step(qs, ks, vs, lam[l].astype(np.float64), pool0[l, sl])
            if use_gamma:
                y = ora.rmsnorm_heads(y[:, :, None, :], host(gamma)[l], eps=1e-5)[:, :, 0, :]
            if use_gate:
                y = ora.sigmoid_gate(y, host(gate)[l, rows])
            for h in range(H):
                tol.assert_bf16_out(o_h[l, rows][:, h], y[:, h], "layer %d o head %d" % (l, h))
                tol.assert_state(pool1[l, sl][:, h], s_ref[:, h], "layer %d state head %d" % (l, h))
        idle = [b for b in range(B) if b not in set(rows.tolist())]
        assert np.all(o_h[l, idle] == 0.0)
        untouched = [s for s in range(P) if s not in set(sl.tolist())]
        assert np.array_equal(pool1[l, untouched], pool0[l, untouched])
