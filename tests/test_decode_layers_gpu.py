"""GPU parity of the decode step over several layers' states in one launch
(lightning_attn_decode_layers) against the fp64 oracle, layer by layer, and
against one single-layer launch per layer (same arithmetic, bit for bit)."""
import numpy as np
import pytest
import torch

import long_context_decayed_amd as la
import oracle as ora
from long_context_decayed_amd.inputs import decay_lambdas_depth, qkv_device, state_device
import tolerances as tol
from gpu_helpers import host, require_gpu, say

pytestmark = pytest.mark.gpu

LAYERS = (0, 23, 46, 69)  # of a 70-layer stack: slopes scaled down with depth, the last undecayed


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _inputs(L, B, H, d, P, seed, dev, scale=1.0):
    q, k, v = (t.reshape(L, B, H, d).contiguous() for t in qkv_device(L * B, H, 1, d, seed=seed, device=dev))
    if scale != 1.0:
        q, k, v = ((t.float() * scale).to(torch.bfloat16).contiguous() for t in (q, k, v))
    lam = np.stack([decay_lambdas_depth(H, l, 70) for l in LAYERS[:L]]).astype(np.float32)
    pool = torch.stack([state_device(P, H, d, seed=seed + 100 + l, device=dev) for l in range(L)]).contiguous()
    return q, k, v, lam, pool


def _slot_tables(L, B, P, seed):
    """Per-layer tables: distinct slots within a layer, some rows idle (-1 or
    past the pool), as when requests are at different layers."""
    rng = np.random.default_rng(seed)
    t = np.empty((L, B), dtype=np.int32)
    for l in range(L):
        t[l] = rng.permutation(P)[:B]
        idle = rng.random(B) < 0.25
        t[l][idle] = rng.choice([-1, P, P + 3], size=int(idle.sum()))
    return t


@pytest.mark.parametrize("d", [64, 128])
def test_decode_layers_against_oracle(dev, d):
    L, B, H, P = 4, 6, 8, 9
    say("decode layers L4 B6 H8 pool 9 d", d)
    q, k, v, lam, pool = _inputs(L, B, H, d, P, 300 + d, dev)
    slots = _slot_tables(L, B, P, 300 + d)
    pool0 = host(pool).astype(np.float64)
    o = la.decode_layers(q, k, v, torch.from_numpy(lam).to(dev), pool, torch.from_numpy(slots).to(dev))
    torch.cuda.synchronize()
    o_h, pool_h = host(o), host(pool).astype(np.float64)
    for l in range(L):
        rows = np.array([b for b in range(B) if 0 <= slots[l, b] < P])
        sl = slots[l, rows]
        o_ref, s_ref = ora.decode_step(host(q)[l, rows], host(k)[l, rows], host(v)[l, rows],
                                       lam[l].astype(np.float64), pool0[l, sl])
        tol.assert_bf16_out(o_h[l, rows], o_ref)
        tol.assert_state(pool_h[l, sl], s_ref)
        idle = [b for b in range(B) if b not in rows]
        assert np.all(o_h[l, idle] == 0.0)
        untouched = [s for s in range(P) if s not in sl]
        assert np.array_equal(pool_h[l, untouched], pool0[l, untouched])


def test_decode_layers_fused_against_oracle(dev):
    """SiLU on q, k, v, each layer's own RMSNorm weights and the gate."""
    L, B, H, P, d = 3, 5, 8, 7, 128
    say("decode layers fused (silu, norm, gate) L3 B5 H8 pool 7 d128")
    q, k, v, lam, pool = _inputs(L, B, H, d, P, 400, dev, scale=3.0 * d ** 0.5 / 4)
    gate = qkv_device(L * B, H, 1, d, seed=401, device=dev)[0].reshape(L, B, H, d).contiguous()
    g = torch.Generator().manual_seed(402)
    gamma = (1.0 + 0.25 * torch.randn((L, H, d), generator=g)).to(torch.float32).to(dev)
    slots = _slot_tables(L, B, P, 403)
    pool0 = host(pool).astype(np.float64)
    o = la.decode_layers(q, k, v, torch.from_numpy(lam).to(dev), pool, torch.from_numpy(slots).to(dev), silu=True,
                         gamma=gamma, gate=gate, eps=1e-5)
    torch.cuda.synchronize()
    o_h, pool_h = host(o), host(pool).astype(np.float64)
    for l in range(L):
        rows = np.array([b for b in range(B) if 0 <= slots[l, b] < P])
        sl = slots[l, rows]
        qs, ks, vs = (ora.silu(host(t)[l, rows]) for t in (q, k, v))
        o_core, s_ref = ora.decode_step(qs, ks, vs, lam[l].astype(np.float64), pool0[l, sl])
        y = ora.rmsnorm_heads(o_core[:, :, None, :], host(gamma)[l], eps=1e-5)[:, :, 0, :]
        y = ora.sigmoid_gate(y, host(gate)[l, rows])
        tol.assert_bf16_out(o_h[l, rows], y)
        tol.assert_state(pool_h[l, sl], s_ref)


@pytest.mark.parametrize("fused", [False, True])
def test_decode_layers_is_one_launch_per_layer(dev, fused):
    """The same rows stepped layer by layer with single-layer launches give
    the same outputs and states bit for bit."""
    L, B, H, P, d = 4, 7, 16, 11, 128
    say("decode layers vs per-layer launches L4 B7 H16 pool 11, fused", fused)
    q, k, v, lam, pool = _inputs(L, B, H, d, P, 500, dev)
    pool2 = pool.clone()
    slots = torch.from_numpy(_slot_tables(L, B, P, 501)).to(dev)
    lam_d = torch.from_numpy(lam).to(dev)
    gate = qkv_device(L * B, H, 1, d, seed=502, device=dev)[0].reshape(L, B, H, d).contiguous() if fused else None
    gamma = (torch.rand((L, H, d), device=dev) + 0.5) if fused else None
    o = la.decode_layers(q, k, v, lam_d, pool, slots, silu=fused, gamma=gamma, gate=gate)
    outs = []
    for l in range(L):
        outs.append(la.decode_fused(q[l], k[l], v[l], lam_d[l].contiguous(), pool2[l], slots[l].contiguous(),
                                    silu=fused, gamma=None if gamma is None else gamma[l].contiguous(),
                                    gate=None if gate is None else gate[l]))
    torch.cuda.synchronize()
    assert torch.equal(o, torch.stack(outs))
    assert torch.equal(pool, pool2)


def test_decode_layers_without_slot_table(dev):
    """slots = None: row b of every layer uses its pool row b (pool larger
    than the batch: the rows past it are untouched)."""
    L, B, H, P, d = 2, 4, 8, 6, 64
    say("decode layers without slot table L2 B4 H8 pool 6 d64")
    q, k, v, lam, pool = _inputs(L, B, H, d, P, 600, dev)
    pool0 = host(pool).astype(np.float64)
    o = la.decode_layers(q, k, v, torch.from_numpy(lam).to(dev), pool)
    torch.cuda.synchronize()
    pool_h = host(pool).astype(np.float64)
    for l in range(L):
        o_ref, s_ref = ora.decode_step(host(q)[l], host(k)[l], host(v)[l], lam[l].astype(np.float64), pool0[l, :B])
        tol.assert_bf16_out(host(o)[l], o_ref)
        tol.assert_state(pool_h[l, :B], s_ref)
        assert np.array_equal(pool_h[l, B:], pool0[l, B:])
