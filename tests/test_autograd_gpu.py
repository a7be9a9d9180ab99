"""GPU checks of the differentiable prefill (lightning_attn): its forward is
the library's prefill and its backward the library's backward, so its outputs
and gradients equal direct fwd / bwd calls bit for bit; the gradients of a
loss on both out and kv_out are held against the fp64 gradient oracle
(adjoint recurrence in plain C) as the backward tests do."""
import numpy as np
import pytest
import torch

import long_context_decayed_amd as la
from long_context_decayed_amd.inputs import qkv_device, state_device
from oracle import crec
import tolerances as tol
from gpu_helpers import host, oracle_threads, require_gpu, say

pytestmark = pytest.mark.gpu

LAMS = np.array([0.0, 0.3, 0.9, 0.999, 1.0, 0.7, 0.97, 1e-3], dtype=np.float32)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _loss_weights(B, H, N, d, dev, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    w = torch.randn((B, H, N, d), generator=g, device=dev, dtype=torch.float32)
    w2 = torch.randn((B, H, d, d), generator=g, device=dev, dtype=torch.float32) * 1e-2
    return w, w2


@pytest.mark.parametrize("dtype,d,n", [(torch.bfloat16, 128, 700), (torch.bfloat16, 64, 3037),
                                       (torch.float32, 64, 1000)])
@pytest.mark.parametrize("with_state", [False, True])
def test_autograd_matches_bwd_and_oracle(dev, dtype, d, n, with_state):
    B, H = 2, 8
    say("autograd prefill B2 H8 N", n, "d", d, dtype, "kv_in", with_state)
    q, k, v = (t.to(dtype) for t in qkv_device(B, H, n, d, seed=300 + n, device=dev))
    lam = torch.from_numpy(LAMS).to(dev)
    s0 = state_device(B, H, d, seed=300 + n, device=dev) if with_state else None
    w, w2 = _loss_weights(B, H, n, d, dev, 310 + n)
    leaves = [t.clone().requires_grad_(True) for t in (q, k, v)]
    s0_leaf = s0.clone().requires_grad_(True) if with_state else None
    out, kv_out = la.lightning_attn(*leaves, lam, kv_in=s0_leaf)
    loss = (out.float() * w).sum() + (kv_out * w2).sum()
    loss.backward()
    torch.cuda.synchronize()

    # the same library calls made directly
    kv_ref = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    out_ref = la.fwd(q, k, v, lam, kv_in=s0, kv_out=kv_ref)
    dout = w.to(dtype)
    dq, dk, dv, ds0 = la.bwd(q, k, v, lam, dout, kv_in=s0, dkv_out=w2, dkv_in=with_state)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), out_ref) and torch.equal(kv_out.detach(), kv_ref)
    for leaf, ref in zip(leaves, (dq, dk, dv)):
        assert torch.equal(leaf.grad, ref)
    if with_state:
        assert torch.equal(s0_leaf.grad, ds0)

    # against the fp64 adjoint recurrence on the same bits
    rq, rk, rv, rs = crec.backward(host(q), host(k), host(v), LAMS.astype(np.float64), host(dout),
                                   None if s0 is None else host(s0).astype(np.float64), host(w2).astype(np.float64),
                                   threads=oracle_threads())
    for name, got, ref in (("dQ", leaves[0].grad, rq), ("dK", leaves[1].grad, rk), ("dV", leaves[2].grad, rv)):
        got = host(got)
        for h in range(H):
            if dtype == torch.float32:
                tol.assert_fp32(got[:, h], ref[:, h], "%s head %d" % (name, h))
            else:  # bf16 gradients: the bf16-output rule, on each head's own RMS
                tol.assert_bf16_out(got[:, h], ref[:, h], "%s head %d" % (name, h))
    if with_state:
        gs = host(s0_leaf.grad)
        for h in range(H):
            tol.assert_state(gs[:, h], rs[:, h], "dkv_in head %d" % h)


def test_autograd_without_kv_in_gradient(dev):
    # kv_in given but not requiring a gradient: the backward asks for none
    B, H, N, d = 1, 8, 512, 128
    say("autograd prefill, kv_in without grad, B1 H8 N512 d128 bf16")
    q, k, v = qkv_device(B, H, N, d, seed=320, device=dev)
    lam = torch.from_numpy(LAMS).to(dev)
    s0 = state_device(B, H, d, seed=320, device=dev)
    leaves = [t.clone().requires_grad_(True) for t in (q, k, v)]
    out, _ = la.lightning_attn(*leaves, lam, kv_in=s0)
    out.float().sum().backward()
    torch.cuda.synchronize()
    dq, dk, dv, _ = la.bwd(q, k, v, lam, torch.ones_like(q), kv_in=s0, dkv_out=torch.zeros_like(s0))
    torch.cuda.synchronize()
    for leaf, ref in zip(leaves, (dq, dk, dv)):
        assert torch.equal(leaf.grad, ref)
