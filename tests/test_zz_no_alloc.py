"""GPU checks of lightning_attn_fwd_noalloc, the prefill whose workspace is the
library's own per-device array: through the C ABI, its outputs and final
states equal those of lightning_attn_fwd_ex (same kernels, same chunking, a
caller workspace) bit for bit, on two calls in a row, the second with a
smaller input, and both are within the parity bar against the fp64 oracle."""
import numpy as np
import pytest
import torch

import long_context_decayed_amd as la
from long_context_decayed_amd.inputs import qkv_device, state_device
import tolerances as tol
from gpu_helpers import host, oracle, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


# decays on both sides of the warm-start test (0, fast, slow, 1)
LAMS = np.array([0.0, 0.7, 0.995, 0.9999, 1.0], dtype=np.float32)


def _case(dev, B, H, N, d, seed, out_dtype, chunk, warm_chunk, with_state):
    q, k, v = qkv_device(B, H, N, d, seed=seed, device=dev)
    lam_np = LAMS[np.arange(H) % len(LAMS)].copy()
    lam = torch.from_numpy(lam_np).to(dev)
    s0 = state_device(B, H, d, seed=seed, device=dev) if with_state else None
    out_a = torch.full((B, H, N, d), float("nan"), device=dev, dtype=out_dtype)
    out_b = torch.full((B, H, N, d), float("nan"), device=dev, dtype=out_dtype)
    kv_a = torch.full((B, H, d, d), float("nan"), device=dev, dtype=torch.float32)
    kv_b = torch.full((B, H, d, d), float("nan"), device=dev, dtype=torch.float32)
    la.fwd_noalloc(q, k, v, lam, out_a, kv_in=s0, kv_out=kv_a, chunk=chunk, warm_chunk=warm_chunk)
    la.fwd(q, k, v, lam, kv_in=s0, kv_out=kv_b, block=64, out=out_b, chunk=chunk, warm_chunk=warm_chunk)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b), "no-alloc output differs from the workspace entry point"
    assert torch.equal(kv_a, kv_b), "no-alloc final state differs from the workspace entry point"
    o_ref, s_ref = oracle(host(q), host(k), host(v), lam_np, None if s0 is None else host(s0).astype(np.float64))
    if out_dtype == torch.float32:
        e = tol.bf16_rms_error(host(out_a), o_ref)
        assert e <= tol.BF16_RMS, e
    else:
        assert tol.bf16_store_violations(host(out_a), o_ref) == 0
    assert tol.state_error(host(kv_a), s_ref) <= tol.STATE_REL


def test_noalloc_matches_workspace_entry_two_calls(dev):
    """A larger call, then a smaller one on the same array (its contents are
    the first call's): both equal the workspace entry point bit for bit."""
    say("noalloc B2 H5 N3000 d128 bf16->fp32 chunk 512 warm 1024, with state")
    _case(dev, 2, 5, 3000, 128, seed=21, out_dtype=torch.float32, chunk=512, warm_chunk=1024, with_state=True)
    say("noalloc B1 H3 N700 d64 bf16->bf16 chunk 256 warm 512, no state")
    _case(dev, 1, 3, 700, 64, seed=22, out_dtype=torch.bfloat16, chunk=256, warm_chunk=512, with_state=False)


def _noalloc_chunk(B, H, N, d):
    """The chunk lightning_attn_fwd_noalloc takes with chunk 0: the default,
    doubled while the workspace exceeds the array (and the chunk is shorter
    than the sequence rounded up to whole blocks)."""
    L = la.chunk_for(B, H, N, 64)
    cap = -(-N // 64) * 64
    while la.workspace_bytes(B, H, N, d, 64, L) > la.NOALLOC_SCRATCH_BYTES and 2 * L <= (1 << 24) and L < cap:
        L *= 2
    return L


def test_noalloc_default_chunk(dev):
    """chunk 0: a workload whose default workspace (128 MiB of chunk states)
    exceeds the array, so the chunk is doubled; equal to the workspace entry
    point at that chunk and its default warm-start chunk."""
    B, H, N, d = 2, 64, 16384, 128
    L = _noalloc_chunk(B, H, N, d)
    assert la.workspace_bytes(B, H, N, d, 64) > la.NOALLOC_SCRATCH_BYTES
    assert L > la.chunk_for(B, H, N, 64)
    Lw = max(la.warm_chunk_for(B, H, N, 64), L)
    say("noalloc default chunk B2 H64 N16384 d128 (chunk %d, warm %d)" % (L, Lw))
    from long_context_decayed_amd.inputs import decay_lambdas
    q, k, v = qkv_device(B, H, N, d, seed=23, device=dev)
    lam = torch.from_numpy(decay_lambdas(H)).to(dev)
    out_a = torch.empty((B, H, N, d), device=dev, dtype=torch.bfloat16)
    kv_a = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    kv_b = torch.empty_like(kv_a)
    la.fwd_noalloc(q, k, v, lam, out_a, kv_out=kv_a)
    out_b = la.fwd(q, k, v, lam, kv_out=kv_b, block=64, chunk=L, warm_chunk=Lw)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert torch.equal(kv_a, kv_b)


def test_noalloc_rejects_a_workspace_beyond_the_array(dev):
    # 4 x 64 heads x 256 chunks x 64 KiB = 4 GiB of chunk states
    say("noalloc rejection B4 H64 N65536 d128 chunk 256 (nothing launched)")
    q = torch.zeros((4, 64, 1 << 16, 128), device=dev, dtype=torch.bfloat16)
    lam = torch.ones(64, device=dev, dtype=torch.float32)
    out = torch.empty_like(q)
    with pytest.raises(la.LightningAttnError) as ei:
        la.fwd_noalloc(q, q, q, lam, out, chunk=256)
    assert ei.value.status == 5
