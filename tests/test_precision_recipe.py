"""Why the prefill kernels feed every fp32 MFMA operand as a bf16 hi + lo pair.

The block-64 arithmetic of the kernels is modelled here in numpy fp32 (not
the HIP code): per 64-token sub-tile, the inter term q S (S the fp32 state),
the masked decayed scores P times V, and the state update S <- lam^64 S +
K^T (decayed V).  Three products take an operand formed in fp32: S, P and the
decayed V.  Fed to a bf16 MFMA as one RNE bf16 value each, the result of the
64-head workload (decays exp(-2^(-(8/H)(h+1)))) misses the fp64 recurrence of
the oracle by more than the parity rule for bf16 inputs allows (max|err| <=
2e-2 RMS of the reference, fp32 output) on its slowest-decaying head; as hi +
lo pairs (hi = truncation, lo = RNE of the remainder) it stays four orders of
magnitude inside it.  Any one of the three as a single value, the other two
kept as pairs, already spends most of the bound there.  The state stays fp32 either way (MFMA accumulators).
"""
import numpy as np
import pytest
import torch

import oracle.crec as crec
import tolerances as tol
from long_context_decayed_amd.inputs import decay_lambdas, qkv_cpu

H, N, D, BLK = 64, 4096, 128, 64


def _bf16_rne(x):
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32).view(np.float32)


def _hi_lo(x):
    """The value a hi + lo operand pair carries: truncated hi plus RNE remainder."""
    x = np.asarray(x, dtype=np.float32)
    hi = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    return hi + _bf16_rne(x - hi)


def _blockwise(q, k, v, lam, op_s, op_p=None, op_v=None):
    """One head, block 64, fp32 accumulation; op_s, op_p and op_v (all op_s
    unless given) are applied to S, P and the decayed V where they enter a
    product."""
    op_p = op_p or op_s
    op_v = op_v or op_s
    f = np.float32
    pw = np.array([float(lam) ** e for e in range(BLK + 1)], dtype=np.float64).astype(f)
    i = np.arange(BLK)
    dmat = np.where(i[:, None] >= i[None, :], pw[np.clip(i[:, None] - i[None, :], 0, BLK)], 0).astype(f)
    row = pw[1:BLK + 1][:, None]
    vdec = pw[BLK - 1 - i][:, None]
    s = np.zeros((D, D), f)
    o = np.empty((len(q), D), f)
    for t0 in range(0, len(q), BLK):
        qb, kb, vb = q[t0:t0 + BLK], k[t0:t0 + BLK], v[t0:t0 + BLK]
        o[t0:t0 + BLK] = (qb @ op_s(s)) * row + op_p((qb @ kb.T) * dmat) @ vb
        s = s * pw[BLK] + kb.T @ op_v(vb * vdec)
    return o


@pytest.fixture(scope="module")
def workload():
    q, k, v = (t.float().numpy()[0] for t in qkv_cpu(1, H, N, D, seed=7, dtype=torch.bfloat16))
    lam = decay_lambdas(H)
    ref, _ = crec.recurrent(q[None].astype(np.float64), k[None].astype(np.float64), v[None].astype(np.float64),
                            lam.astype(np.float64), want_state=False)
    return q, k, v, lam, ref[0]


def test_single_bf16_operands_break_the_bf16_tolerance(workload):
    q, k, v, lam, ref = workload
    r = tol.rms(ref)
    h = H - 1  # slowest decay: the largest state
    err = float(np.abs(_blockwise(q[h], k[h], v[h], lam[h], _bf16_rne) - ref[h]).max() / r)
    assert err > tol.BF16_RMS, err


def test_any_one_single_operand_spends_most_of_it(workload):
    """No one of the three operands can go single on its own either: with the
    other two kept hi + lo, each alone brings the slowest-decaying head past
    half of the bound (about 0.7 to 1.0 of it on this input)."""
    q, k, v, lam, ref = workload
    r = tol.rms(ref)
    h = H - 1
    for ops in ((_bf16_rne, _hi_lo, _hi_lo), (_hi_lo, _bf16_rne, _hi_lo), (_hi_lo, _hi_lo, _bf16_rne)):
        err = float(np.abs(_blockwise(q[h], k[h], v[h], lam[h], *ops) - ref[h]).max() / r)
        assert err > 0.5 * tol.BF16_RMS, err


def test_hi_lo_operands_meet_it_with_margin(workload):
    q, k, v, lam, ref = workload
    r = tol.rms(ref)
    for h in (0, 40, H - 1):
        err = float(np.abs(_blockwise(q[h], k[h], v[h], lam[h], _hi_lo) - ref[h]).max() / r)
        assert err < 1e-3, (h, err)
