"""Shared helpers for the GPU parity tests: device checks, host copies and the
oracle called on the exact bits the GPU consumed."""
import os
import sys

import numpy as np
import pytest
import torch

import long_context_decayed_amd as la
from oracle import crec


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    # With a GPU present the HIP library must be there: load() raises otherwise.
    la.load()
    return torch.device("cuda:0")


def say(*args):
    """Name the case on stdout (flushed) before a GPU step."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def host(t):
    """Device tensor -> float32 numpy (bf16 values embed exactly)."""
    return t.detach().to(torch.float32).cpu().numpy()


def oracle_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle(q, k, v, lam, s0=None, o_range=None, want_state=True):
    """fp64 recurrence on host arrays [..., N, d]; lam is the float32 decay array."""
    return crec.recurrent(q, k, v, np.asarray(lam, dtype=np.float32).astype(np.float64), s0,
                          o_range=o_range, threads=oracle_threads(), want_state=want_state)


def lam_for(h_count, mode="spec"):
    """float32[H] decays: the workload formula, or all ones / just below one."""
    from long_context_decayed_amd.inputs import decay_lambdas
    if mode == "spec":
        return decay_lambdas(h_count)
    if mode == "one":
        return np.ones(h_count, dtype=np.float32)
    if mode == "near_one":
        return np.full(h_count, 1.0 - 2.0 ** -20, dtype=np.float32)
    raise ValueError(mode)
