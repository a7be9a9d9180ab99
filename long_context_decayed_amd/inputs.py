"""Seeded synthetic inputs for causal decayed linear attention.

This module holds only random-number recipes and the per-head decay table of
the workloads; none of the attention arithmetic.  Both the HIP path and the
fp64 oracle are fed from it, so they see the same bits.

Workload recipe
---------------
* Per-head decay.  The MiniMax-M1 fact sheet (archdb), "linear / SSM layer
  configuration" field, gives each lightning head a fixed exponential decay
  with ALiBi-style slopes.  With H heads the slope of head h is
  2^(-(8/H)(h+1)) and the decay is lambda_h = exp(-slope), evaluated in float64
  and rounded once to float32 (H = 64: lambda_0 = 0.39971, lambda_63 = 0.99610).
* Depth-scaled decays.  The same field says the slopes are scaled down
  linearly with depth without giving the law; the plainest reading is
  slope_h * (1 - l / (L - 1)) for layer l of L, so the first layer has the
  slopes above and the last has none (lambda = 1).
* Q, K, V ~ N(0, 1) / sqrt(d): Gaussian stand-ins for the SiLU-activated
  projections of a trained layer (no weights are involved).
* Initial states ~ N(0, std^2) in float32 (std = 0.1 by default).
"""
import math

import numpy as np
import torch

__all__ = [
    "decay_lambdas",
    "decay_lambdas_depth",
    "qkv_cpu",
    "qkv_device",
    "state_device",
    "state_cpu",
    "ternary_device",
]


def decay_lambdas(h_count):
    """float32[H]: lambda_h = exp(-2^(-(8/H)(h+1))), fp64 then one rounding."""
    lam = [math.exp(-(2.0 ** (-(8.0 / h_count) * (h + 1)))) for h in range(h_count)]
    return np.asarray(lam, dtype=np.float64).astype(np.float32)


def decay_lambdas_depth(h_count, layer, n_layers):
    """float32[H] for layer `layer` of `n_layers`: the slopes of decay_lambdas
    scaled by (1 - layer / (n_layers - 1)), fp64 then one rounding."""
    scale = 1.0 - layer / (n_layers - 1) if n_layers > 1 else 1.0
    lam = [math.exp(-(2.0 ** (-(8.0 / h_count) * (h + 1))) * scale) for h in range(h_count)]
    return np.asarray(lam, dtype=np.float64).astype(np.float32)


def qkv_cpu(b, h, n, d, seed=0, dtype=torch.float32):
    """Q, K, V drawn in that order from torch's CPU generator, / sqrt(d).

    Draws happen in float32 and are then cast (RNE) to `dtype`."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    out = []
    for _ in range(3):
        x = torch.randn((b, h, n, d), generator=g, dtype=torch.float32)
        x.mul_(1.0 / math.sqrt(d))
        out.append(x.to(dtype))
    return tuple(out)


def _dev_gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def qkv_device(b, h, n, d, seed, device="cuda", dtype=torch.bfloat16, slice_tokens=None):
    """Q, K, V generated on the device, / sqrt(d), in `dtype`.

    Tensor i (Q=0, K=1, V=2) uses seed*1000003 + i.  Large tensors are filled
    in slices of `slice_tokens` tokens per (b, h) so that no float32 copy of a
    whole tensor is ever materialised; slice j of tensor i is drawn from its
    own generator seeded with (seed*1000003 + i)*65537 + j."""
    out = []
    scale = 1.0 / math.sqrt(d)
    for i in range(3):
        x = torch.empty((b, h, n, d), device=device, dtype=dtype)
        base = seed * 1000003 + i
        if slice_tokens is None or slice_tokens >= n:
            g = _dev_gen(device, base)
            tmp = torch.randn((b, h, n, d), generator=g, device=device, dtype=torch.float32)
            x.copy_(tmp.mul_(scale))
            del tmp
        else:
            for j, t0 in enumerate(range(0, n, slice_tokens)):
                t1 = min(n, t0 + slice_tokens)
                g = _dev_gen(device, base * 65537 + j)
                tmp = torch.randn((b, h, t1 - t0, d), generator=g, device=device,
                                  dtype=torch.float32)
                x[:, :, t0:t1, :].copy_(tmp.mul_(scale))
                del tmp
        out.append(x)
    return tuple(out)


def state_device(b, h, d, seed, std=0.1, device="cuda"):
    """float32 [B, H, d, d] ~ N(0, std^2), one generator seeded with seed*7919+5."""
    g = _dev_gen(device, seed * 7919 + 5)
    return torch.randn((b, h, d, d), generator=g, device=device, dtype=torch.float32).mul_(std)


def state_cpu(b, h, d, seed, std=0.1):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 7919 + 5)
    return torch.randn((b, h, d, d), generator=g, dtype=torch.float32).mul_(std)


def ternary_device(b, h, n, d, seed, device="cuda", dtype=torch.float32):
    """Q, K, V with entries drawn uniformly from {-1, 0, 1}."""
    out = []
    for i in range(3):
        g = _dev_gen(device, seed * 1000003 + 17 + i)
        x = torch.randint(-1, 2, (b, h, n, d), generator=g, device=device, dtype=torch.int32)
        out.append(x.to(dtype))
    return tuple(out)
