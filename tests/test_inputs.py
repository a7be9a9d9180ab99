"""CPU checks of the seeded input recipes (no attention arithmetic here)."""
import math

import numpy as np

from long_context_decayed_amd.inputs import decay_lambdas, decay_lambdas_depth


def test_decay_lambdas_workload_values():
    lam = decay_lambdas(64)
    assert lam.dtype == np.float32 and lam.shape == (64,)
    # slope of head h is 2^(-(8/H)(h+1)): head 0 -> 2^-0.125, head 63 -> 2^-8
    assert lam[0] == np.float32(math.exp(-(2.0 ** -0.125)))
    assert lam[63] == np.float32(math.exp(-(2.0 ** -8)))
    assert np.all(np.diff(lam) > 0)


def test_depth_scaled_decays():
    H, L = 64, 70
    assert np.array_equal(decay_lambdas_depth(H, 0, L), decay_lambdas(H))
    assert np.array_equal(decay_lambdas_depth(H, L - 1, L), np.ones(H, np.float32))
    # the slope -ln(lambda) falls linearly with depth
    s = [-np.log(decay_lambdas_depth(H, l, L).astype(np.float64)) for l in (0, 35, 69)]
    # (float32 rounding of lambda near 1 costs ~1e-5 relative in the slope)
    assert np.allclose(s[1], s[0] * (1 - 35 / 69), rtol=1e-4)
