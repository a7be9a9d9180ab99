"""fp64 CPU oracle for causal decayed linear attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library and imports nothing from it.

Parity status of each function (what pins it lives in tests/test_oracle.py):
  quadratic, recurrent, state_at, decode_step, decode_repeated, window --
  pinned by hand-derived exact values, closed forms, textbook reductions,
  invariants and brute force; none is "parity unpinned".
  backward_quadratic and crec.backward (gradients) -- pinned in
  tests/test_oracle_bwd.py by a hand-worked example, exact central
  differences of the forward oracle, closed forms at lam = 0 and 1 and the
  split-sequence rule.
  silu, rmsnorm_heads, sigmoid_gate (the steps either side of the core) --
  pinned in tests/test_oracle_fused.py by closed-form values, limits and
  invariants.
"""
from .lightning import (  # noqa: F401
    decay_matrix,
    quadratic,
    recurrent,
    state_at,
    decode_step,
    decode_repeated,
    window,
    backward_quadratic,
    silu,
    rmsnorm_heads,
    sigmoid_gate,
)
