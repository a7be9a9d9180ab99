"""Parity criteria between the HIP path and the fp64 oracle.

  * fp32 inputs and outputs: max|O - O_ref| <= 1e-4 * max|O_ref| (normwise
    relative error; elementwise relative error is ill-posed near zero).
  * bf16 inputs, fp32 output: max|O - O_ref| <= 2e-2 * RMS(O_ref), RMS over the
    whole tensor (or sample) checked.
  * bf16 inputs, bf16 output: elementwise |O - O_ref| <= 2e-2 * RMS(O_ref)
    + 2^-8 * |O_ref|.  The extra term is the final round-to-nearest-even to
    bf16, whose error is at most half an ulp, i.e. at most 2^-8 of the value:
    rounding the EXACT result alone already exceeds 2e-2 * RMS on the 64-head
    workloads (slow-decay heads reach about 12x the RMS, and half an ulp of
    those is about 2.5e-2 * RMS), so no bf16-stored output could meet the
    RMS-only rule.  The same kernels also store fp32, and bf16 out must equal
    RNE(fp32 out) bit for bit, which ties the two.
  * fp32 states: max|S - S_ref| <= 1e-3 * max|S_ref|.
"""
import numpy as np

FP32_REL = 1e-4
BF16_RMS = 2e-2
BF16_STORE = 2.0 ** -8
STATE_REL = 1e-3


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def fp32_error(o, ref):
    o, ref = _f64(o), _f64(ref)
    return float(np.abs(o - ref).max() / max(np.abs(ref).max(), 1e-300))


def rms(x):
    x = _f64(x)
    return float(np.sqrt(np.mean(x * x)))


def bf16_rms_error(o, ref, ref_rms=None):
    """max|O - O_ref| / RMS(O_ref)."""
    o, ref = _f64(o), _f64(ref)
    r = rms(ref) if ref_rms is None else ref_rms
    return float(np.abs(o - ref).max() / r)


def bf16_store_violations(o, ref, ref_rms=None):
    """Number of elements breaking |O - O_ref| <= 2e-2 RMS + 2^-8 |O_ref|."""
    o, ref = _f64(o), _f64(ref)
    r = rms(ref) if ref_rms is None else ref_rms
    bound = BF16_RMS * r + BF16_STORE * np.abs(ref)
    return int(np.count_nonzero(np.abs(o - ref) > bound))


def state_error(s, ref):
    s, ref = _f64(s), _f64(ref)
    return float(np.abs(s - ref).max() / max(np.abs(ref).max(), 1e-300))


def assert_fp32(o, ref, what="O"):
    e = fp32_error(o, ref)
    assert e <= FP32_REL, "%s: normwise relative error %.3e > %.1e" % (what, e, FP32_REL)
    return e


def assert_bf16_f32out(o, ref, what="O", ref_rms=None):
    e = bf16_rms_error(o, ref, ref_rms)
    assert e <= BF16_RMS, "%s: max|err| = %.3e x RMS > %.1e" % (what, e, BF16_RMS)
    return e


def assert_bf16_out(o, ref, what="O", ref_rms=None):
    n = bf16_store_violations(o, ref, ref_rms)
    assert n == 0, "%s: %d elements outside 2e-2*RMS + 2^-8*|ref|" % (what, n)


def assert_state(s, ref, what="state"):
    e = state_error(s, ref)
    assert e <= STATE_REL, "%s: relative error %.3e > %.1e" % (what, e, STATE_REL)
    return e
