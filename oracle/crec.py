"""ctypes wrapper for the plain-C fp64 recurrence in oracle/recurrence.c.

TEST INFRASTRUCTURE ONLY (test suite, smoke check, CPU-baseline leg).

The library is built by the repository's build step; if it is missing it is
compiled here with gcc on first use.  Results are checked against the NumPy
forms in tests/test_oracle.py."""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "recurrence.c")
LIB_PATH = os.path.join(_HERE, "liboracle_rec.so")
_lib = None


def build(force=False):
    """Compile oracle/recurrence.c into oracle/liboracle_rec.so with gcc."""
    if force or not os.path.exists(LIB_PATH) or (
        os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp]
        )
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(LIB_PATH)
        lib.lcd_oracle_recurrent.restype = ctypes.c_int
        lib.lcd_oracle_recurrent.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
        ]
        lib.lcd_oracle_backward.restype = ctypes.c_int
        lib.lcd_oracle_backward.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
        ]
        lib.lcd_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads():
    return int(_load().lcd_oracle_max_threads())


def recurrent(q, k, v, lam, s0=None, o_range=None, threads=0, want_state=True):
    """fp64 recurrence over arrays [..., N, d]; lam broadcasts to the leading dims.

    o_range=(t0, t1) stores only o_t for t0 <= t < t1 (default: all tokens).
    Returns (O [..., t1-t0, d] float64, S_final [..., d, d] float64 or None)."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    lead = q.shape[:-2]
    n, d = q.shape[-2], q.shape[-1]
    assert k.shape == q.shape and v.shape == q.shape
    pairs = int(np.prod(lead)) if lead else 1
    lam_p = np.ascontiguousarray(
        np.broadcast_to(np.asarray(lam, dtype=np.float64), lead).reshape(pairs)
    )
    if s0 is not None:
        s0 = np.ascontiguousarray(np.broadcast_to(np.asarray(s0, dtype=np.float64), lead + (d, d)))
    t0, t1 = (0, n) if o_range is None else o_range
    assert 0 <= t0 <= t1 <= n
    o = np.zeros(lead + (t1 - t0, d), dtype=np.float64)
    s_fin = np.zeros(lead + (d, d), dtype=np.float64) if want_state else None
    rc = lib.lcd_oracle_recurrent(
        q.ctypes.data, k.ctypes.data, v.ctypes.data,
        lam_p.ctypes.data, None if s0 is None else s0.ctypes.data,
        o.ctypes.data, t0, t1,
        None if s_fin is None else s_fin.ctypes.data,
        pairs, n, d, int(threads),
    )
    if rc != 0:
        raise MemoryError("oracle recurrence could not allocate its scratch state")
    return o, s_fin


def backward(q, k, v, lam, dout, s0=None, dsn=None, threads=0):
    """fp64 gradients of the recurrence (adjoint recurrence in plain C) for
    arrays [..., N, d]: dout = dL/dO, dsn = dL/dS_final (None = 0).
    Returns (dQ, dK, dV [..., N, d], dS0 [..., d, d]) in float64."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    dout = np.ascontiguousarray(dout, dtype=np.float32)
    lead = q.shape[:-2]
    n, d = q.shape[-2], q.shape[-1]
    assert k.shape == q.shape and v.shape == q.shape and dout.shape == q.shape
    pairs = int(np.prod(lead)) if lead else 1
    lam_p = np.ascontiguousarray(
        np.broadcast_to(np.asarray(lam, dtype=np.float64), lead).reshape(pairs)
    )
    def st(x):
        if x is None:
            return None
        return np.ascontiguousarray(np.broadcast_to(np.asarray(x, dtype=np.float64), lead + (d, d)))
    s0, dsn = st(s0), st(dsn)
    dq = np.zeros(lead + (n, d)); dk = np.zeros(lead + (n, d)); dv = np.zeros(lead + (n, d))
    ds0 = np.zeros(lead + (d, d))
    rc = lib.lcd_oracle_backward(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, lam_p.ctypes.data,
        None if s0 is None else s0.ctypes.data, dout.ctypes.data, None if dsn is None else dsn.ctypes.data,
        dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, ds0.ctypes.data,
        pairs, n, d, int(threads),
    )
    if rc != 0:
        raise MemoryError("oracle backward could not allocate its scratch state")
    return dq, dk, dv, ds0
