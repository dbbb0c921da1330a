"""fp64 CPU oracle for the Mamba-3 sequence mixer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and
shares no code with it.  The arithmetic lives in ``m3_oracle.c`` (plain C,
double precision, one POSIX thread per worker over independent (batch, head)
units); this module only builds it with gcc and marshals numpy arrays.

Every function takes and returns float64 numpy arrays in the library's layouts:
    x [Bt,L,H,R,P]   Bm, Cm [Bt,L,H,R,N]   dt, lam [Bt,L,H]   theta [Bt,L,H,N/2]
    A [H]            h [Bt,H,N,P]          Bprev [Bt,H,R,N]   xprev [Bt,H,R,P]
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m3_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libm3oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile m3_oracle.c into libm3oracle.so with gcc (IEEE double, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.m3o_scan.restype = ctypes.c_int
        lib.m3o_scan.argtypes = [_i64] * 6 + [_dp] * 14 + [ctypes.c_int]
        lib.m3o_decode_step.restype = ctypes.c_int
        lib.m3o_decode_step.argtypes = [_i64] * 5 + [_dp] * 11
        _lib = lib
    return _lib


def _arr(a, shape):
    out = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if out.shape != tuple(shape):
        raise ValueError("oracle: expected shape %s, got %s" % (tuple(shape), out.shape))
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def scan(x, Bm, Cm, dt, A, theta, lam, h0=None, Bprev=None, xprev=None, threads=None):
    """Run the recurrence over all L steps.

    Returns (y [Bt,L,H,R,P], h_L [Bt,H,N,P], B_L [Bt,H,R,N], x_L [Bt,H,R,P]).
    ``h0``/``Bprev``/``xprev`` may be None (zero state, zero previous endpoint).
    """
    x = np.asarray(x)
    Bt, L, H, R, P = x.shape
    N = np.asarray(Bm).shape[-1]
    x = _arr(x, (Bt, L, H, R, P))
    Bm = _arr(Bm, (Bt, L, H, R, N))
    Cm = _arr(Cm, (Bt, L, H, R, N))
    dt = _arr(dt, (Bt, L, H))
    lam = _arr(lam, (Bt, L, H))
    theta = _arr(theta, (Bt, L, H, N // 2))
    A = _arr(A, (H,))
    h0 = None if h0 is None else _arr(h0, (Bt, H, N, P))
    if (Bprev is None) != (xprev is None):
        raise ValueError("oracle: Bprev and xprev must be given together")
    Bprev = None if Bprev is None else _arr(Bprev, (Bt, H, R, N))
    xprev = None if xprev is None else _arr(xprev, (Bt, H, R, P))
    y = np.empty((Bt, L, H, R, P))
    h_out = np.empty((Bt, H, N, P))
    Bp_out = np.empty((Bt, H, R, N))
    xp_out = np.empty((Bt, H, R, P))
    nthreads = int(threads) if threads else default_threads()
    rc = _load().m3o_scan(Bt, L, H, P, N, R, _ptr(x), _ptr(Bm), _ptr(Cm), _ptr(dt),
                          _ptr(A), _ptr(theta), _ptr(lam), _ptr(h0), _ptr(Bprev),
                          _ptr(xprev), _ptr(y), _ptr(h_out), _ptr(Bp_out), _ptr(xp_out),
                          nthreads)
    if rc != 0:
        raise RuntimeError("m3o_scan failed with code %d" % rc)
    return y, h_out, Bp_out, xp_out


def decode_step(x, Bm, Cm, dt, A, theta, lam, h, Bprev, xprev):
    """One step on a state record; returns (y_t, h', Bprev', xprev') as new arrays."""
    x = np.asarray(x)
    Bt, H, R, P = x.shape
    N = np.asarray(Bm).shape[-1]
    x = _arr(x, (Bt, H, R, P))
    Bm = _arr(Bm, (Bt, H, R, N))
    Cm = _arr(Cm, (Bt, H, R, N))
    dt = _arr(dt, (Bt, H))
    lam = _arr(lam, (Bt, H))
    theta = _arr(theta, (Bt, H, N // 2))
    A = _arr(A, (H,))
    h = _arr(h, (Bt, H, N, P)).copy()
    Bprev = _arr(Bprev, (Bt, H, R, N)).copy()
    xprev = _arr(xprev, (Bt, H, R, P)).copy()
    y = np.empty((Bt, H, R, P))
    rc = _load().m3o_decode_step(Bt, H, P, N, R, _ptr(x), _ptr(Bm), _ptr(Cm), _ptr(dt),
                                 _ptr(A), _ptr(theta), _ptr(lam), _ptr(h), _ptr(Bprev),
                                 _ptr(xprev), _ptr(y))
    if rc != 0:
        raise RuntimeError("m3o_decode_step failed with code %d" % rc)
    return y, h, Bprev, xprev
