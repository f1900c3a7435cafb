"""ctypes loader for the plain-C oracle twin (oracle/gdn_ref.c).

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the bench).
``build()`` compiles ``liboracle_ref.so`` next to this file with gcc.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_ref.c")
# GDN_ORACLE_LIBRARY selects another build of gdn_ref.c (for instance the
# host-sanitized one that tests/sanitize_host.py builds); it is never rebuilt here
_LIB_ENV = os.environ.get("GDN_ORACLE_LIBRARY")
_LIB = _LIB_ENV or os.path.join(_HERE, "liboracle_ref.so")
_lib = None


def build(verbose=False):
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           _SRC, "-o", _LIB, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def _load():
    global _lib
    if _lib is None:
        if not _LIB_ENV and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER(ctypes.c_double)
        I, D = ctypes.c_int, ctypes.c_double
        lib.gdn_ref_cte.argtypes = [P, P, P, P, P, D, P, P, P, I, I, I, I, I, I]
        lib.gdn_ref_cte.restype = None
        lib.gdn_ref_tkg.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, D, D]
        lib.gdn_ref_tkg.restype = None
        lib.gdn_ref_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _c(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return _load().gdn_ref_num_threads()


def cte(query, key, value, g_log, beta, scale=1.0, initial_state=None):
    """Same contract as oracle.gdn_ref.cte."""
    lib = _load()
    q, k, v, g, b = map(_c, (query, key, value, g_log, beta))
    B, Hk, S, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[3]
    out = np.empty((B, Hv, S, Dv))
    state = np.empty((B, Hv, Dk, Dv))
    s0 = None if initial_state is None else _c(initial_state)
    lib.gdn_ref_cte(_p(q), _p(k), _p(v), _p(g), _p(b), float(scale),
                    None if s0 is None else _p(s0), _p(out), _p(state),
                    B, Hk, Hv, S, Dk, Dv)
    return out, state


def tkg_unrounded(q, k, v, b, a, A_log, dt_bias, z, norm_weight, state_in,
                  num_v_heads, rms_eps=1e-6, l2_eps=1e-6):
    """Decode step; returns (y before the bf16 rounding, state')."""
    lib = _load()
    q, k, v, b, a, A_log, dt_bias, z, w, s0 = map(
        _c, (q, k, v, b, a, A_log, dt_bias, z, norm_weight, state_in))
    BH, K = q.shape
    V = v.shape[1]
    s1 = np.empty((BH, K, V))
    y = np.empty((BH, V))
    lib.gdn_ref_tkg(_p(q), _p(k), _p(v), _p(b), _p(a), _p(A_log), _p(dt_bias),
                    _p(z), _p(w), _p(s0), _p(s1), _p(y), BH, num_v_heads, K, V,
                    float(l2_eps), float(rms_eps))
    return y, s1
