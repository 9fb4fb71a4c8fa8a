"""ctypes front end of the C fp64 oracle (oracle/ss_oracle.c).

TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the bench's CPU
baseline.  ``build()`` compiles the C file with gcc; ``load()`` builds it first
when the shared object is missing or older than its source.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ss_oracle.c")
LIB = os.path.join(HERE, "libs6oracle.so")

_lib = None


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                           "-shared", "-fPIC", "-std=c11", "-o", tmp, SRC, "-lm"])
    os.replace(tmp, LIB)
    return LIB


def load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.s6o_threads.argtypes = [ctypes.c_int]
        lib.s6o_threads.restype = ctypes.c_int
        lib.s6o_fwd.argtypes = [I, I, I, I] + [P] * 9 + [P, I, P, P, ctypes.c_int]
        lib.s6o_fwd.restype = ctypes.c_int
        lib.s6o_bwd.argtypes = [I, I, I, I] + [P] * 11 + [P] * 9 + [ctypes.c_int]
        lib.s6o_bwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def threads(n: int = 0) -> int:
    """Set (n > 0) and return the OpenMP thread count the oracle runs with."""
    return load().s6o_threads(int(n))


def fwd(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z=None, h0=None, chans=None, want_h_final=True,
        zoh=False):
    """Forward for all channels (chans None) or for channels chans[i] = b*D + d.

    Returns (y, h_final): y [B,D,L] (all) or [len(chans), L]; h_final likewise with N.
    zoh: exact zero-order-hold B̄ instead of the first-order δ·B.
    """
    lib = load()
    x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0 = map(
        _f32, (x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0))
    Bn, D, L = x.shape
    N = A.shape[1]
    if chans is None:
        nchan = Bn * D
        c_arr = None
        y = np.empty((Bn, D, L))
        hf = np.empty((Bn, D, N)) if want_h_final else None
    else:
        c_arr = np.ascontiguousarray(chans, dtype=np.int64)
        nchan = c_arr.size
        y = np.empty((nchan, L))
        hf = np.empty((nchan, N)) if want_h_final else None
    rc = lib.s6o_fwd(Bn, L, D, N, _p(x), _p(dt_raw), _p(dt_bias), _p(A), _p(Bm), _p(Cm),
                     _p(Dskip), _p(z), _p(h0), _p(c_arr), nchan, _p(y), _p(hf), int(bool(zoh)))
    if rc != 0:
        raise RuntimeError(f"s6o_fwd failed: {rc}")
    return y, hf


def bwd(x, dt_raw, dt_bias, A, Bm, Cm, Dskip, dy, z=None, h0=None, dh_final=None, zoh=False):
    """Backward over all channels.  Returns the same dict as oracle.ss_ref.ss_bwd.
    zoh: gradients of the exact zero-order-hold forward."""
    lib = load()
    x, dt_raw, dt_bias, A, Bm, Cm, Dskip, dy, z, h0, dh_final = map(
        _f32, (x, dt_raw, dt_bias, A, Bm, Cm, Dskip, dy, z, h0, dh_final))
    Bn, D, L = x.shape
    N = A.shape[1]
    out = dict(dx=np.empty((Bn, D, L)), ddt_raw=np.empty((Bn, D, L)),
               dz=np.empty((Bn, D, L)) if z is not None else None,
               ddt_bias=np.empty(D), dA=np.empty((D, N)),
               dB=np.empty((Bn, N, L)), dC=np.empty((Bn, N, L)), dD=np.empty(D),
               dh0=np.empty((Bn, D, N)) if h0 is not None else None)
    rc = lib.s6o_bwd(Bn, L, D, N, _p(x), _p(dt_raw), _p(dt_bias), _p(A), _p(Bm), _p(Cm),
                     _p(Dskip), _p(z), _p(h0), _p(dy), _p(dh_final),
                     _p(out["dx"]), _p(out["ddt_raw"]), _p(out["dz"]), _p(out["ddt_bias"]),
                     _p(out["dA"]), _p(out["dB"]), _p(out["dC"]), _p(out["dD"]), _p(out["dh0"]), int(bool(zoh)))
    if rc != 0:
        raise RuntimeError(f"s6o_bwd failed: {rc}")
    return out
