"""ctypes front end of mfma_model.c: the FP8 scaled-MFMA arithmetic rule the
GPU parity tests use to separate the matrix instruction's own truncation
from a kernel mistake (see the rule at the top of mfma_model.c).  Test
infrastructure only; shares no code with the HIP library or the oracle."""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mfma_model.c")
LIB = os.path.join(HERE, "libmfma_model.so")
FP8 = {"e4m3": 0, "e5m2": 1, 0: 0, 1: 1}
_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-pthread", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        L.mm_model.restype = ctypes.c_int
        L.mm_model.argtypes = [_vp, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _i64, _i64, _vp, _vp,
                               _i64, ctypes.c_double, _vp, _vp, ctypes.c_int]
        _lib = L
    return _lib


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def model(qa, sa, fa, qb, sb, fb, ap, ii=None, jj=None, nthreads=None):
    """(value, allowance) of the FP8 rule.  qa [M][K] and qb [N][K] hold one
    code per byte; sa, sb the [rows][K/32] scale bytes.  With ii/jj: the
    listed entries (1-D results); else the full [M][N] output."""
    qa, sa, qb, sb = _c(qa, np.uint8), _c(sa, np.uint8), _c(qb, np.uint8), _c(sb, np.uint8)
    K = qa.shape[1]
    assert qb.shape[1] == K and sa.shape[1] == K // 32 and sb.shape[1] == K // 32
    N = qb.shape[0]
    if ii is None:
        n, shape, pi, pj = qa.shape[0] * N, (qa.shape[0], N), None, None
    else:
        ii, jj = _c(ii, np.int64), _c(jj, np.int64)
        assert ii.shape == jj.shape and ii.ndim == 1
        assert ii.size == 0 or (ii.min() >= 0 and ii.max() < qa.shape[0] and jj.min() >= 0
                                and jj.max() < N)
        n, shape, pi, pj = ii.size, ii.shape, ii.ctypes.data_as(_vp), jj.ctypes.data_as(_vp)
    val = np.zeros(n, np.float64)
    allow = np.zeros(n, np.float64)
    rc = _load().mm_model(qa.ctypes.data_as(_vp), sa.ctypes.data_as(_vp), FP8[fa],
                          qb.ctypes.data_as(_vp), sb.ctypes.data_as(_vp), FP8[fb], K, N, pi, pj, n,
                          float(ap), val.ctypes.data_as(_vp), allow.ctypes.data_as(_vp),
                          nthreads or os.cpu_count() or 1)
    if rc != 0:
        raise ValueError("mfma model: bad arguments")
    return val.reshape(shape), allow.reshape(shape)
