"""Compiled brute-force nearest codewords (``nearest.c``) -- oracle, test infrastructure only.

The same float64 definition as :func:`oracle.codec.encode` and
:func:`oracle.codec.accept_indices` [FQ 2.3], written as plain C loops so that
whole caches can be checked.  Built with gcc into ``oracle/libfq_oracle.so``
(``build()``; loading builds it when it is missing).  Pinned in
``tests/test_oracle_native.py`` against ``codec`` (itself pinned by a
pure-Python loop and ``scipy.spatial.cKDTree``) and against cKDTree directly.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nearest.c")
LIB = os.path.join(HERE, "libfq_oracle.so")
CC = os.environ.get("CC_ORACLE", "gcc")
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99", "-Wall"]

_lib = None


def build(verbose=False):
    """Compile nearest.c (always recompiles)."""
    tmp = LIB + ".tmp"
    r = subprocess.run([CC] + CFLAGS + [SRC, "-o", tmp, "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed for the oracle:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        lib.fqo_nearest.argtypes = [P, I64, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int, P]
        lib.fqo_nearest.restype = ctypes.c_int
        lib.fqo_accept.argtypes = [P, I64, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int, P,
                                   ctypes.c_double, P, P]
        lib.fqo_accept.restype = ctypes.c_int
        lib.fqo_threads.argtypes = [ctypes.c_int]
        lib.fqo_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads(n=0):
    """Set the OpenMP thread count of the searches (n >= 1); return the count in use."""
    return int(library().fqo_threads(int(n)))


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _tables(Pi, C):
    return (np.ascontiguousarray(Pi, dtype=np.float64),
            np.ascontiguousarray(C, dtype=np.float32))


def nearest(x, Pi, C, chunk=1 << 18):
    """Indices [n, nb] (int64) of vectors x [n, d]: codec.encode's indices."""
    x = np.asarray(x)
    n, d = x.shape
    Pi, C = _tables(Pi, C)
    N, k = C.shape
    nb = -(-d // k)
    idx = np.empty((n, nb), dtype=np.int64)
    for s in range(0, n, chunk):
        xs = np.ascontiguousarray(x[s:s + chunk], dtype=np.float64)
        out = np.empty((len(xs), nb), dtype=np.int64)
        if library().fqo_nearest(_p(xs), len(xs), d, _p(Pi), _p(C), N, k, _p(out)) != 0:
            raise ValueError("fqo_nearest: bad arguments")
        idx[s:s + chunk] = out
    return idx


def accept(x, Pi, C, got, window=1e-6, chunk=1 << 18):
    """(n_exact, n_window, n_bad, first_bad_row or -1): codec.accept_indices, compiled.

    Zero vectors must carry index 0 (codec.encode's reading)."""
    x = np.asarray(x)
    n, d = x.shape
    Pi, C = _tables(Pi, C)
    N, k = C.shape
    got = np.asarray(got)
    assert got.shape == (n, -(-d // k)), got.shape
    tot = np.zeros(3, dtype=np.int64)
    first = -1
    for s in range(0, n, chunk):
        xs = np.ascontiguousarray(x[s:s + chunk], dtype=np.float64)
        gs = np.ascontiguousarray(got[s:s + chunk], dtype=np.int64)
        counts = np.zeros(3, dtype=np.int64)
        fb = np.zeros(1, dtype=np.int64)
        if library().fqo_accept(_p(xs), len(xs), d, _p(Pi), _p(C), N, k, _p(gs), float(window),
                                _p(counts), _p(fb)) != 0:
            raise ValueError("fqo_accept: bad arguments")
        tot += counts
        if first < 0 and fb[0] >= 0:
            first = s + int(fb[0])
    return int(tot[0]), int(tot[1]), int(tot[2]), first
