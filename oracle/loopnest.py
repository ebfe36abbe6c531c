"""Loop-nest fp64 reference of a linear layer's F, B and W products (C,
OpenMP over output rows) -- the oracle's plain definition of the three
products, loaded from ``oracle/libzb_oracle.so`` (compiled from
``oracle/loopnest.c`` with gcc; compiled here on first use if missing).

TEST INFRASTRUCTURE ONLY: used by the tests and by the benchmark's
CPU-baseline leg, never by the product library.

"Zero-Bubble Pipeline Parallelism Guide for LLMs", section "Core Innovation
1: Mathematical Decomposition of the Backward Pass": the backward of a
linear layer splits into the input gradient (dX from dY and W) and the
weight gradient (dW from dY and the stashed X), accumulated over
microbatches.  Weights are [out][in]:

    F: Y = X W^T     B: dX = dY W     W: dW += dY^T X
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "loopnest.c")
LIB = os.path.join(HERE, "libzb_oracle.so")
GCC_CMD = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", SRC, "-o", LIB]

_lib = None


def build() -> str:
    """Compile loopnest.c into libzb_oracle.so (plain -O2, no
    architecture-specific flags)."""
    tmp = LIB + ".tmp"
    r = subprocess.run(GCC_CMD[:-1] + [tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed:\n{' '.join(GCC_CMD)}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.POINTER(ctypes.c_double)
        for name in ("zbo_linear_fwd", "zbo_linear_bwd_input", "zbo_linear_bwd_weight"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P]
        L.zbo_max_threads.restype = ctypes.c_int
        L.zbo_max_threads.argtypes = []
        _lib = L
    return _lib


def _f64(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def threads() -> int:
    """OpenMP threads the loop nests run on."""
    return int(lib().zbo_max_threads())


def linear_fwd(X, W) -> np.ndarray:
    """Y[t][o] = sum_i X[t][i] W[o][i]."""
    X, W = _f64(X), _f64(W)
    T, n_in = X.shape
    n_out = W.shape[0]
    if W.shape[1] != n_in:
        raise ValueError("linear_fwd: X and W widths differ")
    Y = np.empty((T, n_out), dtype=np.float64)
    lib().zbo_linear_fwd(T, n_in, n_out, _p(X), _p(W), _p(Y))
    return Y


def linear_bwd_input(dY, W) -> np.ndarray:
    """dX[t][i] = sum_o dY[t][o] W[o][i]."""
    dY, W = _f64(dY), _f64(W)
    T, n_out = dY.shape
    n_in = W.shape[1]
    if W.shape[0] != n_out:
        raise ValueError("linear_bwd_input: dY and W widths differ")
    dX = np.empty((T, n_in), dtype=np.float64)
    lib().zbo_linear_bwd_input(T, n_in, n_out, _p(dY), _p(W), _p(dX))
    return dX


def linear_bwd_weight(dY, X, dW) -> np.ndarray:
    """dW[o][i] += sum_t dY[t][o] X[t][i], in place on the float64 array dW
    (returned)."""
    dY, X = _f64(dY), _f64(X)
    T, n_out = dY.shape
    n_in = X.shape[1]
    if X.shape[0] != T or dW.shape != (n_out, n_in) or dW.dtype != np.float64 or not dW.flags.c_contiguous:
        raise ValueError("linear_bwd_weight: shapes or dW layout")
    lib().zbo_linear_bwd_weight(T, n_in, n_out, _p(dY), _p(X), _p(dW))
    return dW
