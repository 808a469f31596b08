"""CPU oracle for the GQA exp-sum-div graph (fp64).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg may import this package. The product package never does,
and the two share no code; only the seeded input generator feeds both.

Two independent implementations of the same plain definition (the five
operations of the Mirage GQA tutorial graph, "Mirage: Define GQA Computation
Graph" on the Mirage documentation page):

* ``gqa_f64``      -- plain C loops in double precision (``gqa_oracle.c``),
                      OpenMP over query rows; the oracle the GPU is held to.
* ``gqa_numpy_f64`` -- the same graph as numpy float64 array operations
                      (matmul, exp, sum over the key axis, divide, matmul).

Each takes the exact values of fp16 inputs (converted losslessly to float64)
and returns O in float64. Pins (closed forms, invariants, a library witness and
a high-precision brute force) live in ``tests/test_oracle_pins.py``.

The QK-normalised variant (Mirage documentation tutorial "Implement QK
Normalization and Optimize Attention Kernel in Python" / "Superoptimize
Attention with QK Normalization": Q = rms_norm(Q), K = rms_norm(K), then the
same five operations) is ``gqa_qknorm_f64``: ``rms_norm_f64`` on Q and K,
then ``gqa_f64`` on the normalised values. The pages name rms_norm without
its axis, eps or weight; the reading taken is the one the tutorial's stated
purpose (QK normalisation as in Chameleon, i.e. per attention head vector)
supports: every query row and every key vector (a column of the
head-dim-major K) is divided by the root mean square of its D entries,
eps = 1e-6 inside the square root, no weight. Its pins live in
``tests/test_oracle_qknorm_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqa_oracle.so")
SRC_PATH = os.path.join(_HERE, "gqa_oracle.c")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle with gcc (plain -O2, no fast-math) into this folder."""
    cmd = ["gcc", "-O2", "-march=x86-64-v2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp", SRC_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or (
                os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH)):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.mga_oracle_gqa_f64.argtypes = [dp, dp, dp, dp, ctypes.c_long, ctypes.c_long,
                                           ctypes.c_long, ctypes.c_long]
        lib.mga_oracle_gqa_f64.restype = ctypes.c_int
        lib.mga_oracle_threads.argtypes = []
        lib.mga_oracle_threads.restype = ctypes.c_int
        lib.mga_oracle_set_threads.argtypes = [ctypes.c_int]
        lib.mga_oracle_set_threads.restype = None
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the C oracle runs with (OMP_NUM_THREADS or all cores)."""
    return int(_load().mga_oracle_threads())


def set_threads(n: int) -> None:
    """OpenMP threads for later calls of the C oracle (n >= 1); for timing on
    one core. Results do not depend on it."""
    _load().mga_oracle_set_threads(int(n))


def _as_f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _shapes(q, k, v):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be 3-D")
    B, M, Dh = q.shape
    if k.shape[0] != B or k.shape[1] != Dh:
        raise ValueError(f"k must be (B, D, N) = ({B}, {Dh}, N); got {k.shape}")
    N = k.shape[2]
    if v.shape != (B, N, Dh):
        raise ValueError(f"v must be (B, N, D) = ({B}, {N}, {Dh}); got {v.shape}")
    return B, M, N, Dh


def gqa_f64(q, k, v) -> np.ndarray:
    """O = (exp(QK) / rowsum(exp(QK))) V in fp64, plain C loops.

    q: (B, M, D), k: (B, D, N) head-dim-major, v: (B, N, D). Any real dtype;
    values are taken exactly (fp16 -> fp64 is lossless).
    """
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    B, M, N, Dh = _shapes(q64, k64, v64)
    o = np.empty((B, M, Dh), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = _load().mga_oracle_gqa_f64(q64.ctypes.data_as(dp), k64.ctypes.data_as(dp),
                                    v64.ctypes.data_as(dp), o.ctypes.data_as(dp),
                                    B, M, N, Dh)
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc}); N must be >= 1")
    return o


def gqa_numpy_f64(q, k, v) -> np.ndarray:
    """The same graph as numpy float64 array steps, in the graph's order."""
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    _, _, N, _ = _shapes(q64, k64, v64)
    if N < 1:
        raise ValueError("N must be >= 1")
    A = np.matmul(q64, k64)                 # matmul(Q, K)       (B, M, N)
    E = np.exp(A)                           # exp(A)
    S = E.sum(axis=2, keepdims=True)        # reduction(E, 2)    (B, M, 1)
    Dm = E / S                              # div(E, S)
    return np.matmul(Dm, v64)               # matmul(D, V)       (B, M, D)


def rms_norm_f64(x, axis: int, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(mean(x^2 along `axis`) + eps) in float64, no weight: the
    rms_norm step of the QK-normalised attention tutorial, applied to every
    vector along `axis` (the head dim)."""
    x64 = _as_f64(x)
    ms = np.mean(x64 * x64, axis=axis, keepdims=True)
    return x64 / np.sqrt(ms + eps)


def gqa_qknorm_f64(q, k, v, eps: float = 1e-6) -> np.ndarray:
    """Attention with QK normalisation in fp64: Q = rms_norm(Q) over each
    query row's D entries, K = rms_norm(K) over each key's D entries (axis 1
    of the head-dim-major K), then the GQA graph (gqa_f64) on those values.
    The graph keeps no max subtraction; fp64 holds exp(A) for |A| <= D."""
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    _shapes(q64, k64, v64)
    return gqa_f64(rms_norm_f64(q64, axis=2, eps=eps), rms_norm_f64(k64, axis=1, eps=eps), v64)
