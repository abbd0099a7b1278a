"""CPU oracle for half-precision GEMM and LCMA (Strassen-type) products.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library in ``complexity_half_precision_amd`` and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, compiled with gcc into
``liboracle.so`` by :func:`build`); this module only marshals numpy arrays.

Sources, cited by page title and section:

* "FalconGEMM: Surpassing Hardware Peaks with Lower-Complexity Matrix
  Multiplication" (HyperAI write-up), sections "从 Strassen 出发" (Strassen,
  8 -> 7 and 64 -> 49 block products, the LCMA description, algebraic
  equivalence up to rounding), "从 LCMA 到 FalconGEMM" (combine A/B, batched
  products, combine H) and "从缓存重排到 Cost Model" (fp32 on-chip combine, one
  final cast).
* "CUDA-L2: Surpassing cuBLAS Performance for Matrix Multiplication through
  Reinforcement Learning", section "系统架构与训练" (FP32 CPU ground truth,
  exact match on binary inputs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F16, BF16 = 0, 1
_DT = {"f16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16, F16: F16, BF16: BF16}


def build(verbose: bool = False) -> str:
    """Compile ``oracle.c`` with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        # ORACLE_LIBRARY may name another build of oracle.c (the sanitizer build)
        path = os.environ.get("ORACLE_LIBRARY")
        if not path:
            path = _LIB_PATH
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
                build()
        L = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_encode.argtypes = [i32, vp, vp, i64]
        L.oracle_decode.argtypes = [i32, vp, vp, i64]
        L.oracle_gemm_f64.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64]
        L.oracle_gemm_rows_f64.argtypes = [i64, i64, i64, i64, vp, i64, vp, i64, vp, i64]
        L.oracle_strassen_tables.argtypes = [vp, vp, vp]
        L.oracle_strassen_tables.restype = i32
        L.oracle_naive_tables.argtypes = [i32, i32, i32, vp, vp, vp]
        L.oracle_naive_tables.restype = i32
        L.oracle_kron_tables.argtypes = [i32, i32, i32, i32, vp, vp, vp,
                                         i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_brent_violations.argtypes = [i32, i32, i32, i32, vp, vp, vp]
        L.oracle_brent_violations.restype = i64
        L.oracle_lcma_eval.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, i64, i64, i64,
                                       vp, i64, vp, i64, vp, i64, i32, ctypes.POINTER(i64)]
        L.oracle_lcma_eval.restype = i32
        L.oracle_combine_block.argtypes = [i32, i32, vp, i64, i64, vp, i64, vp, i32]
        L.oracle_combine_block.restype = i32
        L.oracle_set_threads.argtypes = [i32]
        L.oracle_max_threads.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def set_threads(n: int) -> None:
    """Host threads of the product loops (results do not depend on it)."""
    lib().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


# --------------------------------------------------------------------------- encodings

def encode(dtype, x) -> np.ndarray:
    """RNE-encode fp64 values to binary16 (``"f16"``) or bfloat16 (``"bf16"``) bit patterns."""
    x = _f64(x)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_encode(_DT[dtype], _p(x), _p(out), x.size)
    return out


def decode(dtype, h) -> np.ndarray:
    """Decode binary16 / bfloat16 bit patterns exactly to fp64."""
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    out = np.empty(h.shape, dtype=np.float64)
    lib().oracle_decode(_DT[dtype], _p(h), _p(out), h.size)
    return out


def round_to(dtype, x) -> np.ndarray:
    """Value of ``x`` after one round-to-nearest-even rounding to ``dtype``."""
    return decode(dtype, encode(dtype, x))


# --------------------------------------------------------------------------- products

def gemm(A, B) -> np.ndarray:
    """C = A @ B in fp64, each element summed with k ascending (definition of the product)."""
    A, B = _f64(A), _f64(B)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = np.empty((M, N), dtype=np.float64)
    lib().oracle_gemm_f64(M, N, K, _p(A), K, _p(B), N, _p(C), N)
    return C


def gemm_rows(A, B, r0: int, r1: int) -> np.ndarray:
    """Rows [r0, r1) of A @ B (same arithmetic as :func:`gemm`)."""
    A, B = _f64(A), _f64(B)
    M, K = A.shape
    N = B.shape[1]
    C = np.empty((r1 - r0, N), dtype=np.float64)
    lib().oracle_gemm_rows_f64(r0, r1, N, K, _p(A), K, _p(B), N, _p(C), N)
    return C


class Desc:
    """An LCMA description: split sizes and the U/V/W coefficient tables (int8)."""

    def __init__(self, ms, ks, ns, U, V, W):
        self.ms, self.ks, self.ns = int(ms), int(ks), int(ns)
        self.U = np.ascontiguousarray(np.asarray(U, dtype=np.int8).reshape(-1, self.ms * self.ks))
        self.V = np.ascontiguousarray(np.asarray(V, dtype=np.int8).reshape(-1, self.ks * self.ns))
        self.W = np.ascontiguousarray(np.asarray(W, dtype=np.int8).reshape(-1, self.ms * self.ns))
        self.rank = self.U.shape[0]
        if self.V.shape[0] != self.rank or self.W.shape[0] != self.rank:
            raise ValueError("U, V, W ranks differ")


def strassen() -> Desc:
    """Strassen's one-level scheme (2x2x2, rank 7)."""
    U = np.empty(28, np.int8)
    V = np.empty(28, np.int8)
    W = np.empty(28, np.int8)
    lib().oracle_strassen_tables(_p(U), _p(V), _p(W))
    return Desc(2, 2, 2, U, V, W)


def naive(ms=2, ks=2, ns=2) -> Desc:
    """The plain block product written as an LCMA (rank ms*ks*ns)."""
    R = ms * ks * ns
    U = np.empty(R * ms * ks, np.int8)
    V = np.empty(R * ks * ns, np.int8)
    W = np.empty(R * ms * ns, np.int8)
    lib().oracle_naive_tables(ms, ks, ns, _p(U), _p(V), _p(W))
    return Desc(ms, ks, ns, U, V, W)


def kron(d1: Desc, d2: Desc) -> Desc:
    """One-level scheme equal to applying ``d1`` then ``d2`` recursively (outer-major blocks)."""
    ms, ks, ns = d1.ms * d2.ms, d1.ks * d2.ks, d1.ns * d2.ns
    R = d1.rank * d2.rank
    U = np.empty(R * ms * ks, np.int8)
    V = np.empty(R * ks * ns, np.int8)
    W = np.empty(R * ms * ns, np.int8)
    lib().oracle_kron_tables(d1.ms, d1.ks, d1.ns, d1.rank, _p(d1.U), _p(d1.V), _p(d1.W),
                             d2.ms, d2.ks, d2.ns, d2.rank, _p(d2.U), _p(d2.V), _p(d2.W),
                             _p(U), _p(V), _p(W))
    return Desc(ms, ks, ns, U, V, W)


def strassen2() -> Desc:
    """Two-level Strassen (4x4x4, rank 49) as a flat table."""
    s = strassen()
    return kron(s, s)


def magnitude(d: Desc) -> Desc:
    """The scheme with every coefficient replaced by its absolute value.  Its
    exact evaluation on |A|, |B| is sum_r |W_r| (sum |U_r| |A|)(sum |V_r| |B|),
    the magnitude that bounds the rounding errors of an evaluation of ``d``
    (not a valid scheme itself: it does not satisfy Brent's identity)."""
    return Desc(d.ms, d.ks, d.ns, np.abs(d.U), np.abs(d.V), np.abs(d.W))


def brent_violations(d: Desc) -> int:
    """Number of index tuples violating Brent's identity (0 = a valid scheme)."""
    return int(lib().oracle_brent_violations(d.ms, d.ks, d.ns, d.rank, _p(d.U), _p(d.V), _p(d.W)))


def lcma(A, B, d: Desc, levels: int = 1, round_operands=None):
    """Evaluate C = A @ B through the scheme ``d`` applied ``levels`` times.

    ``round_operands`` = None keeps every step exact in fp64; ``"f16"``/``"bf16"``
    rounds each combined operand once (RNE) to that type before its product.
    Returns ``(C, n_block_products)``.
    """
    A, B = _f64(A), _f64(B)
    M, K = A.shape
    N = B.shape[1]
    C = np.empty((M, N), dtype=np.float64)
    cnt = ctypes.c_int64(0)
    rd = -1 if round_operands is None else _DT[round_operands]
    rc = lib().oracle_lcma_eval(d.ms, d.ks, d.ns, d.rank, _p(d.U), _p(d.V), _p(d.W), levels,
                                M, N, K, _p(A), K, _p(B), N, _p(C), N, rd, ctypes.byref(cnt))
    if rc == -1:
        raise ValueError("shape does not split evenly into blocks")
    if rc != 0:
        raise MemoryError("oracle out of memory")
    return C, int(cnt.value)


def combine_block(X, coef, rs: int, cs: int, round_operand=None) -> np.ndarray:
    """round(sum_ab coef[a*cs+b] * X_ab) for X split into rs x cs blocks."""
    X = _f64(X)
    rows, cols = X.shape
    coef = np.ascontiguousarray(np.asarray(coef, dtype=np.int8))
    out = np.empty((rows // rs, cols // cs), dtype=np.float64)
    rd = -1 if round_operand is None else _DT[round_operand]
    rc = lib().oracle_combine_block(rs, cs, _p(coef), rows, cols, _p(X), cols, _p(out), rd)
    if rc != 0:
        raise ValueError("shape does not split evenly into blocks")
    return out
