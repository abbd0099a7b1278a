"""Error metrics and gates used to compare a GPU result with the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain numpy in fp64.

* ``e_nw``: normwise error ||C - C_ref||_F / (||A||_F * ||B||_F), the gate for
  half-precision GEMM (<= 1e-3 for binary16, <= 8e-3 for bfloat16).
* ``e_rel``: ||C - C_ref||_F / ||C_ref||_F, whole matrix or per output block.
  The normwise gate alone is blind at large K (||AB||_F / (||A||_F ||B||_F)
  shrinks like 1/sqrt(K) for independent entries), so the tests also require
  e_rel <= 4 u_out, where u_out is the unit roundoff of the output type.
* ``freivalds``: ||C x - A (B x)||_2 / ||A (B x)||_2 for random sign vectors x;
  O(MK + KN) work, so it checks shapes whose full product is too costly.

Why these: the FalconGEMM write-up (section "从缓存重排到 Cost Model") notes
that reordering sums changes rounding, so results are compared within a
tolerance, while the CUDA-L2 explanation (section "系统架构与训练") asks for an
FP32 CPU truth and exact agreement on binary inputs.
"""
from __future__ import annotations

import numpy as np

GATE_NW = {"f16": 1e-3, "bf16": 8e-3}
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def fro(X) -> float:
    return float(np.sqrt(np.sum(np.square(np.asarray(X, dtype=np.float64)))))


def e_nw(C, C_ref, A, B) -> float:
    d = np.asarray(C, np.float64) - np.asarray(C_ref, np.float64)
    den = fro(A) * fro(B)
    return fro(d) / den if den > 0 else fro(d)


def e_rel(C, C_ref) -> float:
    d = np.asarray(C, np.float64) - np.asarray(C_ref, np.float64)
    den = fro(C_ref)
    return fro(d) / den if den > 0 else fro(d)


def e_rel_blocks(C, C_ref, bs: int):
    """e_rel of each of the bs x bs output blocks (rows/cols split evenly, last one ragged)."""
    C = np.asarray(C, np.float64)
    C_ref = np.asarray(C_ref, np.float64)
    M, N = C.shape
    out = []
    rb = [(M * i) // bs for i in range(bs + 1)]
    cb = [(N * j) // bs for j in range(bs + 1)]
    for i in range(bs):
        for j in range(bs):
            out.append(e_rel(C[rb[i]:rb[i + 1], cb[j]:cb[j + 1]], C_ref[rb[i]:rb[i + 1], cb[j]:cb[j + 1]]))
    return out


def freivalds(C, A, B, seeds=(11, 12, 13)) -> float:
    """max over seeded x in {-1, +1}^N of ||C x - A (B x)|| / ||A (B x)||."""
    C = np.asarray(C, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    worst = 0.0
    for s in seeds:
        x = np.random.default_rng(s).integers(0, 2, size=B.shape[1]).astype(np.float64) * 2.0 - 1.0
        ref = A @ (B @ x)
        got = C @ x
        den = float(np.linalg.norm(ref))
        err = float(np.linalg.norm(got - ref))
        worst = max(worst, err / den if den > 0 else err)
    return worst
