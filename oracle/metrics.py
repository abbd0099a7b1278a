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
* ``bound_classic`` / ``bound_lcma`` + ``elementwise``: a per-element error
  bound, so a single wrong tile cannot hide inside a norm.  Classic:
  |C - C_ref| <= u_out |C_ref| + (1 + u_out) gamma_K (|A||B|) + eta, where
  gamma_K = 2 K u_32 bounds fp32 accumulation of K products in any order
  (the factor 2 also covers accumulators that truncate) and eta is half the
  output type's smallest subnormal.  LCMA: the same against the oracle's
  evaluation of the same scheme with the same operand rounding, with
  (|A||B|) replaced by the scheme's magnitude sum_r |W_r| |Ahat_r| |Bhat_r|
  and K by the block depth plus the number of fp32 folds per output.
* ``freivalds_bands``: the Freivalds residual per band of 128 rows (and of
  128 columns, from y^T C - (y^T A) B), each relative to that band's
  reference norm: O(N^2) work that still sees a single wrong 16 x 16 tile
  in a 16384 x 16384 result (the residual of correctly rounded outputs sits
  near 0.5 u_out per band, a zeroed 16 x 16 tile among 16384 columns adds
  about 2.8 u_out).

Why these: the FalconGEMM write-up (section "从缓存重排到 Cost Model") notes
that reordering sums changes rounding, so results are compared within a
tolerance, while the CUDA-L2 explanation (section "系统架构与训练") asks for an
FP32 CPU truth and exact agreement on binary inputs.
"""
from __future__ import annotations

import numpy as np

GATE_NW = {"f16": 1e-3, "bf16": 8e-3}
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
U32 = 2.0 ** -24                                         # fp32 unit roundoff
HALF_SUBNORMAL = {"f16": 2.0 ** -25, "bf16": 2.0 ** -134}


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


def bound_classic(C_ref, absAB, K, dtype):
    """Per-element error bound of a half-precision GEMM with fp32 accumulation
    and one rounding to ``dtype``: absAB = |A| |B| (fp64, from the oracle)."""
    u = UNIT_ROUNDOFF[dtype]
    gamma = 2.0 * K * U32
    return u * np.abs(np.asarray(C_ref, np.float64)) + (1.0 + u) * gamma * np.asarray(absAB, np.float64) \
        + HALF_SUBNORMAL[dtype]


def bound_lcma(C_sh, mag, depth, folds, dtype, op_dtype):
    """Per-element error bound of an LCMA result against the oracle's evaluation
    of the same scheme with operands rounded to ``op_dtype`` (C_sh, unrounded).
    mag = sum_r |W_r| (sum |U_r| |A|)(sum |V_r| |B|), exact; each |Ahat_r| is at
    most (1 + u_op) times its unrounded magnitude.  depth: k-extent of one
    block product; folds: fp32 additions of products into one output."""
    u = UNIT_ROUNDOFF[dtype]
    u_op = UNIT_ROUNDOFF[op_dtype]
    gamma = 2.0 * (depth + folds) * U32
    return u * np.abs(np.asarray(C_sh, np.float64)) \
        + (1.0 + u) * gamma * (1.0 + u_op) ** 2 * np.asarray(mag, np.float64) + HALF_SUBNORMAL[dtype]


def elementwise(C, C_ref, bound):
    """(largest |C - C_ref| / bound, number of elements above their bound)."""
    d = np.abs(np.asarray(C, np.float64) - np.asarray(C_ref, np.float64))
    r = d / np.asarray(bound, np.float64)
    r[np.isnan(r)] = np.inf
    return float(r.max()) if r.size else 0.0, int(np.count_nonzero(r > 1.0))


def freivalds_bands(C, A, B, band=128, seed=11):
    """Relative Freivalds residuals per band: for a seeded x in {-1, 1}^N,
    ||(C x - A (B x))_b|| / ||(A (B x))_b|| for each band b of ``band`` rows,
    and for a seeded y in {-1, 1}^M the same of y^T C - (y^T A) B per band of
    ``band`` columns.  Returns (row residuals, column residuals)."""
    C = np.asarray(C, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    M, N = C.shape
    rng = np.random.default_rng(seed)
    x = rng.integers(0, 2, size=N).astype(np.float64) * 2.0 - 1.0
    y = rng.integers(0, 2, size=M).astype(np.float64) * 2.0 - 1.0
    ref_r = A @ (B @ x)
    res_r = C @ x - ref_r
    ref_c = (y @ A) @ B
    res_c = y @ C - ref_c

    def rel(res, ref, n):
        out = []
        for b in range(0, n, band):
            den = float(np.linalg.norm(ref[b:b + band]))
            num = float(np.linalg.norm(res[b:b + band]))
            out.append(num / den if den > 0 else num)
        return np.array(out)
    return rel(res_r, ref_r, M), rel(res_c, ref_c, N)
