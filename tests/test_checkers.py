"""The GPU tests' checkers, pinned on the CPU: each must pass a correctly
rounded result and reject the mistakes a kernel plausibly makes (a zeroed
16 x 16 MFMA tile, a k-slice dropped from one tile, a wrong product sign).
Results are emulated from the oracle: the exact product (or the exact
evaluation of the scheme with rounded operands) rounded once to the output
type, which is what the GPU path computes up to fp32 accumulation order.
"""
import numpy as np
import pytest

import descriptors as D
import oracle
import seeded_inputs as si
from oracle import metrics


def emulate(dtype, C):
    return oracle.round_to(dtype, C)


def test_elementwise_bound_rejects_one_zeroed_tile_in_a_4096_square_bf16_result():
    M = N = 4096
    K = 256
    A, B = si.gen(M, N, K, "bf16", "normal_sqrtk", 5)
    A64, B64 = si.f64(A), si.f64(B)
    ref = oracle.gemm(A64, B64)
    bound = metrics.bound_classic(ref, oracle.gemm(np.abs(A64), np.abs(B64)), K, "bf16")
    C = emulate("bf16", ref)
    worst, bad = metrics.elementwise(C, ref, bound)
    assert bad == 0 and worst <= 1.0
    # the normwise gates cannot see it: one tile among 2048^2-element blocks
    rng = np.random.default_rng(1)
    i, j = (int(v) * 16 for v in rng.integers(0, 256, 2))
    Cz = C.copy()
    Cz[i:i + 16, j:j + 16] = 0.0
    assert metrics.e_rel(Cz, ref) <= 4 * metrics.UNIT_ROUNDOFF["bf16"]
    assert max(metrics.e_rel_blocks(Cz, ref, 2)) <= 4 * metrics.UNIT_ROUNDOFF["bf16"]
    _, bad = metrics.elementwise(Cz, ref, bound)
    assert bad >= 250
    # one tile missing the products of one 32-wide k-slice
    Ck = C.copy()
    ks = slice(64, 96)
    Ck[i:i + 16, j:j + 16] = emulate("bf16", ref[i:i + 16, j:j + 16] - A64[i:i + 16, ks] @ B64[ks, j:j + 16])
    _, bad = metrics.elementwise(Ck, ref, bound)
    assert bad >= 200


def test_elementwise_bound_of_a_scheme_evaluation():
    M, N, K = 1024, 768, 512
    for dtype, dist, ops, lv in (("bf16", "normal_sqrtk", "bf16", 1), ("f16", "uniform", "f16", 1),
                                 ("bf16", "normal_sqrtk", "f16", 2)):
        A, B = si.gen(M, N, K, dtype, dist, 6)
        A64, B64 = si.f64(A), si.f64(B)
        d = oracle.strassen() if lv == 1 else oracle.strassen2()
        C_sh, _ = oracle.lcma(A64, B64, d, 1, round_operands=ops)
        mag, _ = oracle.lcma(np.abs(A64), np.abs(B64), oracle.magnitude(d), 1)
        bound = metrics.bound_lcma(C_sh, mag, K // d.ks, 4 if lv == 1 else 16, dtype, ops)
        C = emulate(dtype, C_sh)
        worst, bad = metrics.elementwise(C, C_sh, bound)
        assert bad == 0, (dtype, lv)
        Cz = C.copy()
        Cz[512:528, 256:272] = 0.0
        assert metrics.elementwise(Cz, C_sh, bound)[1] >= 250, (dtype, lv)
        # a wrong sign on one product's contribution
        Wbad = d.W.copy()
        r = int(np.flatnonzero(Wbad[:, 0])[0])
        Wbad[r, 0] = -Wbad[r, 0]
        Cw, _ = oracle.lcma(A64, B64, oracle.Desc(d.ms, d.ks, d.ns, d.U, d.V, Wbad), 1, round_operands=ops)
        assert metrics.elementwise(emulate(dtype, Cw), C_sh, bound)[1] > 1000, (dtype, lv)
        # the classic bound is the wrong yardstick for a scheme: its operand
        # roundings exceed it
        ref = oracle.gemm(A64, B64)
        cb = metrics.bound_classic(ref, oracle.gemm(np.abs(A64), np.abs(B64)), K, dtype)
        assert metrics.elementwise(C, ref, cb)[1] > 0


def test_banded_freivalds_sees_one_zeroed_tile_among_16384_columns():
    # outputs distributed like the 16384^3 workload's (shape of C, not its K)
    M, N, K = 512, 16384, 64
    A, B = si.gen(M, N, K, "bf16", "normal_sqrtk", 7)
    A64, B64 = si.f64(A), si.f64(B)
    ref = oracle.gemm(A64, B64)
    u = metrics.UNIT_ROUNDOFF["bf16"]
    C = emulate("bf16", ref)
    rows, cols = metrics.freivalds_bands(C, A64, B64)
    assert rows.max() <= 2 * u and cols.max() <= 2 * u
    Cz = C.copy()
    Cz[200:216, 9000:9016] = 0.0
    rows, cols = metrics.freivalds_bands(Cz, A64, B64)
    assert rows.max() > 2 * u
    # the whole-matrix Freivalds residual does not see it
    assert metrics.freivalds(Cz, A64, B64) <= 4 * u


def test_banded_freivalds_of_winograd_and_a_zeroed_tile_among_16384_columns():
    # Winograd's variant (bfloat16 operands) carries more error than
    # Strassen's, most in C21 and C22: its 128-row and -column bands stay
    # within 3 u_out, and a zeroed 16 x 16 tile in C22 still exceeds 3 u_out
    M, N, K = 512, 16384, 256
    A, B = si.gen(M, N, K, "bf16", "normal_sqrtk", 8)
    A64, B64 = si.f64(A), si.f64(B)
    u = metrics.UNIT_ROUNDOFF["bf16"]
    d = oracle.Desc(2, 2, 2, D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W)
    Cw, _ = oracle.lcma(A64, B64, d, 1, round_operands="bf16")
    C = emulate("bf16", Cw)
    rows, cols = metrics.freivalds_bands(C, A64, B64)
    assert max(rows.max(), cols.max()) <= 3 * u, (rows.max() / u, cols.max() / u)
    Cz = C.copy()
    Cz[400:416, 12000:12016] = 0.0
    rows, cols = metrics.freivalds_bands(Cz, A64, B64)
    assert rows.max() > 3 * u and cols.max() > 3 * u, (rows.max() / u, cols.max() / u)


def test_banded_freivalds_with_64_wide_bands_among_32768_columns():
    # twice the columns halve a zeroed tile's share of a 128-row band; a
    # 64-row band restores it (about 2.8 u_out), above the 2 u_out bound
    M, N, K = 256, 32768, 64
    A, B = si.gen(M, N, K, "bf16", "normal_sqrtk", 9)
    A64, B64 = si.f64(A), si.f64(B)
    u = metrics.UNIT_ROUNDOFF["bf16"]
    C = emulate("bf16", oracle.gemm(A64, B64))
    rows, cols = metrics.freivalds_bands(C, A64, B64, band=64)
    assert rows.max() <= 2 * u and cols.max() <= 2 * u
    Cz = C.copy()
    Cz[100:116, 20000:20016] = 0.0
    rows, cols = metrics.freivalds_bands(Cz, A64, B64, band=64)
    assert rows.max() > 2 * u


@pytest.mark.parametrize("dtype,dist", [("bf16", "normal_sqrtk"), ("f16", "uniform")])
def test_banded_freivalds_levels_of_classic_and_one_level(dtype, dist):
    M = N = 2048
    K = 1024
    A, B = si.gen(M, N, K, dtype, dist, 3)
    A64, B64 = si.f64(A), si.f64(B)
    u = metrics.UNIT_ROUNDOFF[dtype]
    ref = oracle.gemm(A64, B64)
    rows, cols = metrics.freivalds_bands(emulate(dtype, ref), A64, B64)
    assert max(rows.max(), cols.max()) <= 1.0 * u
    C1, _ = oracle.lcma(A64, B64, oracle.strassen(), 1, round_operands=dtype)
    rows, cols = metrics.freivalds_bands(emulate(dtype, C1), A64, B64)
    assert max(rows.max(), cols.max()) <= 2 * u
    Cz = emulate(dtype, C1)
    Cz[1000:1016, 1500:1516] = 0.0
    rows, cols = metrics.freivalds_bands(Cz, A64, B64)
    assert rows.max() > 2 * u and cols.max() > 2 * u
