"""Pins for the CPU oracle: every function is checked against something other than
itself (exact rational brute force, library routines, closed forms, algebraic
identities, product counts), chosen so that a dropped term, a wrong sign or
index, or a transposed operand fails at least one test.
"""
from fractions import Fraction
import itertools

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from oracle import metrics
import descriptors as D


# ----------------------------------------------------------------------------- encodings

def _all_patterns():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_decode_f16_matches_numpy_for_every_pattern():
    h = _all_patterns()
    got = oracle.decode("f16", h)
    want = h.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_bf16_matches_torch_for_every_pattern():
    h = _all_patterns()
    got = oracle.decode("bf16", h)
    want = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_encode_roundtrips_every_finite_pattern(dt):
    h = _all_patterns()
    v = oracle.decode(dt, h)
    ok = ~np.isnan(v)
    assert np.array_equal(oracle.encode(dt, v[ok]), h[ok])


def test_encode_f16_matches_numpy_rounding():
    rng = np.random.default_rng(5)
    # magnitudes from deep subnormal to beyond overflow, both signs
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp2(rng.uniform(-30, 17, 20000)),
        rng.uniform(-1, 1, 5000),
    ])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.encode("f16", x), want)


def test_encode_f16_midpoints_round_to_even():
    # midpoints between consecutive binary16 values (exact in fp64)
    h = np.arange(0x0000, 0x7bff, dtype=np.uint32).astype(np.uint16)
    lo = oracle.decode("f16", h)
    hi = oracle.decode("f16", (h.astype(np.uint32) + 1).astype(np.uint16))
    mid = (lo + hi) / 2
    got = oracle.encode("f16", mid)
    even = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(got, even)
    # largest finite is 65504; 65520 is the midpoint to the next (infinite) binade
    assert oracle.encode("f16", [65504.0, 65519.99, 65520.0, -1e6]).tolist() == [0x7bff, 0x7bff, 0x7c00, 0xfc00]


def test_encode_bf16_matches_torch_from_float32():
    rng = np.random.default_rng(6)
    with np.errstate(over="ignore"):
        x32 = (rng.standard_normal(30000) * np.exp2(rng.uniform(-140, 127, 30000))).astype(np.float32)
    x32 = x32[np.isfinite(x32)]
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.encode("bf16", x32.astype(np.float64))
    assert np.array_equal(got, want)


# ----------------------------------------------------------------------------- classic product

def _exact_product(A, B):
    M, K = len(A), len(A[0])
    N = len(B[0])
    return [[sum((Fraction(A[i][k]) * Fraction(B[k][j]) for k in range(K)), Fraction(0))
             for j in range(N)] for i in range(M)]


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (1, 5, 3), (4, 1, 6), (3, 2, 5), (5, 6, 1), (6, 4, 7)])
def test_gemm_integer_exact_vs_brute_force(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = rng.integers(-9, 10, (M, K)).astype(np.float64)
    B = rng.integers(-9, 10, (K, N)).astype(np.float64)
    C = oracle.gemm(A, B)
    E = _exact_product(A.tolist(), B.tolist())
    assert C.tolist() == [[float(v) for v in row] for row in E]


def test_gemm_half_values_within_fp64_summation_bound():
    rng = np.random.default_rng(1)
    for (M, N, K) in [(3, 7, 13), (8, 3, 31), (5, 5, 64)]:
        A = rng.uniform(-1, 1, (M, K)).astype(np.float16).astype(np.float64)
        B = rng.uniform(-1, 1, (K, N)).astype(np.float16).astype(np.float64)
        C = oracle.gemm(A, B)
        E = _exact_product(A.tolist(), B.tolist())
        gamma = K * 2.0 ** -53 / (1 - K * 2.0 ** -53)
        absprod = np.abs(A) @ np.abs(B)
        for i in range(M):
            for j in range(N):
                assert abs(Fraction(C[i, j]) - E[i][j]) <= Fraction(gamma * absprod[i, j])


def test_gemm_matches_library_matmul_on_rectangular_shapes():
    rng = np.random.default_rng(2)
    for (M, N, K) in [(37, 129, 65), (200, 17, 301), (64, 64, 512)]:
        A = rng.standard_normal((M, K))
        B = rng.standard_normal((K, N))
        C = oracle.gemm(A, B)
        R = A @ B
        assert np.linalg.norm(C - R) / np.linalg.norm(R) < 1e-12


def test_gemm_special_cases():
    rng = np.random.default_rng(3)
    A = rng.uniform(-1, 1, (9, 6))
    assert np.array_equal(oracle.gemm(A, np.eye(6)), A)                 # A I = A
    assert np.array_equal(oracle.gemm(np.eye(9), A), A)                 # I A = A
    assert not oracle.gemm(A, np.zeros((6, 4))).any()                   # A 0 = 0
    x = rng.uniform(-1, 1, (9, 1))
    y = rng.uniform(-1, 1, (1, 5))
    assert np.array_equal(oracle.gemm(x, y), x * y)                     # rank one, single products
    P = np.eye(6)[[3, 0, 5, 1, 4, 2]]                                   # permutation
    assert np.array_equal(oracle.gemm(A, P), A[:, np.argmax(P, axis=0)])
    assert oracle.gemm(np.zeros((3, 0)), np.zeros((0, 4))).tolist() == [[0.0] * 4] * 3  # empty sum


def test_gemm_rows_slice_equals_full_product():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((40, 33))
    B = rng.standard_normal((33, 21))
    assert np.array_equal(oracle.gemm_rows(A, B, 7, 19), oracle.gemm(A, B)[7:19])


# ----------------------------------------------------------------------------- LCMA descriptors

def test_brent_identity_holds_for_the_builtin_schemes():
    assert oracle.brent_violations(oracle.strassen()) == 0
    assert oracle.brent_violations(oracle.strassen2()) == 0
    assert oracle.brent_violations(oracle.naive()) == 0
    assert oracle.brent_violations(oracle.naive(2, 3, 4)) == 0


def test_product_counts_are_7_and_49():
    s, s2 = oracle.strassen(), oracle.strassen2()
    assert (s.ms, s.ks, s.ns, s.rank) == (2, 2, 2, 7)
    assert (s2.ms, s2.ks, s2.ns, s2.rank) == (4, 4, 4, 49)
    assert oracle.naive().rank == 8
    assert oracle.kron(oracle.naive(), oracle.naive()).rank == 64


def test_every_single_entry_corruption_breaks_brent():
    s = oracle.strassen()
    for name in ("U", "V", "W"):
        T = getattr(s, name)
        for idx in itertools.product(range(T.shape[0]), range(T.shape[1])):
            for val in (-1, 0, 1):
                if T[idx] == val:
                    continue
                tabs = {n: getattr(s, n).copy() for n in ("U", "V", "W")}
                tabs[name][idx] = val
                bad = oracle.Desc(2, 2, 2, tabs["U"], tabs["V"], tabs["W"])
                assert oracle.brent_violations(bad) > 0, (name, idx, val)


def test_random_corruptions_of_two_level_break_brent():
    s2 = oracle.strassen2()
    rng = np.random.default_rng(7)
    for _ in range(60):
        tabs = {n: getattr(s2, n).copy() for n in ("U", "V", "W")}
        name = ("U", "V", "W")[rng.integers(3)]
        T = tabs[name]
        r, c = rng.integers(T.shape[0]), rng.integers(T.shape[1])
        T[r, c] = (int(T[r, c]) + 2 + rng.integers(2)) % 3 - 1  # always a different value in {-1, 0, 1}
        assert oracle.brent_violations(oracle.Desc(4, 4, 4, tabs["U"], tabs["V"], tabs["W"])) > 0


def test_strassen_nonzero_counts():
    s = oracle.strassen()
    # 12 nonzeros per table: 5 combined A operands, 5 combined B operands, 18 block additions
    assert [int(np.count_nonzero(getattr(s, n))) for n in ("U", "V", "W")] == [12, 12, 12]
    assert int(np.sum(np.count_nonzero(s.U, axis=1) > 1)) == 5
    assert int(np.sum(np.count_nonzero(s.V, axis=1) > 1)) == 5
    s2 = oracle.strassen2()
    assert [int(np.count_nonzero(getattr(s2, n))) for n in ("U", "V", "W")] == [144, 144, 144]


# ----------------------------------------------------------------------------- LCMA evaluator

@pytest.mark.parametrize("M,N,K", [(2, 2, 2), (6, 10, 14), (16, 8, 12), (40, 24, 32)])
def test_one_level_equals_classic_exactly_on_integers(M, N, K):
    rng = np.random.default_rng(M + N + K)
    A = rng.integers(-2, 3, (M, K)).astype(np.float64)
    B = rng.integers(-2, 3, (K, N)).astype(np.float64)
    C, n = oracle.lcma(A, B, oracle.strassen(), 1)
    assert n == 7
    assert np.array_equal(C, oracle.gemm(A, B))
    Cn, nn = oracle.lcma(A, B, oracle.naive(), 1)
    assert nn == 8 and np.array_equal(Cn, C)


@pytest.mark.parametrize("M,N,K", [(4, 4, 4), (12, 20, 28), (32, 16, 24)])
def test_two_level_recursive_and_flat_equal_classic_on_integers(M, N, K):
    rng = np.random.default_rng(M * N + K)
    A = rng.integers(-2, 3, (M, K)).astype(np.float64)
    B = rng.integers(-2, 3, (K, N)).astype(np.float64)
    ref = oracle.gemm(A, B)
    Cr, nr = oracle.lcma(A, B, oracle.strassen(), 2)
    Cf, nf = oracle.lcma(A, B, oracle.strassen2(), 1)
    assert (nr, nf) == (49, 49)
    assert np.array_equal(Cr, ref) and np.array_equal(Cf, ref)
    Cn, nn = oracle.lcma(A, B, oracle.naive(), 2)
    assert nn == 64 and np.array_equal(Cn, ref)


def test_lcma_exact_mode_on_floats_is_close_to_classic():
    rng = np.random.default_rng(8)
    A = rng.uniform(-1, 1, (64, 96))
    B = rng.uniform(-1, 1, (96, 48))
    ref = A @ B
    for d, lv in ((oracle.strassen(), 1), (oracle.strassen(), 2), (oracle.strassen2(), 1)):
        C, _ = oracle.lcma(A, B, d, lv)
        assert np.linalg.norm(C - ref) / np.linalg.norm(ref) < 1e-13


def test_lcma_rejects_uneven_split():
    A = np.ones((3, 4))
    B = np.ones((4, 4))
    with pytest.raises(ValueError):
        oracle.lcma(A, B, oracle.strassen(), 1)


def test_operand_rounding_is_identity_when_combinations_are_representable():
    rng = np.random.default_rng(9)
    A = rng.integers(-2, 3, (16, 24)).astype(np.float64)
    B = rng.integers(-2, 3, (24, 8)).astype(np.float64)
    ref = oracle.gemm(A, B)
    for dt in ("f16", "bf16"):
        C1, _ = oracle.lcma(A, B, oracle.strassen(), 1, round_operands=dt)
        C2, _ = oracle.lcma(A, B, oracle.strassen2(), 1, round_operands=dt)
        assert np.array_equal(C1, ref) and np.array_equal(C2, ref)


def test_combine_block_special_cases():
    rng = np.random.default_rng(10)
    X = rng.integers(-3, 4, (6, 8)).astype(np.float64)
    # one-hot coefficients select a block exactly
    for a, b in itertools.product(range(2), range(2)):
        coef = np.zeros(4, np.int8)
        coef[a * 2 + b] = 1
        assert np.array_equal(oracle.combine_block(X, coef, 2, 2), X[a * 3:(a + 1) * 3, b * 4:(b + 1) * 4])
    # (1, 0, 0, 1) and (-1, 0, 1, 0): sums of blocks
    assert np.array_equal(oracle.combine_block(X, [1, 0, 0, 1], 2, 2), X[:3, :4] + X[3:, 4:])
    assert np.array_equal(oracle.combine_block(X, [-1, 0, 1, 0], 2, 2), X[3:, :4] - X[:3, :4])
    # rounding: 1 + 2^-11 is a binary16 tie -> 1
    Y = np.array([[1.0, 0.0], [0.0, 2.0 ** -11]])
    assert oracle.combine_block(Y, [1, 0, 0, 1], 2, 2, round_operand="f16").tolist() == [[1.0]]
    assert oracle.combine_block(Y, [1, 0, 0, 1], 2, 2).tolist() == [[1 + 2.0 ** -11]]


# ----------------------------------------------------------------------------- metrics

def test_metrics_closed_forms():
    A = np.full((4, 8), 0.5)       # ||A||_F = sqrt(32) * 0.5 = 2*sqrt(2)
    B = np.full((8, 2), 0.25)      # ||B||_F = sqrt(16) * 0.25 = 1
    C_ref = A @ B                  # every entry 1.0; ||C_ref||_F = sqrt(8)
    C = C_ref.copy()
    C[1, 1] += 0.3
    assert metrics.e_nw(C, C_ref, A, B) == pytest.approx(0.3 / (2 * np.sqrt(2)), rel=1e-15)
    assert metrics.e_rel(C, C_ref) == pytest.approx(0.3 / np.sqrt(8), rel=1e-15)
    blocks = metrics.e_rel_blocks(C, C_ref, 2)
    # C[1, 1] lies in block (0, 1): rows 0-1, column 1, whose reference norm is sqrt(2)
    assert blocks[1] == pytest.approx(0.3 / np.sqrt(2), rel=1e-15)
    assert blocks[0] == blocks[2] == blocks[3] == 0.0


def test_freivalds_detects_one_wrong_entry():
    rng = np.random.default_rng(11)
    A = rng.standard_normal((50, 40))
    B = rng.standard_normal((40, 30))
    C = oracle.gemm(A, B)
    assert metrics.freivalds(C, A, B) < 1e-13
    C[17, 3] += 1.0
    assert metrics.freivalds(C, A, B) > 1e-3


def test_winograd_variant_evaluates_exactly_and_differs_from_strassen():
    # a second rank-7 description: Brent-valid, 7 block products, exact on
    # integers at one and two levels, and not the same table as Strassen's
    d = oracle.Desc(2, 2, 2, D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W)
    assert oracle.brent_violations(d) == 0
    s = oracle.strassen()
    assert not (np.array_equal(d.U, s.U) and np.array_equal(d.V, s.V) and np.array_equal(d.W, s.W))
    rng = np.random.default_rng(4)
    A = rng.integers(-3, 4, (12, 20)).astype(np.float64)
    B = rng.integers(-3, 4, (20, 8)).astype(np.float64)
    C, n = oracle.lcma(A, B, d, 1)
    assert n == 7 and np.array_equal(C, A @ B)
    A = rng.integers(-2, 3, (16, 16)).astype(np.float64)
    B = rng.integers(-2, 3, (16, 16)).astype(np.float64)
    C, n = oracle.lcma(A, B, d, 2)
    assert n == 49 and np.array_equal(C, A @ B)


@pytest.mark.parametrize("dtype,dist,levels,ops,lo,hi", [
    ("f16", "uniform", 1, "f16", 2.5, 3.2),
    ("bf16", "normal_sqrtk", 1, "bf16", 2.5, 3.2),
    ("f16", "uniform", 2, "f16", 5.3, 6.5),             # beyond the 4x gate: opt-in only
    ("bf16", "normal_sqrtk", 2, "bf16", 5.3, 6.5),      # beyond the 4x gate: opt-in only
    ("bf16", "normal_sqrtk", 2, "f16", 0.9, 1.4),       # the default for two levels of bfloat16
])
def test_two_level_error_ratios_from_the_scheme_evaluation(dtype, dist, levels, ops, lo, hi):
    # The error of a scheme evaluated with combined operands rounded to `ops`
    # (then the result rounded once to the output type), over the error of the
    # exact product rounded once: the basis of the library's accuracy gate
    # (at most 4x, else an explicit opt-in).  Casts are the error source the
    # FalconGEMM write-up names (section "从缓存重排到 Cost Model").
    A, B = si.gen(512, 768, 640, dtype, dist, 4)
    A64, B64 = si.f64(A), si.f64(B)
    ref = oracle.gemm(A64, B64)
    e_c = metrics.e_nw(oracle.round_to(dtype, ref), ref, A64, B64)
    d = oracle.strassen() if levels == 1 else oracle.strassen2()
    C, n = oracle.lcma(A64, B64, d, 1, round_operands=ops)
    assert n == d.rank
    e = metrics.e_nw(oracle.round_to(dtype, C), ref, A64, B64)
    assert lo <= e / e_c <= hi, e / e_c
