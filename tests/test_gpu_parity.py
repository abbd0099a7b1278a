"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Every float result passes
  - the normwise gates e_nw = ||C - C_ref||_F / (||A||_F ||B||_F) <= 1e-3
    (binary16), <= 8e-3 (bfloat16), and e_rel = ||C - C_ref||_F / ||C_ref||_F
    <= 4 u_out over the whole matrix and per output block (e_nw alone shrinks
    like 1/sqrt(K));
  - an element-by-element bound: for the classic kernels
    u_out |C_ref| + (1 + u_out) 2K u_32 (|A||B|) (fp32 accumulation, one
    rounding); for an LCMA form, the rounding bound around the oracle's
    evaluation of the same scheme with the same operand rounding;
  - for LCMA forms, e_nw at most 4x the classic kernel's on the same inputs
    (7x for the two-level forms that need an accuracy opt-in).
Integer-valued inputs must match bit for bit.  Where the oracle cannot form
the whole product (16384^3) one row per 256-row band is compared and every
128-row and 128-column band is checked by a Freivalds residual.
"""
import numpy as np
import pytest
import torch

import complexity_half_precision_amd as L
import oracle
import seeded_inputs as si
import descriptors as D
from oracle import metrics

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)


def gen(M, N, K, dtype, dist, seed=0):
    A, B = si.gen(M, N, K, dtype, dist, seed)
    return A, B, si.f64(A), si.f64(B)


def classic(A, B):
    M, K = A.shape
    N = B.shape[1]
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty((M, N), dtype=A.dtype, device=DEV)
    L.gemm_classic(Ad, Bd, C)
    torch.cuda.synchronize()
    return C.cpu()


def planned(A, B, algo, **kw):
    M, K = A.shape
    N = B.shape[1]
    plan = L.lcma_plan_ex(M, N, K, A.dtype, force=algo, **kw)
    assert L.lcma_plan_info(plan)[0] == algo
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty((M, N), dtype=A.dtype, device=DEV)
    ws = L.workspace_for(plan)
    L.lcma_gemm(plan, Ad, Bd, C, ws)
    torch.cuda.synchronize()
    return C.cpu()


RATIO = 4.0          # an LCMA result may carry at most 4x the classic kernel's error on the same inputs
RATIO_OPTIN = 7.0    # opted-in two-level forms: 5.8-5.9x on the oracle's evaluation of the scheme


def abs_product(A64, B64):
    return oracle.gemm(np.abs(A64), np.abs(B64))


def check_float(C, A64, B64, dtype, C_ref=None, blocks=1, absAB=None):
    """A classic result: normwise gates, and every element within its bound
    u_out |C_ref| + gamma_K (|A||B|) (fp32 accumulation, one rounding)."""
    C_ref = oracle.gemm(A64, B64) if C_ref is None else C_ref
    c = si.f64(C)
    assert np.all(np.isfinite(c))
    e = metrics.e_nw(c, C_ref, A64, B64)
    assert e <= metrics.GATE_NW[dtype], e
    u = metrics.UNIT_ROUNDOFF[dtype]
    assert metrics.e_rel(c, C_ref) <= 4 * u
    if blocks > 1:
        assert max(metrics.e_rel_blocks(c, C_ref, blocks)) <= 4 * u
    absAB = abs_product(A64, B64) if absAB is None else absAB
    worst, bad = metrics.elementwise(c, C_ref, metrics.bound_classic(C_ref, absAB, A64.shape[1], dtype))
    assert bad == 0, f"{bad} elements beyond the classic bound (worst {worst:.2f}x)"
    return e


def op_type(dtype, algo, bf16_ops_f16=0, combine="auto"):
    """Type the plan rounds combined operands to (mirrors the planner's rule)."""
    if dtype == "f16":
        return "f16"
    if combine == "at_load" or bf16_ops_f16 == -1:
        return "bf16"
    if bf16_ops_f16 == 1:
        return "f16"
    return "f16" if algo == "l2" else "bf16"


def _splits(M, N, K, S):
    if M % S or N % S or K % S:
        return False
    Nb, Kb = N // S, K // S
    return M >= S and Nb >= 8 and Kb >= 8 and Nb % 8 == 0 and Kb % 8 == 0


def scheme_reference(A64, B64, d, ops, builtin=True):
    """(C_sh, magnitude, block depth) of the oracle's evaluation of scheme d with
    operands rounded to ops; on the zero-padded shape (multiples of 16 S) when
    a forced built-in level pads, cropped back."""
    M, K = A64.shape
    N = B64.shape[1]
    S = d.ms
    if builtin and not _splits(M, N, K, S):
        g = 16 * S
        up = lambda x: -(-x // g) * g
        Ap = np.zeros((up(M), up(K)))
        Bp = np.zeros((up(K), up(N)))
        Ap[:M, :K] = A64
        Bp[:K, :N] = B64
    else:
        Ap, Bp = A64, B64
    C_sh, n = oracle.lcma(Ap, Bp, d, 1, round_operands=ops)
    assert n == d.rank
    mag, _ = oracle.lcma(np.abs(Ap), np.abs(Bp), oracle.magnitude(d), 1)
    return C_sh[:M, :N], mag[:M, :N], Ap.shape[1] // d.ks


def check_scheme(C, A64, B64, dtype, algo, e_classic, C_ref=None, ops=None, desc=None, blocks=None,
                 ratio=RATIO, unfused=False):
    """An LCMA result: normwise gates against the exact product, its error at
    most `ratio` times the classic GPU error on the same inputs, and every
    element within the rounding bound of the oracle's evaluation of the same
    scheme with the same operand rounding.  Returns e_nw."""
    d = desc if desc is not None else (oracle.strassen() if algo == "l1" else oracle.strassen2())
    ops = ops or op_type(dtype, algo)
    C_ref = oracle.gemm(A64, B64) if C_ref is None else C_ref
    c = si.f64(C)
    assert np.all(np.isfinite(c))
    e = metrics.e_nw(c, C_ref, A64, B64)
    assert e <= metrics.GATE_NW[dtype], e
    # relative gates: 4 u_out for the 4x forms, scaled with the band of opted-in forms
    rel_gate = 4 * metrics.UNIT_ROUNDOFF[dtype] * max(1.0, ratio / RATIO)
    assert metrics.e_rel(c, C_ref) <= rel_gate
    bs = blocks if blocks is not None else d.ms
    if bs > 1 and min(c.shape) >= bs:
        assert max(metrics.e_rel_blocks(c, C_ref, bs)) <= rel_gate
    assert e <= ratio * e_classic if e_classic > 0 else e == 0, (e, e_classic, ratio)
    C_sh, mag, depth = scheme_reference(A64, B64, d, ops, builtin=desc is None)
    folds = int((d.W != 0).sum(axis=0).max()) + 2          # products per output, plus a split fix-up add
    bound = metrics.bound_lcma(C_sh, mag, depth * (2 if unfused else 1), folds, dtype, ops)
    worst, bad = metrics.elementwise(c, C_sh, bound)
    assert bad == 0, f"{bad} elements beyond the scheme's bound (worst {worst:.2f}x)"
    return e


def classic_error(A, B, A64, B64, dtype, C_ref):
    return check_float(classic(A, B), A64, B64, dtype, C_ref)


def check_exact(C, A64, B64, dtype):
    want = oracle.encode(dtype, oracle.gemm(A64, B64))
    got = si.bits(C)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"


# ---------------------------------------------------------------- classic

CLASSIC_SHAPES = [
    (1, 8, 8), (7, 13, 5), (3, 1, 9), (33, 40, 24), (64, 64, 64), (65, 72, 136),
    (100, 200, 304), (257, 136, 72), (300, 520, 1000), (513, 264, 520),
    (4100, 4104, 72),          # 256 x 256 tiles with ragged tails in M and N
    (1000, 1064, 256),         # 128 x 128 four-wave tiles (short K): interior (grouped loads) and edge tiles
    (640, 384, 4096),          # 128 x 128 tiles, long K (eight-wave kernel): all interior
    (1000, 1064, 2056),        # 128 x 128 tiles, long K (eight-wave kernel): edge tiles, K tail
    (1000, 1064, 2040),        # 128 x 128 tiles just below the long-K switch (four-wave kernel)
    (17, 1000, 520),           # streaming kernel (32-row A), N and K tails
    (60, 2056, 1000),          # streaming kernel (64-row A, 64-k stages), N and K tails
    (33, 4104, 4104),          # 64-k stages: an odd stage count per wave and a k tail of 8
    (20, 1032, 1032),          # up to 32 rows, long K: 64-k stages on two waves, k tail of 8
    (64, 136, 72),             # one stage per wave at most, ragged N
    (17, 8264, 1032),          # up to 32 rows, more than 128 column strips: the shared ring, all tails ragged
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", CLASSIC_SHAPES)
def test_classic_matches_oracle(M, N, K, dtype):
    say("classic", M, N, K, dtype)
    A, B, A64, B64 = gen(M, N, K, dtype, "uniform", seed=M + N + K)
    check_float(classic(A, B), A64, B64, dtype)


@pytest.mark.parametrize("dtype,dist", [("f16", "int2"), ("bf16", "int1")])
@pytest.mark.parametrize("M,N,K", [(33, 40, 24), (130, 200, 96), (257, 136, 120), (512, 512, 256), (4100, 264, 64),
                                   (1000, 1064, 256), (4096, 4104, 96), (48, 1000, 200), (64, 14336, 256),
                                   (40, 1032, 248)])
def test_classic_integer_inputs_are_exact(M, N, K, dtype, dist):
    say("classic exact", M, N, K, dtype)
    A, B, A64, B64 = gen(M, N, K, dtype, dist, seed=7)
    check_exact(classic(A, B), A64, B64, dtype)


def test_classic_strided_operands_and_output():
    say("classic strided")
    M, N, K = 200, 136, 72
    Abig, Bbig, _, _ = gen(M, N + 24, K + 40, "f16", "uniform", seed=3)
    A = Abig[:, :K]                     # lda = K + 40
    B = Bbig[:K, :N]                    # ldb = N + 24
    A64, B64 = si.f64(A), si.f64(B)
    Ad, Bd = Abig.to(DEV)[:, :K], Bbig.to(DEV)[:K, :N]
    Cbig = torch.full((M, N + 16), 7.0, dtype=torch.float16, device=DEV)
    C = Cbig[:, :N]
    L.gemm_classic(Ad, Bd, C)
    torch.cuda.synchronize()
    check_float(C.cpu(), A64, B64, "f16")
    assert torch.all(Cbig[:, N:].cpu() == 7.0)     # nothing written outside C


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 256), (1024, 768, 512), (40, 1032, 520)])
def test_classic_strided_aligned_paths(M, N, K):
    # leading dimensions larger than the extents (multiples of 8 elements, so
    # the direct-to-LDS kernels run): 256 x 256 and 128 x 128 four-wave tiles
    # and the streaming kernel
    say("classic strided aligned", M, N, K)
    Abig, Bbig, _, _ = gen(M, N + 24, K + 40, "bf16", "normal_sqrtk", seed=21)
    A, B = Abig[:, :K], Bbig[:K, :N]
    A64, B64 = si.f64(A), si.f64(B)
    Ad, Bd = Abig.to(DEV)[:, :K], Bbig.to(DEV)[:K, :N]
    Cbig = torch.full((M, N + 16), 7.0, dtype=torch.bfloat16, device=DEV)
    C = Cbig[:, :N]
    L.gemm_classic(Ad, Bd, C)
    torch.cuda.synchronize()
    check_float(C.cpu(), A64, B64, "bf16")
    assert torch.all(Cbig[:, N:].cpu() == 7.0)


def test_classic_unaligned_pointers():
    say("classic unaligned")
    M, N, K = 96, 80, 64
    A, B, A64, B64 = gen(M, N, K, "bf16", "uniform", seed=4)
    flatA = torch.zeros(M * K + 1, dtype=torch.bfloat16, device=DEV)
    flatA[1:] = A.reshape(-1).to(DEV)
    Ad = flatA[1:].view(M, K)            # 2-byte offset: element-wise load path
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    L.gemm_classic(Ad, B.to(DEV), C)
    torch.cuda.synchronize()
    check_float(C.cpu(), A64, B64, "bf16")


def test_classic_empty_and_zero_k():
    say("classic empty")
    A = torch.empty((0, 16), dtype=torch.float16, device=DEV)
    B = torch.ones((16, 8), dtype=torch.float16, device=DEV)
    C = torch.empty((0, 8), dtype=torch.float16, device=DEV)
    L.gemm_classic(A, B, C)
    A = torch.ones((5, 0), dtype=torch.float16, device=DEV)
    B = torch.ones((0, 24), dtype=torch.float16, device=DEV)
    C = torch.full((5, 24), 3.0, dtype=torch.float16, device=DEV)
    L.gemm_classic(A, B, C, K=0)
    torch.cuda.synchronize()
    assert torch.all(C.cpu() == 0)


def test_classic_is_deterministic():
    say("classic determinism")
    A, B, _, _ = gen(1024, 1024, 1024, "bf16", "normal_sqrtk", seed=5)
    r = [si.bits(classic(A, B)) for _ in range(3)]
    assert np.array_equal(r[0], r[1]) and np.array_equal(r[0], r[2])


@pytest.mark.parametrize("M,N,K,dist", [
    (4096, 4096, 512, "int2"),      # 256 x 256 tiles, interior grouped loads, 16 k-tiles: the steady-state loop
    (1024, 1024, 2048, "int1"),     # 128 x 128 eight-wave kernel for long K (7 k-tiles in flight), interior
    (1000, 1064, 2048, "int1"),     # the same with edge tiles
    (24, 8200, 1024, "int1"),       # streaming kernel with a ring shared by its waves (more than 128 strips)
])
def test_classic_integer_inputs_exact_through_the_full_size_loops(M, N, K, dist):
    # |C| <= 2048 (2 * 2 * 512, or 2048 * 1): every partial sum and the result
    # are exact binary16 integers, so any order gives the exact product
    say("classic exact full loops", M, N, K)
    A, B, A64, B64 = gen(M, N, K, "f16", dist, seed=8)
    check_exact(classic(A, B), A64, B64, "f16")


# ---------------------------------------------------------------- one level

def test_l1_square_512_f16_matches_oracle_and_ratio():
    say("l1 512 f16")
    A, B, A64, B64 = gen(**si.SQUARE_512_F16)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "f16", C_ref)
    check_scheme(planned(A, B, "l1"), A64, B64, "f16", "l1", e_c, C_ref)


@pytest.mark.parametrize("algo,combine", [("l1", "auto"), ("l2", "auto"), ("l2", "l2_on_chip")])
def test_lcma_integer_inputs_are_exact(algo, combine):
    say("exact", algo, combine)
    A, B, A64, B64 = gen(**si.SQUARE_512_F16_INT)
    # integer inputs carry no rounding error, so the accuracy opt-in of
    # binary16 two levels costs nothing here
    check_exact(planned(A, B, algo, combine=combine, accuracy_optin=1), A64, B64, "f16")
    A, B, A64, B64 = gen(256, 512, 384, "bf16", "int1", seed=2)
    check_exact(planned(A, B, algo, combine=combine), A64, B64, "bf16")


@pytest.mark.parametrize("ops", [-1, 1])
def test_l1_bf16_operand_modes(ops):
    say("l1 bf16 ops", ops)
    A, B, A64, B64 = gen(1024, 1024, 1024, "bf16", "normal_sqrtk", seed=9)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "bf16", C_ref)
    check_scheme(planned(A, B, "l1", bf16_ops_f16=ops), A64, B64, "bf16", "l1", e_c, C_ref,
                 ops=op_type("bf16", "l1", ops))


def test_prepass_operands_are_rne_of_the_exact_combination():
    say("prepass bits")
    M = N = K = 512
    for dtype, dist in (("f16", "uniform"), ("bf16", "normal_sqrtk")):
        A, B, A64, B64 = gen(M, N, K, dtype, dist, seed=11)
        plan = L.lcma_plan_ex(M, N, K, dtype, force="l1")
        ws = L.workspace_for(plan)
        L.lcma_prepass(plan, A.to(DEV), B.to(DEV), ws)
        torch.cuda.synchronize()
        wsh = ws.cpu()
        d = oracle.strassen()
        for side, X, T in ((0, A64, d.U), (1, B64, d.V)):
            for r in range(7):
                off, ld, odt = L.lcma_plan_operand(plan, side, r)
                if off < 0:
                    continue
                odt = "f16" if odt == L.F16 else "bf16"
                rows, cols = (M // 2, K // 2) if side == 0 else (K // 2, N // 2)
                got = wsh[off:off + rows * cols * 2].view(torch.int16).numpy().view(np.uint16).reshape(rows, cols)
                exact = oracle.combine_block(X, T[r], 2, 2)
                want = oracle.encode(odt, exact)
                # the kernel sums in fp32: where that sum is exact the result must be bitwise equal
                fp32_exact = np.float32(exact).astype(np.float64) == exact
                assert np.array_equal(got[fp32_exact], want[fp32_exact]), (side, r)
                assert fp32_exact.mean() > 0.99


def _unpack_a(x, rows, cols):
    """Row-major view of a tile-packed A operand (the layout lcma_plan_operand
    states for ld 0): block (tr, t) of 256 rows x 32 columns at element
    (tr * cols + 32 t) * 256, chunk c of block row rr at position c ^ ((rr >> 1) & 3)."""
    t = x.reshape(rows // 256, cols // 32, 256, 4, 8)
    rr = np.arange(256)[:, None]
    pos = np.arange(4)[None, :]
    out = np.empty_like(t)
    out[:, :, rr, pos ^ ((rr >> 1) & 3), :] = t[:, :, rr, pos, :]
    return out.transpose(0, 2, 1, 3, 4).reshape(rows, cols)


def test_unfused_prepass_writes_tile_packed_a_operands():
    # blocks of 4096 x 4096 on whole 256 x 256 tiles: the A operands are
    # tile-packed (ld 0), the B operands row-major with rows padded by 64
    # elements; both are the RNE of the exact combination, bit for bit where
    # the fp32 sum is exact
    say("unfused packed operands")
    M, N, K = 8192, 8192, 512
    A, B, A64, B64 = gen(M, N, K, "bf16", "normal_sqrtk", seed=12)
    plan = L.lcma_plan_ex(M, N, K, "bf16", force="l1", combine="unfused")
    ws = L.workspace_for(plan)
    L.lcma_prepass(plan, A.to(DEV), B.to(DEV), ws)
    torch.cuda.synchronize()
    d = oracle.strassen()
    for side, X, T in ((0, A64, d.U), (1, B64, d.V)):
        rows, cols = (M // 2, K // 2) if side == 0 else (K // 2, N // 2)
        for r in range(7):
            off, ld, odt = L.lcma_plan_operand(plan, side, r)
            assert off >= 0 and ld == (0 if side == 0 else cols + 64)
            odt = "f16" if odt == L.F16 else "bf16"
            if side == 0:
                got = ws[off:off + rows * cols * 2].cpu().view(torch.int16).numpy().view(np.uint16)
                got = _unpack_a(got, rows, cols)
            else:
                raw = ws[off:off + ((rows - 1) * ld + cols) * 2].cpu().view(torch.int16).numpy().view(np.uint16)
                got = np.lib.stride_tricks.as_strided(raw, (rows, cols), (ld * 2, 2))
            exact = oracle.combine_block(X, T[r], 2, 2)
            want = oracle.encode(odt, exact)
            fp32_exact = np.float32(exact).astype(np.float64) == exact
            assert np.array_equal(got[fp32_exact], want[fp32_exact]), (side, r)
            assert fp32_exact.mean() > 0.99


@pytest.mark.parametrize("M,N,K,dtype", [(400, 272, 144, "f16"), (600, 528, 512, "bf16")])
def test_l1_ragged_group_tiles(M, N, K, dtype):
    # quadrants that do not fill whole 128 x 128 group tiles (and a k tail in
    # the first shape): the fused kernel's bounded loads and edge stores
    say("l1 ragged", M, N, K, dtype)
    dist = "uniform" if dtype == "f16" else "normal_sqrtk"
    A, B, A64, B64 = gen(M, N, K, dtype, dist, seed=17)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, dtype, C_ref)
    check_scheme(planned(A, B, "l1"), A64, B64, dtype, "l1", e_c, C_ref)
    idist = "int2" if dtype == "f16" else "int1"
    A, B, A64, B64 = gen(M, N, min(K, 256), dtype, idist, seed=18)
    check_exact(planned(A, B, "l1"), A64, B64, dtype)


@pytest.mark.parametrize("split", ["none", "all"])
def test_l1_split_modes_reproducible(split):
    say("l1 split", split)
    A, B, A64, B64 = gen(1024, 768, 512, "f16", "uniform", seed=13)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "f16", C_ref)
    runs = [planned(A, B, "l1", split=split) for _ in range(3)]
    check_scheme(runs[0], A64, B64, "f16", "l1", e_c, C_ref)
    b = [si.bits(c) for c in runs]
    assert np.array_equal(b[0], b[1]) and np.array_equal(b[0], b[2])


@pytest.mark.parametrize("n", [2560, 6144])
def test_l1_tail_split_shapes(n):
    # 2560: 100 groups on 256 CUs (every group split); 6144: 576 groups (64-group split tail)
    say("l1 tail", n)
    A, B, A64, B64 = gen(n, n, 512, "bf16", "normal_sqrtk", seed=n)
    plan = L.lcma_plan_ex(n, n, 512, "bf16", force="l1")
    items, _ = L.lcma_plan_schedule(plan)
    assert any(it[4] >= 0 for it in items)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "bf16", C_ref)
    check_scheme(planned(A, B, "l1"), A64, B64, "bf16", "l1", e_c, C_ref)


@pytest.mark.parametrize("M,N,split", [(2560, 2560, "auto"), (4096, 5120, "none"), (4096, 5120, "all"),
                                       (4096, 5120, "auto")])
def test_l1_plain_order_equals_locality_order(M, N, split):
    # The order moves groups and split pieces between compute units.  When the
    # same groups are split under both orders (none, all; 2560^2 splits all
    # 100 groups) each group's arithmetic (product order, split point,
    # commutative fix-up add) is the same, so the results are bitwise equal.
    # With a partial tail (4096 x 5120: 64 of 320 groups) the two orders put
    # different output tiles in the tail, whose split sums associate
    # differently: then both must meet the oracle's gates.
    say("l1 order", M, N, split)
    A, B, A64, B64 = gen(M, N, 256, "bf16", "normal_sqrtk", seed=M + N)
    C0 = planned(A, B, "l1", split=split)
    C1 = planned(A, B, "l1", split=split, order="plain")
    tail = split == "auto" and (M // 256) * (N // 256) % 256 != 0
    if not tail:
        assert np.array_equal(si.bits(C0), si.bits(C1))
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "bf16", C_ref)
    for C in (C0, C1) if tail else (C1,):
        check_scheme(C, A64, B64, "bf16", "l1", e_c, C_ref)


# ---------------------------------------------------------------- padded shapes

@pytest.mark.parametrize("algo,M,N,K,dtype,dist", [
    ("l1", 511, 520, 500, "f16", "int2"),            # integer inputs: exact
    ("l2", 300, 200, 250, "f16", "int2"),
    ("l1", 1000, 1032, 520, "bf16", "normal_sqrtk"),
    ("l2", 1000, 1032, 520, "bf16", "normal_sqrtk"),
    ("l1", 1, 4096, 4096, "bf16", "normal_sqrtk"),   # one row, padded to 32
])
def test_padded_lcma_matches_oracle(algo, M, N, K, dtype, dist):
    # a forced level on a shape that does not split evenly runs on zero-padded
    # copies of A and B and crops the padded product into C
    say("padded", algo, M, N, K, dtype)
    A, B, A64, B64 = gen(M, N, K, dtype, dist, seed=M + 2 * N + 3 * K)
    C = planned(A, B, algo, accuracy_optin=int(dist.startswith("int")))
    if dist.startswith("int"):
        check_exact(C, A64, B64, dtype)
    else:
        C_ref = oracle.gemm(A64, B64)
        e_c = classic_error(A, B, A64, B64, dtype, C_ref)
        check_scheme(C, A64, B64, dtype, algo, e_c, C_ref)


@pytest.mark.parametrize("M,N,K,dtype", [(64, 4096, 14336, "bf16"), (33, 8200, 10248, "f16"), (48, 1032, 8192, "bf16"),
                                       (57, 136, 8200, "f16"), (1, 1024, 14336, "bf16"), (1, 1032, 12296, "f16"),
                                       (13, 4104, 8200, "bf16"), (32, 136, 8200, "f16"), (8, 8064, 14336, "bf16"),
                                       (29, 1000, 12344, "bf16"), (40, 2056, 4104, "f16"), (3, 3976, 6152, "bf16"),
                                       (48, 28680, 4104, "bf16"), (20, 14336, 12296, "f16"), (3, 1030, 14330, "f16"),
                                       (50, 2050, 6150, "bf16")])
def test_decode_k_split_matches_oracle(M, N, K, dtype):
    # classic plans of up to 64 rows with long K: 2, 4 or 8 workgroups per
    # 128-column strip, one part of K each, partials through the workspace
    # and a second kernel that adds them (32- and 64-row tiles; ragged rows,
    # columns and k; one strip and many; K and N not multiples of 8, where
    # the plan pads into its workspace and splits the padded product)
    say("decode K split", M, N, K, dtype)
    A, B, A64, B64 = gen(M, N, K, dtype, "uniform" if dtype == "f16" else "normal_sqrtk", seed=61)
    plan = L.lcma_plan_ex(M, N, K, dtype, force="classic")
    assert L.lcma_plan_info(plan)[1] > 0
    check_float(planned(A, B, "classic"), A64, B64, dtype)


@pytest.mark.parametrize("M,N,K", [(64, 4104, 8200), (24, 1032, 14344), (5, 1024, 14336)])
def test_decode_k_split_integer_inputs_are_exact(M, N, K):
    # {-1, 0, 1} inputs: every partial sum is an exact fp32 integer, and the
    # products stay within binary16's exact integers (checked below)
    say("decode K split exact", M, N, K)
    A, B, A64, B64 = gen(M, N, K, "f16", "int1", seed=62)
    assert np.abs(oracle.gemm(A64, B64)).max() <= 2048
    check_exact(planned(A, B, "classic"), A64, B64, "f16")


@pytest.mark.parametrize("M,N,K", [(64, 2056, 8192), (16, 1024, 14336), (2048, 512, 8192)])
def test_decode_k_split_any_workspace_contents_and_repeated_calls(M, N, K):
    # the split needs no cleared workspace: random initial bytes, then calls
    # with other inputs on the same workspace, then the first inputs again
    # (bit for bit the first result)
    say("decode K split workspace reuse", M, N, K)
    plan = L.lcma_plan_ex(M, N, K, "bf16", force="classic")
    ws = L.workspace_for(plan)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device=DEV))
    outs = []
    for seed in (71, 72, 71):
        A, B, A64, B64 = gen(M, N, K, "bf16", "normal_sqrtk", seed=seed)
        C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        L.lcma_gemm(plan, A.to(DEV), B.to(DEV), C, ws)
        torch.cuda.synchronize()
        check_float(C.cpu(), A64, B64, "bf16")
        outs.append(si.bits(C.cpu()))
    assert np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("M,N,K,dtype", [(4096, 256, 8192, "bf16"), (256, 8192, 4096, "f16"), (1000, 264, 8200, "bf16"),
                                       (300, 136, 16392, "f16"), (128, 14336, 4096, "bf16"), (65, 128, 4104, "bf16")])
def test_classic_k_split_matches_oracle(M, N, K, dtype):
    # classic plans beyond 64 rows with few 128 x 128 tiles and long K: S
    # pieces of K per tile write fp32 planes, a second kernel adds them in
    # piece order (ragged rows, columns and k; S = 2, 4, 8)
    say("classic K split", M, N, K, dtype)
    A, B, A64, B64 = gen(M, N, K, dtype, "uniform" if dtype == "f16" else "normal_sqrtk", seed=63)
    plan = L.lcma_plan_ex(M, N, K, dtype, force="classic")
    assert L.lcma_plan_info(plan)[1] > 0
    check_float(planned(A, B, "classic"), A64, B64, dtype)


def test_classic_tail_round_k_split_matches_oracle():
    # 17 x 17 tiles of 256 on 256 compute units: one full round, then 33
    # tail tiles split into 4 pieces of K (ragged edge tiles and k)
    say("classic tail split")
    M = N = K = 4104
    A, B, A64, B64 = gen(M, N, K, "bf16", "normal_sqrtk", seed=65)
    plan = L.lcma_plan_ex(M, N, K, "bf16", force="classic")
    assert L.lcma_plan_info(plan)[1] > 0
    check_float(planned(A, B, "classic"), A64, B64, "bf16")


def test_classic_tail_round_k_split_integer_inputs_are_exact():
    say("classic tail split exact")
    A, B, A64, B64 = gen(2304, 7424, 4096, "f16", "int1", seed=66)
    assert L.lcma_plan_info(L.lcma_plan_ex(2304, 7424, 4096, "f16", force="classic"))[1] > 0
    assert np.abs(oracle.gemm(A64, B64)).max() <= 2048
    check_exact(planned(A, B, "classic"), A64, B64, "f16")


def test_classic_k_split_integer_inputs_are_exact():
    say("classic K split exact")
    A, B, A64, B64 = gen(2048, 512, 8192, "f16", "int1", seed=64)
    assert np.abs(oracle.gemm(A64, B64)).max() <= 2048
    check_exact(planned(A, B, "classic"), A64, B64, "f16")


@pytest.mark.parametrize("M,N,K,ldc_pad", [(1024, 1024, 8192, 3), (4096, 256, 8192, 16)])
def test_classic_k_split_strided_operands_and_output(M, N, K, ldc_pad):
    say("classic K split strided", M, N, K, ldc_pad)
    Abig, Bbig, _, _ = gen(M, N + 24, K + 40, "bf16", "normal_sqrtk", seed=91)
    A, B = Abig[:, :K], Bbig[:K, :N]
    A64, B64 = si.f64(A), si.f64(B)
    Ad, Bd = Abig.to(DEV)[:, :K], Bbig.to(DEV)[:K, :N]
    plan = L.lcma_plan_ex(M, N, K, "bf16", force="classic")
    assert L.lcma_plan_info(plan)[1] > 0
    Cbig = torch.full((M, N + ldc_pad), 7.0, dtype=torch.bfloat16, device=DEV)
    C = Cbig[:, :N]
    L.lcma_gemm(plan, Ad, Bd, C, L.workspace_for(plan))
    torch.cuda.synchronize()
    check_float(C.cpu(), A64, B64, "bf16")
    assert torch.all(Cbig[:, N:].cpu() == 7.0)


@pytest.mark.parametrize("M,N,K", [(8, 1024, 8192), (256, 512, 8192)])
def test_k_split_plans_run_unsplit_on_unaligned_operands(M, N, K):
    # a plan with a K-split workspace, called with A 2 bytes off 16-byte
    # alignment: the element-load kernels run instead (same result bound)
    say("K split plan, unaligned A", M, N, K)
    A, B, A64, B64 = gen(M, N, K, "bf16", "normal_sqrtk", seed=92)
    plan = L.lcma_plan_ex(M, N, K, "bf16", force="classic")
    assert L.lcma_plan_info(plan)[1] > 0
    flat = torch.zeros(M * K + 1, dtype=torch.bfloat16, device=DEV)
    flat[1:] = A.reshape(-1).to(DEV)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    L.lcma_gemm(plan, flat[1:].view(M, K), B.to(DEV), C, L.workspace_for(plan))
    torch.cuda.synchronize()
    check_float(C.cpu(), A64, B64, "bf16")


@pytest.mark.parametrize("M,N,K,ldc_pad", [(5, 1032, 8192, 3), (40, 2056, 4104, 16)])
def test_decode_k_split_strided_operands_and_output(M, N, K, ldc_pad):
    # leading dimensions beyond the extents (lda, ldb multiples of 8, so the
    # split runs); ldc = N + 3 takes the reduction's 2-byte C stores, N + 16
    # its 8-byte stores; nothing outside C is written
    say("decode K split strided", M, N, K, ldc_pad)
    Abig, Bbig, _, _ = gen(M, N + 24, K + 40, "bf16", "normal_sqrtk", seed=90)
    A, B = Abig[:, :K], Bbig[:K, :N]
    A64, B64 = si.f64(A), si.f64(B)
    Ad, Bd = Abig.to(DEV)[:, :K], Bbig.to(DEV)[:K, :N]
    plan = L.lcma_plan_ex(M, N, K, "bf16", force="classic")
    assert L.lcma_plan_info(plan)[1] > 0
    Cbig = torch.full((M, N + ldc_pad), 7.0, dtype=torch.bfloat16, device=DEV)
    C = Cbig[:, :N]
    L.lcma_gemm(plan, Ad, Bd, C, L.workspace_for(plan))
    torch.cuda.synchronize()
    check_float(C.cpu(), A64, B64, "bf16")
    assert torch.all(Cbig[:, N:].cpu() == 7.0)


@pytest.mark.parametrize("M,N,K", [(48, 4104, 8200), (8, 4104, 14336), (1024, 1024, 8192), (2304, 7424, 4096)])
def test_decode_k_split_graph_replays_with_new_inputs(M, N, K):
    # a captured call (the split kernel and the kernel that adds its
    # partials) replays with the inputs changed in place: each replay equals
    # the eager product, bit for bit
    say("decode K split graph", M, N, K)
    plan = L.lcma_plan_ex(M, N, K, "bf16", force="classic")
    ws = L.workspace_for(plan)
    Ad = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    Bd = torch.empty((K, N), dtype=torch.bfloat16, device=DEV)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    A, B, _, _ = gen(M, N, K, "bf16", "normal_sqrtk", seed=80)
    Ad.copy_(A.to(DEV)); Bd.copy_(B.to(DEV))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.lcma_gemm(plan, Ad, Bd, C, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.lcma_gemm(plan, Ad, Bd, C, ws)
    for seed in (81, 82, 83):
        A, B, A64, B64 = gen(M, N, K, "bf16", "normal_sqrtk", seed=seed)
        Ad.copy_(A.to(DEV)); Bd.copy_(B.to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = si.bits(C.cpu())
        C2 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        L.lcma_gemm(plan, Ad, Bd, C2, L.workspace_for(plan))
        torch.cuda.synchronize()
        assert np.array_equal(got, si.bits(C2.cpu())), seed
        check_float(C.cpu(), A64, B64, "bf16")


@pytest.mark.parametrize("M,N,K,dtype,dist", [(300, 522, 1000, "f16", "uniform"), (257, 13, 64, "bf16", "normal_sqrtk"),
                                              (1, 14337, 4096, "bf16", "decode"), (1000, 1064, 2050, "bf16", "normal_sqrtk"),
                                              (513, 264, 519, "f16", "int2")])
def test_classic_plan_with_ragged_k_or_n(M, N, K, dtype, dist):
    # a classic plan pads K and N to multiples of 8 in its workspace, runs the
    # 16-byte-load kernels and crops C; gemm_classic takes the element-load
    # kernel on the same inputs
    say("classic ragged plan", M, N, K, dtype)
    A, B, A64, B64 = gen(M, N, K, dtype, dist, seed=M + N + K + 1)
    plan = L.lcma_plan_ex(M, N, K, dtype)
    assert L.lcma_plan_info(plan)[0] == "classic" and L.lcma_plan_info(plan)[1] > 0
    C = planned(A, B, "classic")
    if dist.startswith("int"):
        check_exact(C, A64, B64, dtype)
        check_exact(classic(A, B), A64, B64, dtype)
    else:
        C_ref, absAB = oracle.gemm(A64, B64), abs_product(A64, B64)
        check_float(C, A64, B64, dtype, C_ref, absAB=absAB)
        check_float(classic(A, B), A64, B64, dtype, C_ref, absAB=absAB)


def test_padded_lcma_strided_and_split_calls():
    # strided, unaligned operands; lcma_prepass + lcma_fused equal lcma_gemm;
    # nothing is written outside C
    say("padded strided")
    M, N, K = 333, 250, 210
    Abig, Bbig, _, _ = gen(M, N + 3, K + 5, "f16", "uniform", seed=5)
    A, B = Abig[:, :K], Bbig[:K, :N]
    A64, B64 = si.f64(A), si.f64(B)
    Ad, Bd = Abig.to(DEV)[:, :K], Bbig.to(DEV)[:K, :N]
    plan = L.lcma_plan_ex(M, N, K, "f16", force="l1")
    ws = L.workspace_for(plan)
    Cbig = torch.full((M, N + 7), 7.0, dtype=torch.float16, device=DEV)
    C = Cbig[:, :N]
    L.lcma_gemm(plan, Ad, Bd, C, ws)
    C2 = torch.empty((M, N), dtype=torch.float16, device=DEV)
    L.lcma_prepass(plan, Ad, Bd, ws)
    L.lcma_fused(plan, Ad, Bd, C2, ws)
    torch.cuda.synchronize()
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A.contiguous(), B.contiguous(), A64, B64, "f16", C_ref)
    check_scheme(C.cpu(), A64, B64, "f16", "l1", e_c, C_ref)
    assert torch.equal(C.cpu(), C2.cpu())
    assert torch.all(Cbig[:, N:].cpu() == 7.0)


def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M, N, K = (int(x) for x in rng.integers(1, 700, size=3))
        algo = ["classic", "l1", "l2", "auto"][i % 4]
        dtype = ["f16", "bf16"][(i // 4) % 2]
        cases.append((i, M, N, K, algo, dtype))
    return cases


@pytest.mark.parametrize("i,M,N,K,algo,dtype", _random_cases(32, 2024))
def test_random_shapes_every_path(i, M, N, K, algo, dtype):
    # seeded random shapes (1..699 per dimension, mostly ragged): classic plans
    # (padded when K or N is not a multiple of 8), forced one and two levels
    # (zero-padded when the shape does not split), and the planner's choice
    say("random", i, M, N, K, algo, dtype)
    A, B, A64, B64 = gen(M, N, K, dtype, "uniform", seed=7000 + i)
    optin = int(algo == "l2" and dtype == "f16")
    plan = L.lcma_plan_ex(M, N, K, dtype, force=algo, accuracy_optin=optin)
    chosen = L.lcma_plan_info(plan)[0]
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty((M, N), dtype=A.dtype, device=DEV)
    L.lcma_gemm(plan, Ad, Bd, C, L.workspace_for(plan))
    torch.cuda.synchronize()
    C_ref = oracle.gemm(A64, B64)
    if chosen == "classic":
        check_float(C.cpu(), A64, B64, dtype, C_ref)
    else:
        e_c = classic_error(A, B, A64, B64, dtype, C_ref)
        check_scheme(C.cpu(), A64, B64, dtype, chosen, e_c, C_ref, ratio=RATIO_OPTIN if optin else RATIO)


# ---------------------------------------------------------------- unfused path (any valid description)

def winograd():
    return L.Desc(2, 2, 2, D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W)


def winograd_oracle():
    return oracle.Desc(2, 2, 2, D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W)


def planned_desc(A, B, desc, **kw):
    M, K = A.shape
    N = B.shape[1]
    plan = L.lcma_plan_ex(M, N, K, A.dtype, desc=desc, force="l1", **kw)
    assert L.lcma_plan_info(plan)[0] == "l1"
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.full((M, N), 5.0, dtype=A.dtype, device=DEV)
    ws = L.workspace_for(plan)
    L.lcma_gemm(plan, Ad, Bd, C, ws)
    torch.cuda.synchronize()
    return C.cpu()


@pytest.mark.parametrize("M,N,K,dtype,scheme", [(8192, 8192, 512, "bf16", "builtin"),
                                                (8208, 8192, 528, "f16", "winograd")])
def test_unfused_group_kernel_matches_oracle(M, N, K, dtype, scheme):
    # blocks of at least 4096 x 4096: one persistent launch runs every product
    # per 256 x 256 position (interior tiles, then ragged rows and K)
    say("unfused group", M, N, K, dtype, scheme)
    dist = "uniform" if dtype == "f16" else "normal_sqrtk"
    A, B, A64, B64 = gen(M, N, K, dtype, dist, seed=37)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, dtype, C_ref)
    if scheme == "builtin":
        C = planned(A, B, "l1", combine="unfused")
        check_scheme(C, A64, B64, dtype, "l1", e_c, C_ref, unfused=True)
    else:
        C = planned_desc(A, B, winograd())
        check_scheme(C, A64, B64, dtype, "l1", e_c, C_ref, desc=winograd_oracle(), unfused=True)


@pytest.mark.parametrize("scheme", ["builtin", "winograd", "winograd_signed"])
def test_unfused_group_kernel_integer_inputs_are_exact(scheme):
    # the persistent unfused kernel (k-loops of 8 k-tiles over 4096 x 4096
    # blocks, chained accumulators and fp32 folds) on binary16 integers:
    # |combined operands| <= 4 (Winograd: <= 8), |H| <= 64 * 256 and every
    # partial sum of the chained runs below 2^24, all exact.  Winograd's
    # searched schedule chains four runs and negates one.
    say("unfused group exact", scheme)
    A, B, A64, B64 = gen(8192, 8192, 512, "f16", "int2", seed=38)
    if scheme == "builtin":
        C = planned(A, B, "l1", combine="unfused")
    elif scheme == "winograd":
        C = planned_desc(A, B, winograd())
    else:
        # an equivalent form with permuted products and flipped signs: other
        # chains, carries and negated folds, same result
        C = planned_desc(A, B, L.Desc(2, 2, 2, *D.equivalent(D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W, 3)))
    check_exact(C, A64, B64, "f16")


@pytest.mark.parametrize("M,N,K,dtype", [(1024, 1024, 1024, "bf16"), (512, 768, 640, "f16"), (400, 272, 144, "f16")])
def test_unfused_winograd_variant_matches_oracle(M, N, K, dtype):
    say("unfused winograd", M, N, K, dtype)
    dist = "uniform" if dtype == "f16" else "normal_sqrtk"
    A, B, A64, B64 = gen(M, N, K, dtype, dist, seed=31)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, dtype, C_ref)
    check_scheme(planned_desc(A, B, winograd()), A64, B64, dtype, "l1", e_c, C_ref, desc=winograd_oracle(),
                 unfused=True)
    idist = "int2" if dtype == "f16" else "int1"
    A, B, A64, B64 = gen(M, N, min(K, 256), dtype, idist, seed=32)
    check_exact(planned_desc(A, B, winograd()), A64, B64, dtype)


def test_unfused_builtin_and_naive_descriptions():
    say("unfused builtin / naive")
    A, B, A64, B64 = gen(768, 512, 1024, "bf16", "normal_sqrtk", seed=33)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "bf16", C_ref)
    check_scheme(planned(A, B, "l1"), A64, B64, "bf16", "l1", e_c, C_ref)
    check_scheme(planned(A, B, "l1", combine="unfused"), A64, B64, "bf16", "l1", e_c, C_ref, unfused=True)
    d8 = oracle.naive()
    # the plain block product: no operand is combined, so its error is classic's
    check_scheme(planned_desc(A, B, L.Desc(2, 2, 2, d8.U, d8.V, d8.W)), A64, B64, "bf16", "l1", e_c, C_ref,
                 desc=d8, ratio=2.0, unfused=True)
    A, B, A64, B64 = gen(512, 512, 256, "f16", "int2", seed=34)
    check_exact(planned(A, B, "l1", combine="unfused"), A64, B64, "f16")
    check_exact(planned_desc(A, B, L.Desc(2, 2, 2, d8.U, d8.V, d8.W)), A64, B64, "f16")


# ---------------------------------------------------------------- two levels

def test_l2_bf16_matches_oracle_and_ratio():
    say("l2 bf16")
    A, B, A64, B64 = gen(1024, 1024, 1024, "bf16", "normal_sqrtk", seed=17)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "bf16", C_ref)
    check_scheme(planned(A, B, "l2"), A64, B64, "bf16", "l2", e_c, C_ref)


def test_l2_on_chip_matches_oracle():
    say("l2 on chip bf16")
    A, B, A64, B64 = gen(1024, 1024, 1024, "bf16", "normal_sqrtk", seed=17)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "bf16", C_ref)
    check_scheme(planned(A, B, "l2", combine="l2_on_chip"), A64, B64, "bf16", "l2", e_c, C_ref)
    say("l2 on chip f16 split (opted in)")
    A, B, A64, B64 = gen(512, 768, 1024, "f16", "uniform", seed=19)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "f16", C_ref)
    check_scheme(planned(A, B, "l2", combine="l2_on_chip", split="all", accuracy_optin=1), A64, B64, "f16", "l2",
                 e_c, C_ref, ratio=RATIO_OPTIN)


@pytest.mark.parametrize("combine", ["auto", "l2_on_chip"])
def test_l2_bf16_operands_match_the_oracle_with_the_same_rounding(combine):
    # bfloat16 combined operands (not the default for two levels, opted in:
    # about 5.8x the classic error): the GPU result must equal the oracle's
    # evaluation of the same scheme with the same operand rounding up to fp32
    # accumulation order and the final cast
    say("l2 bf16 operands", combine)
    A, B, A64, B64 = gen(512, 1024, 768, "bf16", "normal_sqrtk", seed=29)
    with pytest.raises(L.LcmaError):
        L.lcma_plan_ex(512, 1024, 768, "bf16", force="l2", combine=combine, bf16_ops_f16=-1)
    C2 = planned(A, B, "l2", combine=combine, bf16_ops_f16=-1, accuracy_optin=1)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "bf16", C_ref)
    e = check_scheme(C2, A64, B64, "bf16", "l2", e_c, C_ref, ops="bf16", ratio=RATIO_OPTIN)
    assert e > 4.5 * e_c          # the documented band (5.8x on the oracle): above the 4x gate, below 7x


@pytest.mark.parametrize("split", ["auto", "none", "all"])
def test_l2_outer_level_ragged_blocks(split):
    # blocks of 272 x 136 x 264: the 128-row group tiles end ragged in M and
    # N, k-tiles ragged in K; every split mode of the outer launches
    say("l2 ragged", split)
    A, B, A64, B64 = gen(1088, 1056, 544, "bf16", "normal_sqrtk", seed=23)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "bf16", C_ref)
    C2 = planned(A, B, "l2", split=split)
    check_scheme(C2, A64, B64, "bf16", "l2", e_c, C_ref)
    assert np.array_equal(si.bits(C2), si.bits(planned(A, B, "l2", split=split)))


def test_l2_f16_and_split_all():
    say("l2 f16 split (opted in)")
    A, B, A64, B64 = gen(512, 768, 1024, "f16", "uniform", seed=19)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "f16", C_ref)
    C0 = planned(A, B, "l2", accuracy_optin=1)
    e0 = check_scheme(C0, A64, B64, "f16", "l2", e_c, C_ref, ratio=RATIO_OPTIN)
    assert e0 > 4.5 * e_c          # the documented band (5.8-5.9x on the oracle)
    C1 = planned(A, B, "l2", split="all", accuracy_optin=1)
    check_scheme(C1, A64, B64, "f16", "l2", e_c, C_ref, ratio=RATIO_OPTIN)
    assert np.array_equal(si.bits(C1), si.bits(planned(A, B, "l2", split="all", accuracy_optin=1)))


# ---------------------------------------------------------------- combine at load

def test_at_load_integer_inputs_are_exact():
    say("at_load exact")
    A, B, A64, B64 = gen(**si.SQUARE_512_F16_INT)
    check_exact(planned(A, B, "l1", combine="at_load"), A64, B64, "f16")
    A, B, A64, B64 = gen(256, 512, 384, "bf16", "int1", seed=2)
    check_exact(planned(A, B, "l1", combine="at_load"), A64, B64, "bf16")


# 512^3 and 1024^3: whole group tiles; 400 x 272 x 144 and 600 x 528 x 512:
# ragged group tiles (blocks of 200 x 136 x 72 and 300 x 264 x 256);
# 500 x 520 x 260: padded to 512 x 544 x 288
@pytest.mark.parametrize("M,N,K,dtype,dist", [(512, 512, 512, "f16", "uniform"),
                                              (1024, 1024, 1024, "bf16", "normal_sqrtk"),
                                              (400, 272, 144, "f16", "uniform"),
                                              (600, 528, 512, "bf16", "normal_sqrtk"),
                                              (500, 520, 260, "f16", "uniform")])
def test_at_load_matches_oracle(M, N, K, dtype, dist):
    say("at_load", M, N, K, dtype)
    A, B, A64, B64 = gen(M, N, K, dtype, dist, seed=21)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, dtype, C_ref)
    C = planned(A, B, "l1", combine="at_load")
    check_scheme(C, A64, B64, dtype, "l1", e_c, C_ref, ops=op_type(dtype, "l1", combine="at_load"))


def test_at_load_halves_strides_and_repeats():
    say("at_load halves")
    M, N, K = 768, 640, 1024
    A, B, A64, B64 = gen(M, N, K, "bf16", "normal_sqrtk", seed=23)
    # without a split the plan needs no workspace at all
    plan = L.lcma_plan_ex(M, N, K, "bf16", force="l1", combine="at_load", split="none")
    assert L.lcma_plan_info(plan)[:2] == ("l1", 0)
    Ad, Bd = A.to(DEV), B.to(DEV)
    C0 = torch.empty((M, N), dtype=A.dtype, device=DEV)
    L.lcma_gemm(plan, Ad, Bd, C0, None)
    # the two halves: the pre-pass half has nothing to do
    C1 = torch.full((M, N), 3.0, dtype=A.dtype, device=DEV)
    L.lcma_prepass(plan, Ad, Bd, None)
    L.lcma_fused(plan, Ad, Bd, C1, None)
    # strided operands and output
    As = torch.zeros((M, K + 24), dtype=A.dtype, device=DEV)
    Bs = torch.zeros((K, N + 40), dtype=A.dtype, device=DEV)
    Cs = torch.full((M, N + 8), 7.0, dtype=A.dtype, device=DEV)
    As[:, :K] = Ad
    Bs[:, :N] = Bd
    L.lcma_gemm(plan, As, Bs, Cs, None, lda=K + 24, ldb=N + 40, ldc=N + 8)
    C2 = torch.empty((M, N), dtype=A.dtype, device=DEV)
    L.lcma_gemm(plan, Ad, Bd, C2, None)
    torch.cuda.synchronize()
    ref = si.bits(C0.cpu())
    assert np.array_equal(si.bits(C1.cpu()), ref)
    assert np.array_equal(si.bits(Cs[:, :N].cpu()), ref)
    assert np.all(Cs[:, N:].cpu().float().numpy() == 7.0)
    assert np.array_equal(si.bits(C2.cpu()), ref)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "bf16", C_ref)
    check_scheme(C0.cpu(), A64, B64, "bf16", "l1", e_c, C_ref, ops="bf16")


# 2560 x 2560 x 1024: 100 groups on 256 workers, the tail split by default;
# 1024^3 and 600 x 528 x 512 (ragged tiles): every group split
@pytest.mark.parametrize("M,N,K,split", [(2560, 2560, 1024, "auto"), (1024, 1024, 1024, "all"),
                                         (600, 528, 512, "all")])
def test_at_load_split_groups(M, N, K, split):
    say("at_load split", M, N, K, split)
    A, B, A64, B64 = gen(M, N, K, "bf16", "normal_sqrtk", seed=25)
    plan = L.lcma_plan_ex(M, N, K, "bf16", force="l1", combine="at_load", split=split)
    items, _ = L.lcma_plan_schedule(plan)
    assert any(it[4] >= 0 for it in items)
    ws = L.workspace_for(plan)
    # stale fix-up counters: the call must clear them itself
    ws.fill_(0x7F)
    Ad, Bd = A.to(DEV), B.to(DEV)
    outs = []
    for _ in range(2):
        C = torch.full((M, N), 9.0, dtype=A.dtype, device=DEV)
        L.lcma_gemm(plan, Ad, Bd, C, ws)
        torch.cuda.synchronize()
        outs.append(C.cpu())
    # fp32 addition of the two pieces' partials commutes: repeats are bitwise equal
    assert np.array_equal(si.bits(outs[0]), si.bits(outs[1]))
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "bf16", C_ref)
    check_scheme(outs[0], A64, B64, "bf16", "l1", e_c, C_ref, ops="bf16")


# ---------------------------------------------------------------- special values

def _special_inputs(dtype):
    A, B, A64, B64 = gen(512, 512, 512, dtype, "uniform", seed=41)
    A, B = A.clone(), B.clone()
    A[3, 5] = float("nan")          # block A11
    A[300, 7] = float("inf")        # block A21
    B[9, 400] = float("-inf")       # block B12
    B[260, 20] = float("nan")       # block B21
    return A, B, si.f64(A), si.f64(B)


def _same_specials(C, C_ref):
    c = si.f64(C)
    assert np.array_equal(np.isnan(c), np.isnan(C_ref)), (np.isnan(c).sum(), np.isnan(C_ref).sum())
    for sgn in (1, -1):
        assert np.array_equal(c == sgn * np.inf, C_ref == sgn * np.inf)
    fin = np.isfinite(C_ref)
    return c, fin


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_nan_and_inf_propagate_as_the_oracle_says(dtype):
    # NaN and Inf inputs propagate through IEEE arithmetic.  The classic
    # product spreads a non-finite A[i, k] over row i; a scheme spreads it
    # through every product whose combined operands contain it, which differs
    # (a NaN in A11 reaches C11, C12 and C22 through P1, P3, P5 and P6).  The
    # GPU's pattern of NaN, +Inf and -Inf must equal the oracle's evaluation of
    # the same computation, and the finite entries its bounds.
    say("special values", dtype)
    A, B, A64, B64 = _special_inputs(dtype)
    with np.errstate(invalid="ignore", over="ignore"):
        C_ref = oracle.gemm(A64, B64)
        c, fin = _same_specials(classic(A, B), C_ref)
        Af, Bf = np.nan_to_num(A64, nan=0, posinf=0, neginf=0), np.nan_to_num(B64, nan=0, posinf=0, neginf=0)
        bound = metrics.bound_classic(C_ref, abs_product(Af, Bf), 512, dtype)
        assert metrics.elementwise(c[fin], C_ref[fin], bound[fin])[1] == 0
        for combine in ("prepass", "at_load", "unfused"):
            C_sh, _ = oracle.lcma(A64, B64, oracle.strassen(), 1, round_operands=op_type(dtype, "l1", combine=combine))
            assert not np.array_equal(np.isnan(C_sh), np.isnan(C_ref))     # the scheme spreads it differently
            _same_specials(planned(A, B, "l1", combine=combine), C_sh)


def test_binary16_operand_overflow_of_two_levels_is_inf_as_the_oracle_says():
    # Two levels of bfloat16 inputs round combined operands to binary16 by
    # default: a combination of up to four entries at or beyond 65520 rounds
    # to +-Inf (the classic product of the same inputs stays finite).  The
    # GPU's non-finite pattern must equal the oracle's evaluation of the scheme
    # with binary16 operands.
    say("binary16 operand overflow")
    M = N = K = 512
    A, B, _, _ = gen(M, N, K, "bf16", "normal_sqrtk", seed=43)
    A = A.clone()
    for bi in range(4):                 # the same local entry of every 128 x 128 block of A
        for bk in range(4):
            A[bi * 128 + 10, bk * 128 + 20] = 20000.0
    A64, B64 = si.f64(A), si.f64(B)
    with np.errstate(invalid="ignore", over="ignore"):
        C_ref = oracle.gemm(A64, B64)
        assert np.all(np.isfinite(C_ref)) and np.all(np.isfinite(si.f64(classic(A, B))))
        C_sh, _ = oracle.lcma(A64, B64, oracle.strassen2(), 1, round_operands="f16")
        assert not np.all(np.isfinite(C_sh))
        _same_specials(planned(A, B, "l2"), C_sh)


# ---------------------------------------------------------------- full-size workloads

def test_square_4096_bf16_classic_and_one_level():
    say("4096 bf16")
    A, B, A64, B64 = gen(**si.SQUARE_4096_BF16)
    C_ref = oracle.gemm(A64, B64)
    e_c = check_float(classic(A, B), A64, B64, "bf16", C_ref, blocks=2)
    for ops in (-1, 1):
        say("4096 bf16 l1 ops", ops)
        check_scheme(planned(A, B, "l1", bf16_ops_f16=ops), A64, B64, "bf16", "l1", e_c, C_ref,
                     ops=op_type("bf16", "l1", ops))
    # the same product with the combination done while staging tiles
    say("4096 bf16 l1 at load")
    check_scheme(planned(A, B, "l1", combine="at_load"), A64, B64, "bf16", "l1", e_c, C_ref, ops="bf16")


@pytest.mark.parametrize("m", si.DECODE_MS)
def test_skinny_decode_shapes(m):
    say("decode", m)
    w = si.decode_shape(m)
    A, B, A64, B64 = gen(**w)
    plan = L.lcma_plan(w["M"], w["N"], w["K"], "bf16")
    assert L.lcma_plan_info(plan)[0] == "classic"
    check_float(classic(A, B), A64, B64, "bf16")


def test_sweep_shapes_auto():
    for wl in si.sweep_workloads():
        M, N, K = wl["M"], wl["N"], wl["K"]
        say("sweep", M, N, K)
        A, B, A64, B64 = gen(**wl)
        plan = L.lcma_plan(M, N, K, "f16")
        algo = L.lcma_plan_info(plan)[0]
        assert algo == "classic"
        Ad, Bd = A.to(DEV), B.to(DEV)
        C = torch.empty((M, N), dtype=torch.float16, device=DEV)
        L.lcma_gemm(plan, Ad, Bd, C, L.workspace_for(plan))
        torch.cuda.synchronize()
        check_float(C.cpu(), A64, B64, "f16")
        del Ad, Bd, C


@pytest.mark.parametrize("i", range(24))
def test_sweep_shapes_forced_levels(i):
    # every seeded sweep shape through forced one and two levels (zero-padded
    # where a shape does not split; two levels on binary16 inputs opted in,
    # checked against its documented ratio band)
    wl = si.sweep_workloads()[i]
    M, N, K = wl["M"], wl["N"], wl["K"]
    A, B, A64, B64 = gen(**wl)
    C_ref = oracle.gemm(A64, B64)
    e_c = classic_error(A, B, A64, B64, "f16", C_ref)
    for algo in ("l1", "l2"):
        say("sweep forced", algo, M, N, K)
        C = planned(A, B, algo, accuracy_optin=int(algo == "l2"))
        check_scheme(C, A64, B64, "f16", algo, e_c, C_ref, ratio=RATIO if algo == "l1" else RATIO_OPTIN)


def test_square_16384_bf16_sampled():
    # The oracle cannot form the whole 16384^3 product here.  Checked instead:
    # one full row in every 256-row band of tiles (a seeded row per band), so
    # every output tile of every kernel is seen: classic elementwise within
    # its bound, LCMA per 256-column segment of each row within 4 u_out; and
    # the Freivalds residual of every 128-row and 128-column band within
    # 2 u_out (about 0.5 u_out for correctly rounded outputs; a zeroed 16 x 16
    # tile adds about 2.8 u_out).  Winograd's variant carries 3.7x the classic
    # error overall and up to 4.4x in its C21 and C22 blocks (band residuals
    # up to 2.3 u_out), so its bands are held to 3 u_out: a zeroed tile on top
    # of that noise still reaches about 3.5 u_out.
    say("16384 bf16")
    w = si.SQUARE_16384_BF16
    A, B = si.gen(**w)
    A64, B64 = si.f64(A), si.f64(B)
    n = w["M"]
    rng = np.random.default_rng(2)
    rows = np.array([b + int(rng.integers(0, 256)) for b in range(0, n, 256)])
    ref = oracle.gemm(A64[rows], B64)
    absAB = oracle.gemm(np.abs(A64[rows]), np.abs(B64))
    u = metrics.UNIT_ROUNDOFF["bf16"]
    res = {}
    # one level: the planner's choice at this size (the unfused path) and the
    # fused group kernel after a pre-pass; two levels with binary16 operands
    for name, algo, kw in (("classic", "classic", {}), ("l1", "l1", {}), ("l1_fused", "l1", {"combine": "prepass"}),
                           ("l1_winograd", "l1", {"desc": winograd()}), ("l2", "l2", {})):
        say("16384", name)
        C = si.f64(planned(A, B, algo, **kw))
        got = C[rows]
        assert np.all(np.isfinite(got))
        res[name] = metrics.e_rel(got, ref)
        assert res[name] <= 4 * u, (name, res[name])
        if name == "classic":
            worst, bad = metrics.elementwise(got, ref, metrics.bound_classic(ref, absAB, n, "bf16"))
            assert bad == 0, (worst, bad)
        else:
            seg = [metrics.e_rel(got[:, c:c + 256], ref[:, c:c + 256]) for c in range(0, n, 256)]
            assert max(seg) <= 4 * u, (name, max(seg))
        rb, cb = metrics.freivalds_bands(C, A64, B64)
        assert max(rb.max(), cb.max()) <= (3 if name == "l1_winograd" else 2) * u, (name, rb.max(), cb.max())
        del C, got
    assert max(res["l1"], res["l1_fused"], res["l1_winograd"], res["l2"]) <= 4 * res["classic"]


def test_square_32768_bf16_sampled_unfused():
    # The size at which the unfused one level overtakes the classic kernel:
    # classic, Strassen on the unfused path (the planner's one level here)
    # and Winograd's variant (searched run schedule; 16 positions per
    # workgroup, 1 GiB fp32 blocks).  Checked like 16384^3 with one seeded row
    # per 1024-row band: classic elementwise within its bound, LCMA per
    # 256-column segment within 4 u_out and within 4x the classic error, and
    # the Freivalds residual of every 64-row and 64-column band within 2 u_out
    # (3 u_out for Winograd's variant): at this width a zeroed 16 x 16 tile
    # adds about 2.8 u_out to a 64-wide band, as to a 128-wide one at 16384.
    say("32768 bf16")
    w = si.SQUARE_32768_BF16
    A, B = si.gen(**w)
    n = w["M"]
    rng = np.random.default_rng(3)
    rows = np.array([b + int(rng.integers(0, 1024)) for b in range(0, n, 1024)])
    A64, B64 = si.f64(A), si.f64(B)
    A64r = A64[rows]
    say("32768 oracle rows")
    ref = oracle.gemm(A64r, B64)
    absAB = oracle.gemm(np.abs(A64r), np.abs(B64))
    u = metrics.UNIT_ROUNDOFF["bf16"]
    res = {}
    for name, kw in (("classic", dict(algo="classic")), ("l1", dict(algo="l1")),
                     ("winograd", dict(algo="l1", desc=winograd()))):
        say("32768", name)
        kw = dict(kw)
        C = planned(A, B, kw.pop("algo"), **kw)
        got = si.f64(C[rows])
        assert np.all(np.isfinite(got))
        res[name] = metrics.e_rel(got, ref)
        assert res[name] <= 4 * u, (name, res[name])
        if name == "classic":
            worst, bad = metrics.elementwise(got, ref, metrics.bound_classic(ref, absAB, n, "bf16"))
            assert bad == 0, (worst, bad)
        else:
            seg = [metrics.e_rel(got[:, c:c + 256], ref[:, c:c + 256]) for c in range(0, n, 256)]
            assert max(seg) <= 4 * u, (name, max(seg))
        rb, cb = metrics.freivalds_bands(si.f64(C), A64, B64, band=64)
        assert max(rb.max(), cb.max()) <= (3 if name == "winograd" else 2) * u, (name, rb.max(), cb.max())
        del C, got
    assert max(res["l1"], res["winograd"]) <= 4 * res["classic"], res


def test_prepared_calls_equal_lcma_gemm():
    # a call prepared once (arguments checked once) enqueues the same work as
    # lcma_gemm: bitwise equal results, repeatable, for a streaming-kernel plan
    # and a one-level plan with a workspace
    say("prepared calls")
    for (M, N, K, algo) in ((16, 14336, 4096, "classic"), (512, 512, 512, "l1")):
        A, B, A64, B64 = gen(M, N, K, "bf16", "normal_sqrtk", seed=44)
        Ad, Bd = A.to(DEV), B.to(DEV)
        plan = L.lcma_plan_ex(M, N, K, "bf16", force=algo)
        ws = L.workspace_for(plan)
        C1 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        C2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        L.lcma_gemm(plan, Ad, Bd, C1, ws)
        call = L.lcma_gemm_prepared(plan, Ad, Bd, C2, ws)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        assert torch.equal(C1, C2), (M, N, K, algo)


# ---------------------------------------------------------------- graph capture

@pytest.mark.parametrize("algo,kw", [("classic", {}), ("l1", {"split": "all"}), ("l2", {})])
def test_graph_capture_replays_match_eager(algo, kw):
    # Every path launches only kernels (the split counters are cleared by the
    # pre-pass kernel, not a memset), so a call can be captured into a HIP
    # graph; each replay, with eager work and synchronisation in between,
    # must reproduce the eager result bit for bit.
    say("graph", algo, kw)
    M = N = K = 1024
    A, B, _, _ = gen(M, N, K, "bf16", "normal_sqrtk", seed=31)
    Ad, Bd = A.to(DEV), B.to(DEV)
    plan = L.lcma_plan_ex(M, N, K, "bf16", force=algo, **kw)
    ws = L.workspace_for(plan)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    L.lcma_gemm(plan, Ad, Bd, C, ws)
    torch.cuda.synchronize()
    eager = C.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.lcma_gemm(plan, Ad, Bd, C, ws)      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.lcma_gemm(plan, Ad, Bd, C, ws)
    for rep in range(4):
        C.fill_(float(rep + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, eager), rep
        # eager work on the same buffers between replays
        L.lcma_gemm(plan, Ad, Bd, C, ws)
        torch.cuda.synchronize()
        assert torch.equal(C, eager), rep


# ---------------------------------------------------------------- measurement references

def test_measurement_references_run_and_copy_exactly():
    say("measurement references")
    n = (64 << 20) + 48                       # not a multiple of the chunking
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros_like(src)
    L.lcma_measure_copy(src, dst)
    word = torch.zeros(2, dtype=torch.int32, device=DEV)
    L.lcma_measure_read(src, word[:1])       # reads src; may write word[0] only
    out = torch.full((2 * 512,), float("nan"), dtype=torch.float32, device=DEV)
    flops = L.lcma_measure_mfma(out, 2, 10, "bf16")
    torch.cuda.synchronize()
    assert torch.equal(src, dst) and int(word[1]) == 0
    assert flops == 2 * 8 * 10 * 16 * 16384
    assert torch.all(torch.isfinite(out))
