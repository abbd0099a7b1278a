"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Gates (normwise, from the accuracy target of the build):
  e_nw = ||C - C_ref||_F / (||A||_F ||B||_F) <= 1e-3 (binary16), <= 8e-3 (bfloat16),
  e_nw(LCMA) <= 4 * e_nw(classic GPU) on the same inputs.
Because e_nw shrinks like 1/sqrt(K) for independent entries, every float case
also requires e_rel = ||C - C_ref||_F / ||C_ref||_F <= 4 u_out (whole matrix
and per output block); integer-valued inputs must match bit for bit.
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


def check_float(C, A64, B64, dtype, C_ref=None, blocks=1):
    C_ref = oracle.gemm(A64, B64) if C_ref is None else C_ref
    c = si.f64(C)
    assert np.all(np.isfinite(c))
    e = metrics.e_nw(c, C_ref, A64, B64)
    assert e <= metrics.GATE_NW[dtype], e
    u = metrics.UNIT_ROUNDOFF[dtype]
    assert metrics.e_rel(c, C_ref) <= 4 * u
    if blocks > 1:
        assert max(metrics.e_rel_blocks(c, C_ref, blocks)) <= 4 * u
    return e


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
    (60, 2056, 1000),          # streaming kernel (64-row A), N and K tails
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", CLASSIC_SHAPES)
def test_classic_matches_oracle(M, N, K, dtype):
    say("classic", M, N, K, dtype)
    A, B, A64, B64 = gen(M, N, K, dtype, "uniform", seed=M + N + K)
    check_float(classic(A, B), A64, B64, dtype)


@pytest.mark.parametrize("dtype,dist", [("f16", "int2"), ("bf16", "int1")])
@pytest.mark.parametrize("M,N,K", [(33, 40, 24), (130, 200, 96), (257, 136, 120), (512, 512, 256), (4100, 264, 64),
                                   (1000, 1064, 256), (4096, 4104, 96), (48, 1000, 200)])
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


# ---------------------------------------------------------------- one level

def test_l1_square_512_f16_matches_oracle_and_ratio():
    say("l1 512 f16")
    A, B, A64, B64 = gen(**si.SQUARE_512_F16)
    C_ref = oracle.gemm(A64, B64)
    e_c = check_float(classic(A, B), A64, B64, "f16", C_ref)
    C1 = planned(A, B, "l1")
    e_1 = check_float(C1, A64, B64, "f16", C_ref, blocks=2)
    assert e_1 <= 4 * e_c, (e_1, e_c)
    # against the oracle's evaluation with binary16 combined operands: only
    # fp32 accumulation order and the final rounding differ
    C_sh, n = oracle.lcma(A64, B64, oracle.strassen(), 1, round_operands="f16")
    assert n == 7
    assert metrics.e_rel(si.f64(C1), C_sh) <= 2 * metrics.UNIT_ROUNDOFF["f16"]


@pytest.mark.parametrize("algo,combine", [("l1", "auto"), ("l2", "auto"), ("l2", "l2_on_chip")])
def test_lcma_integer_inputs_are_exact(algo, combine):
    say("exact", algo, combine)
    A, B, A64, B64 = gen(**si.SQUARE_512_F16_INT)
    check_exact(planned(A, B, algo, combine=combine), A64, B64, "f16")
    A, B, A64, B64 = gen(256, 512, 384, "bf16", "int1", seed=2)
    check_exact(planned(A, B, algo, combine=combine), A64, B64, "bf16")


@pytest.mark.parametrize("ops", [-1, 1])
def test_l1_bf16_operand_modes(ops):
    say("l1 bf16 ops", ops)
    A, B, A64, B64 = gen(1024, 1024, 1024, "bf16", "normal_sqrtk", seed=9)
    C_ref = oracle.gemm(A64, B64)
    e_c = check_float(classic(A, B), A64, B64, "bf16", C_ref)
    e_1 = check_float(planned(A, B, "l1", bf16_ops_f16=ops), A64, B64, "bf16", C_ref, blocks=2)
    assert e_1 <= 4 * e_c


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


@pytest.mark.parametrize("M,N,K,dtype", [(400, 272, 144, "f16"), (600, 528, 512, "bf16")])
def test_l1_ragged_group_tiles(M, N, K, dtype):
    # quadrants that do not fill whole 128 x 128 group tiles (and a k tail in
    # the first shape): the fused kernel's bounded loads and edge stores
    say("l1 ragged", M, N, K, dtype)
    dist = "uniform" if dtype == "f16" else "normal_sqrtk"
    A, B, A64, B64 = gen(M, N, K, dtype, dist, seed=17)
    C_ref = oracle.gemm(A64, B64)
    e_c = check_float(classic(A, B), A64, B64, dtype, C_ref)
    e_1 = check_float(planned(A, B, "l1"), A64, B64, dtype, C_ref, blocks=2)
    assert e_1 <= 4 * e_c, (e_1, e_c)
    idist = "int2" if dtype == "f16" else "int1"
    A, B, A64, B64 = gen(M, N, min(K, 256), dtype, idist, seed=18)
    check_exact(planned(A, B, "l1"), A64, B64, dtype)


@pytest.mark.parametrize("split", ["none", "all"])
def test_l1_split_modes_reproducible(split):
    say("l1 split", split)
    A, B, A64, B64 = gen(1024, 768, 512, "f16", "uniform", seed=13)
    C_ref = oracle.gemm(A64, B64)
    runs = [planned(A, B, "l1", split=split) for _ in range(3)]
    check_float(runs[0], A64, B64, "f16", C_ref, blocks=2)
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
    C = si.f64(planned(A, B, "l1"))
    rows = np.random.default_rng(1).choice(n, 24, replace=False)
    ref = np.stack([oracle.gemm_rows(A64, B64, r, r + 1)[0] for r in rows])
    assert metrics.e_rel(C[rows], ref) <= 4 * metrics.UNIT_ROUNDOFF["bf16"]
    assert metrics.freivalds(C, A64, B64) <= 4 * metrics.UNIT_ROUNDOFF["bf16"]


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
    rows = np.random.default_rng(2).choice(M, 16, replace=False)
    ref = np.stack([oracle.gemm_rows(A64, B64, r, r + 1)[0] for r in rows])
    for C in (C0, C1):
        assert metrics.e_rel(si.f64(C)[rows], ref) <= 4 * metrics.UNIT_ROUNDOFF["bf16"]
    assert metrics.freivalds(si.f64(C1), A64, B64) <= 4 * metrics.UNIT_ROUNDOFF["bf16"]


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
    C = planned(A, B, algo)
    if dist.startswith("int"):
        check_exact(C, A64, B64, dtype)
    else:
        check_float(C, A64, B64, dtype)


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
        check_float(C, A64, B64, dtype)
        check_float(classic(A, B), A64, B64, dtype)


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
    check_float(C.cpu(), A64, B64, "f16")
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
    plan = L.lcma_plan_ex(M, N, K, dtype, force=algo)
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty((M, N), dtype=A.dtype, device=DEV)
    L.lcma_gemm(plan, Ad, Bd, C, L.workspace_for(plan))
    torch.cuda.synchronize()
    check_float(C.cpu(), A64, B64, dtype)


# ---------------------------------------------------------------- unfused path (any valid description)

def winograd():
    return L.Desc(2, 2, 2, D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W)


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
    if scheme == "builtin":
        C = planned(A, B, "l1", combine="unfused")
        C_sh, _ = oracle.lcma(A64, B64, oracle.strassen(), 1, round_operands=dtype)
    else:
        C = planned_desc(A, B, winograd())
        dw = oracle.Desc(2, 2, 2, D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W)
        C_sh, _ = oracle.lcma(A64, B64, dw, 1, round_operands=dtype)
    check_float(C, A64, B64, dtype, C_ref, blocks=2)
    assert metrics.e_rel(si.f64(C), C_sh) <= 2 * metrics.UNIT_ROUNDOFF[dtype]


@pytest.mark.parametrize("M,N,K,dtype", [(1024, 1024, 1024, "bf16"), (512, 768, 640, "f16"), (400, 272, 144, "f16")])
def test_unfused_winograd_variant_matches_oracle(M, N, K, dtype):
    say("unfused winograd", M, N, K, dtype)
    dist = "uniform" if dtype == "f16" else "normal_sqrtk"
    A, B, A64, B64 = gen(M, N, K, dtype, dist, seed=31)
    C_ref = oracle.gemm(A64, B64)
    e_c = check_float(classic(A, B), A64, B64, dtype, C_ref)
    e_w = check_float(planned_desc(A, B, winograd()), A64, B64, dtype, C_ref, blocks=2)
    assert e_w <= 4 * e_c, (e_w, e_c)
    # against the oracle's evaluation of the same description with operands
    # rounded to the operand type: only the fp32 order and the final rounding differ
    dw = oracle.Desc(2, 2, 2, D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W)
    C_sh, n = oracle.lcma(A64, B64, dw, 1, round_operands=dtype)
    assert n == 7
    assert metrics.e_rel(si.f64(planned_desc(A, B, winograd())), C_sh) <= 2 * metrics.UNIT_ROUNDOFF[dtype]
    idist = "int2" if dtype == "f16" else "int1"
    A, B, A64, B64 = gen(M, N, min(K, 256), dtype, idist, seed=32)
    check_exact(planned_desc(A, B, winograd()), A64, B64, dtype)


def test_unfused_builtin_and_naive_descriptions():
    say("unfused builtin / naive")
    A, B, A64, B64 = gen(768, 512, 1024, "bf16", "normal_sqrtk", seed=33)
    C_ref = oracle.gemm(A64, B64)
    e_c = check_float(classic(A, B), A64, B64, "bf16", C_ref)
    e_f = check_float(planned(A, B, "l1"), A64, B64, "bf16", C_ref, blocks=2)
    e_u = check_float(planned(A, B, "l1", combine="unfused"), A64, B64, "bf16", C_ref, blocks=2)
    assert e_u <= 4 * e_c and e_f <= 4 * e_c
    d8 = oracle.naive()
    e_n = check_float(planned_desc(A, B, L.Desc(2, 2, 2, d8.U, d8.V, d8.W)), A64, B64, "bf16", C_ref, blocks=2)
    assert e_n <= 2 * e_c
    A, B, A64, B64 = gen(512, 512, 256, "f16", "int2", seed=34)
    check_exact(planned(A, B, "l1", combine="unfused"), A64, B64, "f16")
    check_exact(planned_desc(A, B, L.Desc(2, 2, 2, d8.U, d8.V, d8.W)), A64, B64, "f16")


# ---------------------------------------------------------------- two levels

def test_l2_bf16_matches_oracle_and_ratio():
    say("l2 bf16")
    A, B, A64, B64 = gen(1024, 1024, 1024, "bf16", "normal_sqrtk", seed=17)
    C_ref = oracle.gemm(A64, B64)
    e_c = check_float(classic(A, B), A64, B64, "bf16", C_ref)
    C2 = planned(A, B, "l2")
    e_2 = check_float(C2, A64, B64, "bf16", C_ref, blocks=4)
    assert e_2 <= 4 * e_c
    C_sh, n = oracle.lcma(A64, B64, oracle.strassen2(), 1, round_operands="f16")
    assert n == 49
    assert metrics.e_rel(si.f64(C2), C_sh) <= 2 * metrics.UNIT_ROUNDOFF["bf16"]


def test_l2_on_chip_matches_oracle():
    say("l2 on chip bf16")
    A, B, A64, B64 = gen(1024, 1024, 1024, "bf16", "normal_sqrtk", seed=17)
    C_ref = oracle.gemm(A64, B64)
    e_c = check_float(classic(A, B), A64, B64, "bf16", C_ref)
    C2 = planned(A, B, "l2", combine="l2_on_chip")
    e_2 = check_float(C2, A64, B64, "bf16", C_ref, blocks=4)
    assert e_2 <= 4 * e_c
    say("l2 on chip f16 split")
    A, B, A64, B64 = gen(512, 768, 1024, "f16", "uniform", seed=19)
    check_float(planned(A, B, "l2", combine="l2_on_chip", split="all"), A64, B64, "f16", blocks=4)


@pytest.mark.parametrize("combine", ["auto", "l2_on_chip"])
def test_l2_bf16_operands_match_the_oracle_with_the_same_rounding(combine):
    # bfloat16 combined operands (not the default for two levels): the GPU
    # result must equal the oracle's evaluation of the same scheme with the
    # same operand rounding up to fp32 accumulation order and the final cast
    say("l2 bf16 operands", combine)
    A, B, A64, B64 = gen(512, 1024, 768, "bf16", "normal_sqrtk", seed=29)
    C2 = planned(A, B, "l2", combine=combine, bf16_ops_f16=-1)
    check_float(C2, A64, B64, "bf16", blocks=4)
    C_sh, n = oracle.lcma(A64, B64, oracle.strassen2(), 1, round_operands="bf16")
    assert n == 49
    assert metrics.e_rel(si.f64(C2), C_sh) <= 2 * metrics.UNIT_ROUNDOFF["bf16"]


@pytest.mark.parametrize("split", ["auto", "none", "all"])
def test_l2_outer_level_ragged_blocks(split):
    # blocks of 272 x 136 x 264: the 128-row group tiles end ragged in M and
    # N, k-tiles ragged in K; every split mode of the outer launches
    say("l2 ragged", split)
    A, B, A64, B64 = gen(1088, 1056, 544, "bf16", "normal_sqrtk", seed=23)
    C_ref = oracle.gemm(A64, B64)
    e_c = check_float(classic(A, B), A64, B64, "bf16", C_ref)
    C2 = planned(A, B, "l2", split=split)
    e_2 = check_float(C2, A64, B64, "bf16", C_ref, blocks=4)
    assert e_2 <= 4 * e_c
    assert np.array_equal(si.bits(C2), si.bits(planned(A, B, "l2", split=split)))


def test_l2_f16_and_split_all():
    say("l2 f16 split")
    A, B, A64, B64 = gen(512, 768, 1024, "f16", "uniform", seed=19)
    C_ref = oracle.gemm(A64, B64)
    C0 = planned(A, B, "l2")
    check_float(C0, A64, B64, "f16", C_ref, blocks=4)
    C1 = planned(A, B, "l2", split="all")
    check_float(C1, A64, B64, "f16", C_ref, blocks=4)
    assert np.array_equal(si.bits(C1), si.bits(planned(A, B, "l2", split="all")))


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
    e_c = check_float(classic(A, B), A64, B64, dtype, C_ref)
    C = planned(A, B, "l1", combine="at_load")
    e = check_float(C, A64, B64, dtype, C_ref, blocks=2)
    assert e <= 4 * e_c, (e, e_c)
    if (M, N, K) != (500, 520, 260):
        # against the oracle's evaluation with each combined operand rounded
        # once to the operand type: only the fp32 accumulation order and the
        # final rounding differ
        C_sh, n = oracle.lcma(A64, B64, oracle.strassen(), 1, round_operands=dtype)
        assert n == 7
        assert metrics.e_rel(si.f64(C), C_sh) <= 2 * metrics.UNIT_ROUNDOFF[dtype]


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
    check_float(C0.cpu(), A64, B64, "bf16", blocks=2)


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
    e_c = check_float(classic(A, B), A64, B64, "bf16", C_ref)
    e = check_float(outs[0], A64, B64, "bf16", C_ref, blocks=2)
    assert e <= 4 * e_c, (e, e_c)


# ---------------------------------------------------------------- full-size workloads

def test_square_4096_bf16_classic_and_one_level():
    say("4096 bf16")
    A, B, A64, B64 = gen(**si.SQUARE_4096_BF16)
    C_ref = oracle.gemm(A64, B64)
    e_c = check_float(classic(A, B), A64, B64, "bf16", C_ref, blocks=2)
    for ops in (-1, 1):
        C1 = planned(A, B, "l1", bf16_ops_f16=ops)
        e_1 = check_float(C1, A64, B64, "bf16", C_ref, blocks=2)
        assert e_1 <= 4 * e_c, (ops, e_1, e_c)
        assert metrics.freivalds(si.f64(C1), A64, B64) <= 4 * metrics.UNIT_ROUNDOFF["bf16"]
    # the same product with the combination done while staging tiles
    C1 = planned(A, B, "l1", combine="at_load")
    e_1 = check_float(C1, A64, B64, "bf16", C_ref, blocks=2)
    assert e_1 <= 4 * e_c, ("at_load", e_1, e_c)
    assert metrics.freivalds(si.f64(C1), A64, B64) <= 4 * metrics.UNIT_ROUNDOFF["bf16"]


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
        Ad, Bd = A.to(DEV), B.to(DEV)
        C = torch.empty((M, N), dtype=torch.float16, device=DEV)
        L.lcma_gemm(plan, Ad, Bd, C, L.workspace_for(plan))
        torch.cuda.synchronize()
        check_float(C.cpu(), A64, B64, "f16")
        del Ad, Bd, C


def test_square_16384_bf16_sampled():
    say("16384 bf16")
    w = si.SQUARE_16384_BF16
    A, B = si.gen(**w)
    A64, B64 = si.f64(A), si.f64(B)
    n = w["M"]
    rows = np.random.default_rng(2).choice(n, 8, replace=False)
    ref = np.stack([oracle.gemm_rows(A64, B64, r, r + 1)[0] for r in rows])
    u = metrics.UNIT_ROUNDOFF["bf16"]
    res = {}
    # one level: the planner's choice at this size (the unfused path) and the
    # fused group kernel after a pre-pass
    for name, algo, kw in (("classic", "classic", {}), ("l1", "l1", {}), ("l1_fused", "l1", {"combine": "prepass"}),
                           ("l2", "l2", {})):
        say("16384", name)
        C = si.f64(planned(A, B, algo, **kw))
        res[name] = metrics.e_rel(C[rows], ref)
        assert res[name] <= 4 * u, (name, res[name])
        assert metrics.freivalds(C, A64, B64, seeds=(11,)) <= 4 * u
        del C
    assert max(res["l1"], res["l1_fused"], res["l2"]) <= 4 * res["classic"]


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
