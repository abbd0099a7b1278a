"""Host-side checks of liblcma.so that need no GPU: exported symbols, descriptor
validation (against the oracle's Brent check), argument validation, the cost
model's rules and the persistent schedule's coverage.

Planning uses ``num_cus`` so no device query happens; every invalid call must
return its status before touching the GPU.
"""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import complexity_half_precision_amd as L
import oracle
import descriptors as D
import seeded_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CUS = 256


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "lcma.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    keywords = {"if", "for", "while", "sizeof", "return"}
    return sorted({n for n in names if n not in keywords and (n.startswith("lcma_") or n.startswith("gemm_"))})


def test_library_binds_to_the_one_hip_runtime_in_the_process():
    # Imported before anything else, the binding must not pull in a second HIP
    # runtime beside torch's (that copy sees no device on a GPU host).
    import subprocess
    import sys
    code = ("import complexity_half_precision_amd, torch; "
            "print(len({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1"


def test_every_declared_symbol_is_exported():
    declared = _declared_functions()
    assert len(declared) >= 14
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert set(L.EXPORTED) <= set(declared)


def test_status_strings():
    for s in range(7):
        assert L.lcma_status_str(s) and "unknown" not in L.lcma_status_str(s)
    assert "unknown" in L.lcma_status_str(99)


# ---------------------------------------------------------------- descriptors

def test_builtin_tables_equal_the_oracle_tables():
    for lv, d in ((1, oracle.strassen()), (2, oracle.strassen2())):
        ms, ks, ns, rank, U, V, W = L.lcma_desc_builtin(lv)
        assert (ms, ks, ns, rank) == (d.ms, d.ks, d.ns, d.rank)
        assert np.array_equal(U, d.U) and np.array_equal(V, d.V) and np.array_equal(W, d.W)


def test_validator_agrees_with_oracle_brent_on_corruptions():
    ms, ks, ns, rank, U, V, W = L.lcma_desc_builtin(1)
    assert L.lcma_desc_validate(L.Desc(ms, ks, ns, U, V, W)) == L.OK
    rng = np.random.default_rng(3)
    for _ in range(40):
        tabs = [U.copy(), V.copy(), W.copy()]
        t = tabs[rng.integers(3)]
        r, c = rng.integers(t.shape[0]), rng.integers(t.shape[1])
        t[r, c] = (int(t[r, c]) + 2 + rng.integers(2)) % 3 - 1
        want = oracle.brent_violations(oracle.Desc(2, 2, 2, *tabs)) == 0
        got = L.lcma_desc_validate(L.Desc(2, 2, 2, *tabs)) == L.OK
        assert got == want
    # out-of-range coefficients and bad shapes
    bad = U.copy()
    bad[0, 0] = 100
    assert L.lcma_desc_validate(L.Desc(2, 2, 2, bad, V, W)) == L.E_BAD_DESCRIPTOR


def test_non_builtin_descriptors_plan_the_unfused_path():
    # a valid description that is not a built-in scheme: one level of it, unfused
    d = oracle.naive()
    desc = L.Desc(2, 2, 2, d.U, d.V, d.W)
    assert L.lcma_desc_validate(desc) == L.OK
    p = L.lcma_plan_ex(512, 512, 768, "f16", desc=desc, force="l1", num_cus=CUS)
    algo, ws, est = L.lcma_plan_info(p)
    assert algo == "l1" and est > 0
    # every combined operand written (8 per side), then 4 fp32 output blocks
    Mb, Nb, Kb = 256, 256, 384
    off_a, ld_a, _ = L.lcma_plan_operand(p, 0, 3)
    off_b, ld_b, _ = L.lcma_plan_operand(p, 1, 0)
    assert (off_a, ld_a) == (3 * Mb * Kb * 2, Kb) and ld_b == Nb and off_b == 8 * Mb * Kb * 2
    assert ws == 8 * Mb * Kb * 2 + 8 * Kb * Nb * 2 + 4 * Mb * Nb * 4
    with pytest.raises(L.LcmaError):
        L.lcma_plan_schedule(p)
    # automatic planning never picks it; two levels of it are not built
    p = L.lcma_plan_ex(512, 512, 512, "f16", desc=desc, force="auto", num_cus=CUS)
    assert L.lcma_plan_info(p)[0] == "classic"
    with pytest.raises(L.LcmaError) as e:
        L.lcma_plan_ex(512, 512, 512, "f16", desc=desc, force="l2", num_cus=CUS)
    assert e.value.status == L.E_UNSUPPORTED
    # more blocks per side than the unfused path takes
    big = oracle.naive(4, 4, 5)
    with pytest.raises(L.LcmaError) as e:
        L.lcma_plan_ex(512, 640, 512, "f16", desc=L.Desc(4, 4, 5, big.U, big.V, big.W), force="l1", num_cus=CUS)
    assert e.value.status == L.E_UNSUPPORTED


def test_winograd_variant_validates_in_library_and_oracle():
    d = oracle.Desc(2, 2, 2, D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W)
    assert oracle.brent_violations(d) == 0
    desc = L.Desc(2, 2, 2, D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W)
    assert L.lcma_desc_validate(desc) == L.OK
    # every single-entry change breaks it, in both checkers
    for T in range(3):
        for x in range(28):
            tabs = [D.WINOGRAD_U.copy(), D.WINOGRAD_V.copy(), D.WINOGRAD_W.copy()]
            t = tabs[T].reshape(-1)
            t[x] = (int(t[x]) + 2) % 3 - 1 if t[x] != 0 else 1
            bad_o = oracle.Desc(2, 2, 2, *tabs)
            assert oracle.brent_violations(bad_o) > 0
            assert L.lcma_desc_validate(L.Desc(2, 2, 2, *tabs)) == L.E_BAD_DESCRIPTOR
    p = L.lcma_plan_ex(1024, 1024, 1024, "bf16", desc=desc, force="l1", num_cus=CUS)
    assert L.lcma_plan_info(p)[0] == "l1"
    # the library's own copy of the table, written from the same formulas
    ms, ks, ns, rank, U, V, W = L.lcma_desc_winograd()
    assert (ms, ks, ns, rank) == (2, 2, 2, 7)
    assert np.array_equal(U, D.WINOGRAD_U) and np.array_equal(V, D.WINOGRAD_V) and np.array_equal(W, D.WINOGRAD_W)
    assert L.lcma_desc_validate(L.winograd_desc()) == L.OK
    assert L._lib_desc_winograd(None) == L.E_INVALID


def simulate_runs(runs, R, nblocks):
    """Replays a run schedule on symbolic products: each run's accumulators
    are a vector over the R products; block o receives fold[o] times them.
    Returns the per-block sums (an R x nblocks matrix) and the fp32 bytes
    the folds move per block element (2 for one fold, else 8k - 6)."""
    acc = np.zeros(R, np.int64)
    got = np.zeros((R, nblocks), np.int64)
    k = np.zeros(nblocks, np.int64)
    assert sorted(r[0] for r in runs) == list(range(R))
    for j, (prod, carry, fold) in enumerate(runs):
        assert carry in (0, 1, 2) and (j > 0 or carry == 0)
        acc = (np.zeros(R, np.int64) if carry == 0 else acc if carry == 1 else -acc)
        acc[prod] += 1
        for o in range(nblocks):
            if fold[o]:
                got[:, o] += fold[o] * acc
                k[o] += 1
    return got, int(sum(2 if c == 1 else 8 * c - 6 for c in k))


def test_unfused_run_schedules_rebuild_each_output_block():
    # The persistent unfused kernel's runs (order, carried accumulators,
    # folds) must sum to each output block's column of W.  Strassen's
    # pairing schedule moves 56 fp32 bytes per block element; Winograd's
    # searched one 32; the rank-8 block product (beyond the search) pairs
    # its products so each block takes one fold.
    n = 8192
    cases = [(None, oracle.strassen().W, 56),
             (L.Desc(2, 2, 2, D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W), D.WINOGRAD_W, 32)]
    d8 = oracle.naive()
    cases.append((L.Desc(2, 2, 2, d8.U, d8.V, d8.W), d8.W, 8))
    for desc, W, want in cases:
        if desc is None:
            p = L.lcma_plan_ex(n, n, n, "bf16", force="l1", combine="unfused", num_cus=CUS)
        else:
            p = L.lcma_plan_ex(n, n, n, "bf16", desc=desc, force="l1", num_cus=CUS)
        runs = L.lcma_plan_runs(p, 4)
        got, fold_bytes = simulate_runs(runs, W.shape[0], 4)
        assert np.array_equal(got, W.astype(np.int64)), runs
        assert fold_bytes == want, (fold_bytes, runs)


@pytest.mark.parametrize("seed", range(8))
def test_run_schedule_search_is_invariant_under_equivalent_descriptions(seed):
    # permuting the products and flipping signs changes the tables but not
    # the least fold bytes a schedule can reach: the search finds 56 for
    # every form of Strassen's scheme and 32 for every form of Winograd's,
    # and its runs rebuild the transformed W exactly
    for U0, V0, W0, want in ((oracle.strassen().U, oracle.strassen().V, oracle.strassen().W, 56),
                             (D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W, 32)):
        U, V, W = D.equivalent(U0, V0, W0, seed)
        d = oracle.Desc(2, 2, 2, U, V, W)
        assert oracle.brent_violations(d) == 0
        p = L.lcma_plan_ex(8192, 8192, 8192, "bf16", desc=L.Desc(2, 2, 2, U, V, W), force="l1", num_cus=CUS)
        got, fold_bytes = simulate_runs(L.lcma_plan_runs(p, 4), 7, 4)
        assert np.array_equal(got, W.astype(np.int64))
        assert fold_bytes == want, (seed, fold_bytes)


def test_winograd_schedule_meets_the_lower_bound():
    # A block written by one fold equals one snapshot, a signed prefix sum of
    # one chain of carried runs.  Every column of Winograd's W contains
    # product 1, which lies in one chain, so two single-fold blocks would
    # have nested supports; no two columns do.  Hence at most one block takes
    # one fold (2 bytes) and the others at least two (10 bytes each): 32 is
    # the least any schedule moves, and the searched schedule reaches it.
    W = D.WINOGRAD_W.astype(np.int64)
    sup = [set(np.nonzero(W[:, o])[0]) for o in range(4)]
    assert all(0 in s for s in sup)
    assert not any(a <= b for a, b in itertools.permutations(sup, 2))
    p = L.lcma_plan_ex(8192, 8192, 8192, "f16", desc=L.Desc(2, 2, 2, D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W),
                       force="l1", num_cus=CUS)
    assert simulate_runs(L.lcma_plan_runs(p, 4), 7, 4)[1] == 2 + 3 * 10


def test_run_schedules_exist_only_for_persistent_unfused_plans():
    cases = [L.lcma_plan_ex(4096, 4096, 4096, "bf16", force="classic", num_cus=CUS),
             L.lcma_plan_ex(4096, 4096, 4096, "bf16", force="l1", combine="prepass", num_cus=CUS),
             # 512 x 512 blocks: 4 positions, the per-product kernels
             L.lcma_plan_ex(1024, 1024, 1024, "bf16", force="l1", combine="unfused", num_cus=CUS)]
    for p in cases:
        with pytest.raises(L.LcmaError) as e:
            L.lcma_plan_runs(p, 4)
        assert e.value.status == L.E_INVALID
    p = L.lcma_plan_ex(8192, 8192, 8192, "bf16", force="l1", combine="unfused", num_cus=CUS)
    prod, carry = ctypes.c_int32(), ctypes.c_int32()
    fold = (ctypes.c_int8 * 4)()
    for j in (-1, 7):
        assert L._lib_plan_runs(p.handle, j, ctypes.byref(prod), ctypes.byref(carry), fold) == L.E_INVALID
    assert L._lib_plan_runs(p.handle, 0, None, ctypes.byref(carry), fold) == L.E_INVALID


def test_builtin_scheme_can_be_forced_unfused():
    p = L.lcma_plan_ex(1024, 1024, 1024, "bf16", force="l1", combine="unfused", num_cus=CUS)
    algo, ws, _ = L.lcma_plan_info(p)
    assert algo == "l1" and ws == 7 * 512 * 512 * 2 * 2 + 4 * 512 * 512 * 4
    with pytest.raises(L.LcmaError):
        L.lcma_plan_ex(1024, 1024, 1024, "bf16", force="l2", combine="unfused", num_cus=CUS)
    # padding changes only the shape: two levels stay unsupported unfused
    with pytest.raises(L.LcmaError) as e:
        L.lcma_plan_ex(1000, 1000, 1000, "bf16", force="l2", combine="unfused", num_cus=CUS)
    assert e.value.status == L.E_UNSUPPORTED


def test_plan_rejects_bad_descriptor():
    ms, ks, ns, rank, U, V, W = L.lcma_desc_builtin(1)
    V2 = V.copy()
    V2[3, 0] = 1
    with pytest.raises(L.LcmaError) as e:
        L.lcma_plan_ex(64, 64, 64, "f16", desc=L.Desc(2, 2, 2, U, V2, W), num_cus=CUS)
    assert e.value.status == L.E_BAD_DESCRIPTOR


# ---------------------------------------------------------------- planning

@pytest.mark.parametrize("args", [(-1, 4, 4), (4, -1, 4), (4, 4, -1), (1 << 40, 4, 4)])
def test_plan_rejects_bad_sizes(args):
    with pytest.raises(L.LcmaError) as e:
        L.lcma_plan_ex(*args, "f16", num_cus=CUS)
    assert e.value.status == L.E_INVALID


def test_plan_rejects_bad_enums():
    h = ctypes.c_void_p()
    opts = L.lcma_options(0, 0, 0, CUS, 0.0, 0.0)
    assert L._lib_plan_ex(8, 8, 8, 7, None, 0, ctypes.byref(opts), ctypes.byref(h)) == L.E_INVALID
    assert L._lib_plan_ex(8, 8, 8, 0, None, 9, ctypes.byref(opts), ctypes.byref(h)) == L.E_INVALID
    bad = L.lcma_options(7, 0, 0, CUS, 0.0, 0.0)
    assert L._lib_plan_ex(8, 8, 8, 0, None, 0, ctypes.byref(bad), ctypes.byref(h)) == L.E_INVALID
    assert L._lib_plan_ex(8, 8, 8, 0, None, 0, ctypes.byref(opts), None) == L.E_INVALID


@pytest.mark.parametrize("M,N,K,algo", [(511, 512, 512, "l1"), (512, 512, 8, "l1"), (512, 12, 512, "l1"),
                                        (512, 512, 100, "l2"), (1, 4096, 4096, "l1"), (1000, 1032, 520, "l2")])
def test_forced_lcma_on_unsplittable_shape_is_padded(M, N, K, algo):
    # zero-padded to multiples of (blocks per side) x 16, planned as that
    # product, cropped into C; the workspace holds the padded copies and the
    # padded plan's own workspace
    g = (2 if algo == "l1" else 4) * 16
    up = lambda x: -(-x // g) * g
    Mp, Np, Kp = up(M), up(N), up(K)
    # two levels on binary16 inputs exceed the 4x accuracy gate: opt in
    opt = int(algo == "l2")
    p = L.lcma_plan_ex(M, N, K, "f16", force=algo, num_cus=CUS, accuracy_optin=opt)
    chosen, ws, est = L.lcma_plan_info(p)
    inner = L.lcma_plan_ex(Mp, Np, Kp, "f16", force=algo, num_cus=CUS, accuracy_optin=opt)
    _, ws_in, est_in = L.lcma_plan_info(inner)
    assert chosen == algo
    assert ws >= 2 * (Mp * Kp + Kp * Np + Mp * Np) + ws_in
    assert est > est_in
    # the schedule and operands are the padded plan's
    if L.lcma_plan_info(inner)[0] == algo:
        try:
            assert L.lcma_plan_schedule(p)[0] == L.lcma_plan_schedule(inner)[0]
        except L.LcmaError:
            pass
    # a workspace smaller than reported fails before any device work
    assert L._lib_gemm(p.handle, 4096, K, 4096, N, 8192, N, 1 << 20, ws - 1, None) == L.E_WORKSPACE
    # automatic planning keeps classic for shapes that do not split
    assert L.lcma_plan_info(L.lcma_plan_ex(M, N, K, "f16", num_cus=CUS))[0] == "classic"


@pytest.mark.parametrize("M,N,K", [(100, 200, 300), (257, 13, 64), (1, 14337, 4096), (4100, 4100, 4100)])
def test_classic_plan_pads_k_and_n_to_multiples_of_8(M, N, K):
    p = L.lcma_plan_ex(M, N, K, "bf16", num_cus=CUS)
    chosen, ws, est = L.lcma_plan_info(p)
    assert chosen == "classic"
    Np, Kp = -(-N // 8) * 8, -(-K // 8) * 8
    inner = L.lcma_plan_ex(M, Np, Kp, "bf16", force="classic", num_cus=CUS)
    inner_ws = L.lcma_plan_info(inner)[1]                # a K split of the padded product, if any
    assert ws >= 2 * (M * Kp + Kp * Np + M * Np) + inner_ws
    assert est > L.lcma_plan_info(inner)[2]
    # aligned shapes need no workspace beyond a K split's, none with split="none"
    assert L.lcma_plan_info(L.lcma_plan_ex(M, Np, Kp, "bf16", num_cus=CUS))[1] == inner_ws
    assert L.lcma_plan_info(L.lcma_plan_ex(M, Np, Kp, "bf16", split="none", num_cus=CUS))[1] == 0
    # the two halves are for LCMA plans only
    assert L._lib_prepass(p.handle, 4096, K, 4096, N, 1 << 20, ws, None) == L.E_INVALID


def test_padding_is_only_for_the_built_in_schemes():
    # a description that is not built in runs one level of itself unfused and
    # needs M, K, N divisible by its block counts
    d = oracle.naive(2, 2, 2)
    desc = L.Desc(2, 2, 2, d.U, d.V, d.W)
    with pytest.raises(L.LcmaError) as e:
        L.lcma_plan_ex(511, 512, 512, "f16", desc=desc, force="l1", num_cus=CUS)
    assert e.value.status == L.E_UNSUPPORTED


def test_zero_sized_plans_are_valid():
    for M, N, K in ((0, 8, 8), (8, 0, 8), (8, 8, 0), (0, 0, 0)):
        p = L.lcma_plan_ex(M, N, K, "bf16", num_cus=CUS)
        assert L.lcma_plan_info(p)[0] == "classic"


def test_auto_picks_classic_for_skinny_and_sweep_shapes():
    # memory-bound shapes gain nothing from fewer multiplications
    for m in si.DECODE_MS:
        p = L.lcma_plan_ex(m, 14336, 4096, "bf16", num_cus=CUS)
        assert L.lcma_plan_info(p)[0] == "classic"
    for (M, N, K) in si.sweep_shapes():
        p = L.lcma_plan_ex(M, N, K, "f16", num_cus=CUS)
        algo, _, est = L.lcma_plan_info(p)
        F = 2.0 * M * N * K
        B = 2.0 * (M * K + K * N + M * N)
        if F / B < 2500e12 / 8000e9:     # below the ridge point
            assert algo == "classic", (M, N, K)


def test_estimates_are_monotone_in_each_dimension():
    # non-decreasing (below one round of tiles the time is one tile's), and
    # strictly larger across the whole range
    base = (2048, 2048, 2048)
    for d in range(3):
        est = []
        for v in (512, 1024, 2048, 4096, 8192):
            shp = list(base)
            shp[d] = v
            p = L.lcma_plan_ex(*shp, "bf16", force="classic", num_cus=CUS)
            est.append(L.lcma_plan_estimate(p, "classic"))
        assert all(b >= a for a, b in zip(est, est[1:])) and est[-1] > 2 * est[0]


def test_auto_never_picks_two_levels_for_binary16_inputs():
    for n in (4096, 8192, 16384):
        p = L.lcma_plan_ex(n, n, n, "f16", num_cus=CUS)
        assert L.lcma_plan_info(p)[0] != "l2"


def test_efficient_fused_kernel_makes_lcma_attractive_only_when_compute_bound():
    # With a fused kernel as efficient as the classic one, the 1/8 fewer
    # multiplications win on big squares but never on memory-bound shapes.
    p = L.lcma_plan_ex(16384, 16384, 16384, "bf16", num_cus=CUS, classic_eff=0.45, fused_eff=0.45)
    assert L.lcma_plan_info(p)[0] in ("l1", "l2")
    p = L.lcma_plan_ex(1, 14336, 4096, "bf16", num_cus=CUS, classic_eff=0.45, fused_eff=0.45)
    assert L.lcma_plan_info(p)[0] == "classic"
    # with a lower MFMA peak the ridge drops, and the same holds
    p = L.lcma_plan_ex(16384, 16384, 16384, "bf16", num_cus=CUS, peak_tflops=200.0, fused_eff=0.43)
    assert L.lcma_plan_info(p)[0] in ("l1", "l2")


def test_measured_efficiencies_pick_classic_on_big_squares():
    # the fused kernels as they stand sustain a much lower fraction of peak
    for n in (4096, 8192, 16384):
        p = L.lcma_plan_ex(n, n, n, "bf16", num_cus=CUS)
        assert L.lcma_plan_info(p)[0] == "classic", n


def test_auto_picks_the_unfused_one_level_from_24576_cubed():
    # with the default efficiencies the model's unfused estimate (pre-pass,
    # products at the classic rate, the run schedule's folds) falls 2% below
    # the classic one from 24576^3 on; measured on MI355X, the unfused one
    # level is 1.014-1.024x the classic kernel at 24576^3 and 32768^3 (the
    # bench's 32768^3 leg reports the pick and whether it agrees)
    for n, want in ((16384, "classic"), (24576, "l1"), (32768, "l1")):
        p = L.lcma_plan_ex(n, n, n, "bf16", num_cus=CUS)
        assert L.lcma_plan_info(p)[0] == want, n
        if want == "l1":
            # the unfused path, all products in one persistent launch
            assert len(L.lcma_plan_runs(p, 4)) == 7
    # the model treats binary16 inputs alike (one level keeps the input type
    # for its operands); that pick is the model's, not measured
    p = L.lcma_plan_ex(32768, 32768, 32768, "f16", num_cus=CUS)
    assert L.lcma_plan_info(p)[0] == "l1"


def test_efficiency_options_are_validated():
    for kw in ({"classic_eff": -0.1}, {"classic_eff": 1.5}, {"fused_eff": 2.0}, {"fused_eff": float("nan")}):
        with pytest.raises(L.LcmaError):
            L.lcma_plan_ex(512, 512, 512, "f16", num_cus=CUS, **kw)


def test_workspace_layout_of_one_level_plan():
    M = N = K = 4096
    p = L.lcma_plan_ex(M, N, K, "bf16", force="l1", num_cus=CUS)
    algo, ws, _ = L.lcma_plan_info(p)
    assert algo == "l1"
    blk = (M // 2) * (K // 2) * 2
    # 5 combined operands per side are written, singletons are read in place
    offs_a = [L.lcma_plan_operand(p, 0, r)[0] for r in range(7)]
    offs_b = [L.lcma_plan_operand(p, 1, r)[0] for r in range(7)]
    assert sum(o >= 0 for o in offs_a) == 5 and sum(o >= 0 for o in offs_b) == 5
    assert [o < 0 for o in offs_a] == [False, False, True, True, False, False, False]
    assert [o < 0 for o in offs_b] == [False, True, False, False, True, False, False]
    assert ws >= 10 * blk
    # operand regions do not overlap
    starts = sorted(o for o in offs_a + offs_b if o >= 0)
    assert all(b - a >= blk for a, b in zip(starts, starts[1:]))


def test_unfused_plan_packs_its_a_operands_only_on_whole_tiles():
    # one persistent launch on whole 256 x 256 tiles: every combined A operand
    # is tile-packed (ld 0); the B operands stay row-major, their rows padded
    # by 64 elements in one persistent launch (one launch per product: ld Nb)
    for (M, N, K), packed, group in (((8192, 8192, 512), True, True), ((8192, 8192, 528), False, True),
                                     ((8192, 8000, 512), False, True), ((2048, 2048, 512), False, False)):
        p = L.lcma_plan_ex(M, N, K, "bf16", force="l1", combine="unfused", num_cus=CUS)
        assert L.lcma_plan_info(p)[0] == "l1"
        ldb = N // 2 + (64 if group else 0)
        offs = []
        for r in range(7):
            off_a, ld_a, _ = L.lcma_plan_operand(p, 0, r)
            off_b, ld_b, _ = L.lcma_plan_operand(p, 1, r)
            assert off_a >= 0 and off_b >= 0
            assert ld_a == (0 if packed else K // 2), (M, N, K, ld_a)
            assert ld_b == ldb, (M, N, K, ld_b)
            offs.append(off_b)
        assert [o - offs[0] for o in offs] == [r * (K // 2) * ldb * 2 for r in range(7)]


def test_decode_shaped_classic_plans_take_the_k_split_workspace():
    # up to 64 rows with K long against the number of 128-column strips:
    # S = 2, 4 or 8 workgroups per strip, each an fp32 partial tile of 64 x
    # 128 (32 KiB; 32 x 128, 16 KiB, up to 32 rows)
    for (M, N, K), strips, S in (((64, 4096, 14336), 32, 8), ((33, 8192, 8192), 64, 4), ((48, 104, 8200), 1, 8),
                                 ((64, 14336, 10240), 112, 2), ((40, 8192, 14336), 64, 4), ((64, 2048, 4096), 16, 8),
                                 ((64, 1024, 14336), 8, 8), ((1, 1024, 14336), 8, 8), ((32, 1024, 12288), 8, 8),
                                 ((1, 4096, 14336), 32, 8), ((16, 8192, 8192), 64, 4), ((8, 8192, 14336), 64, 4),
                                 ((32, 2048, 4096), 16, 8), ((17, 1032, 12288), 9, 8), ((1, 1024, 8192), 8, 8),
                                 ((32, 4096, 4096), 32, 8), ((64, 4096, 8184), 32, 8), ((1, 1024, 2048), 8, 8),
                                 ((64, 1024, 4088), 8, 8), ((8, 8192, 8192), 64, 4), ((1, 2048, 4096), 16, 8),
                                 ((40, 4096, 12280), 32, 8), ((64, 2048, 2048), 16, 4), ((1, 4096, 2048), 32, 4),
                                 ((1, 8192, 4096), 64, 4), ((64, 28672, 4096), 224, 2), ((32, 14336, 14336), 112, 2),
                                 ((48, 9000, 8192), 71, 2)):
        p = L.lcma_plan_ex(M, N, K, "bf16", force="classic", num_cus=CUS)
        algo, ws, _ = L.lcma_plan_info(p)
        assert algo == "classic"
        part = 32768 if M > 32 else 16384
        assert ws == -(-(strips * S * part) // 256) * 256, (M, N, K, ws)
    for M, N, K in ((65, 4096, 2040), (64, 14336, 4096), (64, 8200, 4096), (64, 4096, 2040), (64, 1024, 2040),
                    (1, 8, 8), (8, 8192, 4088), (16, 8320, 14336), (1, 14336, 4096), (32, 4104, 4088),
                    (1, 1024, 2040), (1, 28672, 14336), (64, 2048, 2040), (32, 14336, 8192), (64, 16384, 4096)):
        p = L.lcma_plan_ex(M, N, K, "bf16", force="classic", num_cus=CUS)
        assert L.lcma_plan_info(p)[1] == 0, (M, N, K)


def test_few_tile_classic_plans_split_k_into_fp32_planes():
    # beyond 64 rows, 128 x 128 tiles filling at most half the compute
    # units with K >= 4096: S planes of M x N fp32 (tiles x S <= CUs, 768 of
    # K per piece at least)
    for (M, N, K), S in (((4096, 256, 8192), 4), ((256, 8192, 4096), 2), ((256, 256, 16384), 8),
                         ((128, 14336, 4096), 2), ((1000, 264, 8200), 8), ((300, 136, 16392), 8),
                         ((1024, 1024, 8192), 4), ((65, 128, 4096), 4), ((4096, 256, 4096), 4),
                         ((1024, 512, 6144), 8), ((512, 1024, 4096), 4)):
        p = L.lcma_plan_ex(M, N, K, "bf16", force="classic", num_cus=CUS)
        algo, ws, _ = L.lcma_plan_info(p)
        assert algo == "classic"
        assert ws == -(-(S * M * N * 4) // 256) * 256, (M, N, K, ws)
    # full rounds of tiles, short K, or not multiples of 8 (those pad first)
    for M, N, K in ((2048, 2048, 8192), (4096, 4096, 4096), (4096, 256, 2048), (1024, 1024, 4088), (1024, 1024, 4080),
                    (8192, 8192, 8192)):
        p = L.lcma_plan_ex(M, N, K, "bf16", force="classic", num_cus=CUS)
        assert L.lcma_plan_info(p)[1] == 0, (M, N, K)


def test_multi_round_classic_plans_split_the_tail_round():
    # 256 x 256 grids of more than one round: the T tiles of the last round
    # split K into S compact fp32 tiles each (S * T * 256 KiB)
    for (M, N, K), T, S in (((4104, 4104, 4104), 33, 4), ((3328, 5120, 8192), 4, 8), ((7168, 7168, 7168), 16, 4),
                            ((6144, 6144, 12288), 64, 4), ((2304, 7424, 4096), 5, 4)):
        p = L.lcma_plan_ex(M, N, K, "bf16", force="classic", num_cus=CUS)
        assert L.lcma_plan_info(p)[1] == S * T * 256 * 256 * 4, (M, N, K)
    for M, N, K in ((4096, 4096, 4096), (16384, 16384, 16384), (10240, 10240, 4096), (6144, 6144, 6144),
                    (5120, 5120, 8192), (4104, 4104, 2048)):
        p = L.lcma_plan_ex(M, N, K, "bf16", force="classic", num_cus=CUS)
        assert L.lcma_plan_info(p)[1] == 0, (M, N, K)
    # the cost model (which models the unsplit classic kernels) keeps classic
    # on these shapes, where classic runs the tail split and LCMA is slower
    for M, N, K in ((7168, 7168, 7168), (6144, 6144, 12288), (4104, 4104, 4104), (3328, 5120, 8192),
                    (8448, 8192, 8192), (2304, 7424, 4096)):
        assert L.lcma_plan_info(L.lcma_plan_ex(M, N, K, "bf16", num_cus=CUS))[0] == "classic", (M, N, K)
    # split="none": no K split, no workspace
    for M, N, K in ((3328, 5120, 8192), (4096, 256, 8192), (1, 4096, 14336)):
        assert L.lcma_plan_info(L.lcma_plan_ex(M, N, K, "bf16", force="classic", split="none", num_cus=CUS))[1] == 0


def test_ragged_decode_plans_pad_then_split():
    # K or N not a multiple of 8: the plan pads A, B and C into its workspace
    # and runs the padded product's plan after them, here a K split
    up = lambda x: -(-x // 256) * 256
    for (M, N, K), S in (((3, 1030, 14330), 8), ((50, 2050, 6150), 8)):
        Np, Kp = -(-N // 8) * 8, -(-K // 8) * 8
        strips = -(-Np // 128)
        inner = L.lcma_plan_info(L.lcma_plan_ex(M, Np, Kp, "bf16", force="classic", num_cus=CUS))[1]
        assert inner == up(strips * S * (16384 if M <= 32 else 32768))
        ws = L.lcma_plan_info(L.lcma_plan_ex(M, N, K, "bf16", force="classic", num_cus=CUS))[1]
        assert ws == up(up(up(M * Kp * 2) + Kp * Np * 2) + M * Np * 2) + inner, (M, N, K, ws)


def test_bf16_two_level_writes_every_operand_in_binary16():
    p = L.lcma_plan_ex(4096, 4096, 4096, "bf16", force="l2", num_cus=CUS)
    for r in range(49):
        off, ld, dt = L.lcma_plan_operand(p, 0, r)
        assert off >= 0 and dt == L.F16


# ---------------------------------------------------------------- schedule

def _check_schedule(plan, R, expect_split):
    items, order = L.lcma_plan_schedule(plan)
    assert sorted(order[:R]) == list(range(R))
    pieces = {}
    for (w, g, p0, p1, slot) in items:
        assert 0 <= p0 < p1 <= R
        pieces.setdefault(g, []).append((p0, p1, slot, w))
    G = len(pieces)
    for g, ps in pieces.items():
        covered = sorted(x for (p0, p1, _, _) in ps for x in range(p0, p1))
        assert covered == list(range(R)), g         # every product of every group exactly once
        assert len(ps) <= 2                        # at most a 2-way split
        if len(ps) == 2:
            assert ps[0][2] == ps[1][2] >= 0        # both pieces share one fix-up slot
        else:
            assert ps[0][2] == -1
    slots = [ps[0][2] for ps in pieces.values() if len(ps) == 2]
    assert len(slots) == len(set(slots))
    n_split = len(slots)
    if expect_split == "none":
        assert n_split == 0
    elif expect_split == "all":
        assert n_split == G
    return items, G, n_split


@pytest.mark.parametrize("M,cus", [(4096, 256), (4096, 240), (3072, 256), (2560, 256), (512, 256),
                                   (4096, 7), (1024, 1), (6144, 304)])
def test_schedule_covers_every_product_once(M, cus):
    p = L.lcma_plan_ex(M, M, M, "f16", force="l1", num_cus=cus)
    items, G, n_split = _check_schedule(p, 7, None)
    # the tail is split only when it fits twice into the workers
    T = G % cus
    assert n_split == (T if (T > 0 and 2 * T <= cus) else 0)
    # makespan in products: full rounds of 7 plus a split tail of <= 4
    load = {}
    for (w, g, p0, p1, slot) in items:
        load[w] = load.get(w, 0) + (p1 - p0)
    unsplit = 7 * -(-G // cus)
    assert max(load.values()) <= unsplit


@pytest.mark.parametrize("split", ["none", "all"])
def test_forced_split_modes(split):
    p = L.lcma_plan_ex(1024, 1024, 1024, "f16", force="l1", split=split, num_cus=256)
    _check_schedule(p, 7, split)
    # two levels: the schedule of one outer launch (7 inner products per
    # group tile over the M/4 x N/4 blocks), shared by all 7 launches
    p2 = L.lcma_plan_ex(1024, 1024, 1024, "bf16", force="l2", split=split, num_cus=256)
    _, G2, _ = _check_schedule(p2, 7, split)
    assert G2 == (256 // 128) ** 2
    # all 49 products in one group on chip
    p3 = L.lcma_plan_ex(1024, 1024, 1024, "bf16", force="l2", split=split, combine="l2_on_chip", num_cus=256)
    _, G3, _ = _check_schedule(p3, 49, split)
    assert G3 == (256 // 64) ** 2


def test_split_pieces_of_a_group_sit_on_adjacent_workers():
    # 2560^3 one-level: 10 x 10 = 100 groups on 256 workers -> all 100 split
    p = L.lcma_plan_ex(2560, 2560, 2560, "f16", force="l1", num_cus=256)
    items, G, n_split = _check_schedule(p, 7, None)
    assert G == 100 and n_split == 100
    by_group = {}
    for (w, g, p0, p1, slot) in items:
        by_group.setdefault(g, []).append((w, p0))
    for g, ws in by_group.items():
        (w0, a), (w1, b) = sorted(ws, key=lambda x: x[1])
        assert a == 0 and w1 == w0 + 1 and w0 % 2 == 0   # first half on even, second on odd worker


def _xcd_halves(items):
    halves = {}
    for (w, g, p0, p1, slot) in items:
        if slot >= 0:
            halves.setdefault(w % 8, set()).add(p0 == 0)
    return halves


@pytest.mark.parametrize("M,N", [(2560, 2560), (4096, 5120)])
def test_plain_order_is_a_valid_schedule_that_mixes_halves(M, N):
    # 2560^2: 100 groups, all split; 4096 x 5120: 320 groups, a split tail of 64
    pa = L.lcma_plan_ex(M, N, 1024, "bf16", force="l1", num_cus=256)
    pp = L.lcma_plan_ex(M, N, 1024, "bf16", force="l1", num_cus=256, order="plain")
    ia, Ga, na = _check_schedule(pa, 7, None)
    ip, Gp, nq = _check_schedule(pp, 7, None)
    assert (Ga, na) == (Gp, nq) and na > 0
    T = na
    # same pieces, only placed differently
    assert sorted(x[1:4] for x in ia) == sorted(x[1:4] for x in ip)
    # locality order: every XCD runs one kind of half; plain: every XCD runs both
    assert all(len(h) == 1 for h in _xcd_halves(ia).values())
    assert len(_xcd_halves(ip)) == 8 and all(len(h) == 2 for h in _xcd_halves(ip).values())
    # plain placement: first halves of tail group t on worker t, second on T + t
    for (w, g, p0, p1, slot) in ip:
        if slot >= 0:
            assert w == (slot if p0 == 0 else T + slot)
    # plain order of whole groups: row-major, worker w takes groups w, w + P, ...
    for (w, g, p0, p1, slot) in ip:
        if slot < 0:
            assert g % 256 == w


def test_one_level_combine_follows_the_cost_model():
    # Left to the planner, one level of the built-in scheme runs the unfused
    # path where its estimate is lower (large blocks) and the fused group
    # kernel below; an explicit split or order keeps the fused kernel.
    def fused(plan):
        try:
            L.lcma_plan_schedule(plan)
            return True
        except L.LcmaError:
            return False
    for n, want_fused in ((4096, True), (6144, True), (8192, False), (16384, False)):
        p = L.lcma_plan_ex(n, n, n, "bf16", force="l1", num_cus=256)
        assert fused(p) == want_fused, n
        pf = L.lcma_plan_ex(n, n, n, "bf16", force="l1", combine="prepass", num_cus=256)
        pu = L.lcma_plan_ex(n, n, n, "bf16", force="l1", combine="unfused", num_cus=256)
        assert fused(pf) and not fused(pu)
        assert L.lcma_plan_info(p)[2] == min(L.lcma_plan_info(pf)[2], L.lcma_plan_info(pu)[2]) or want_fused
    p = L.lcma_plan_ex(16384, 16384, 16384, "bf16", force="l1", split="none", num_cus=256)
    assert fused(p)
    p = L.lcma_plan_ex(16384, 16384, 16384, "bf16", force="l1", order="plain", num_cus=256)
    assert fused(p)


def test_invalid_order_is_rejected():
    with pytest.raises(L.LcmaError):
        L.lcma_plan_ex(1024, 1024, 1024, "f16", force="l1", num_cus=256, order=2)


# ---------------------------------------------------------------- call validation (no device work)

def test_invalid_calls_fail_before_touching_the_device():
    p = L.lcma_plan_ex(512, 512, 512, "f16", force="l1", num_cus=CUS)
    _, ws, _ = L.lcma_plan_info(p)
    assert ws > 0
    # null operands
    assert L._lib_gemm(p.handle, None, 512, 4096, 512, 8192, 512, 1 << 20, ws, None) == L.E_INVALID
    # leading dimension too small
    assert L._lib_gemm(p.handle, 4096, 511, 4096, 512, 8192, 512, 1 << 20, ws, None) == L.E_INVALID
    # workspace missing / too small / misaligned
    assert L._lib_gemm(p.handle, 4096, 512, 4096, 512, 8192, 512, None, 0, None) == L.E_WORKSPACE
    assert L._lib_gemm(p.handle, 4096, 512, 4096, 512, 8192, 512, 1 << 20, ws - 1, None) == L.E_WORKSPACE
    assert L._lib_gemm(p.handle, 4096, 512, 4096, 512, 8192, 512, (1 << 20) + 16, ws, None) == L.E_WORKSPACE
    # misaligned operand on an LCMA plan
    assert L._lib_gemm(p.handle, 4098, 512, 4096, 512, 8192, 512, 1 << 20, ws, None) == L.E_UNSUPPORTED
    assert L._lib_gemm(p.handle, 4096, 516, 4096, 512, 8192, 512, 1 << 20, ws, None) == L.E_UNSUPPORTED
    # classic without a plan
    assert L._lib_classic(-1, 8, 8, 0, 16, 8, 16, 8, 16, 8, None) == L.E_INVALID
    assert L._lib_classic(8, 8, 8, 5, 16, 8, 16, 8, 16, 8, None) == L.E_INVALID
    assert L._lib_classic(8, 8, 8, 0, None, 8, 16, 8, 16, 8, None) == L.E_INVALID
    assert L._lib_classic(8, 8, 8, 0, 16, 8, 16, 8, 16, 7, None) == L.E_INVALID
    # empty products need no pointers
    assert L._lib_classic(0, 8, 8, 0, None, 8, None, 8, None, 8, None) == L.OK
    assert L._lib_classic(8, 0, 8, 0, None, 8, None, 8, None, 8, None) == L.OK
    # plan-less calls on non-LCMA plans
    pc = L.lcma_plan_ex(512, 512, 512, "f16", force="classic", num_cus=CUS)
    assert L._lib_prepass(pc.handle, 4096, 512, 4096, 512, 1 << 20, 0, None) == L.E_INVALID
    assert L._lib_plan_operand(pc.handle, 0, 0, None, None, None) == L.E_INVALID


# ---------------------------------------------------------------- combine at load

def test_combine_at_load_plans_one_level_without_a_workspace():
    p = L.lcma_plan_ex(1024, 1024, 1024, "bf16", force="l1", combine="at_load", split="none", num_cus=CUS)
    chosen, ws, est = L.lcma_plan_info(p)
    assert chosen == "l1" and ws == 0 and est > 0
    # no combined operand is ever written
    with pytest.raises(L.LcmaError) as e:
        L.lcma_plan_operand(p, 0, 0)
    assert e.value.status == L.E_INVALID
    # whole groups only, each on one worker, every group once
    items, order = L.lcma_plan_schedule(p)
    assert all(it[4] == -1 and (it[2], it[3]) == (0, 7) for it in items)
    assert sorted(it[1] for it in items) == list(range(len(items)))
    assert sorted(order[:7]) == list(range(7))
    # the same in binary16, and a forced padded shape wraps it like any L1 plan
    p = L.lcma_plan_ex(512, 512, 512, "f16", force="l1", combine="at_load", split="none", num_cus=CUS)
    assert L.lcma_plan_info(p)[:2] == ("l1", 0)
    # a partial last round is split like the pre-pass path's: two pieces per
    # tail group, partials and counters in the workspace
    pa = L.lcma_plan_ex(2560, 2560, 2560, "bf16", force="l1", combine="at_load", num_cus=256)
    pp = L.lcma_plan_ex(2560, 2560, 2560, "bf16", force="l1", combine="prepass", num_cus=256)
    items_a, _ = L.lcma_plan_schedule(pa)
    items_p, _ = L.lcma_plan_schedule(pp)
    assert items_a == items_p and any(it[4] >= 0 for it in items_a)
    ws_a, ws_p = L.lcma_plan_info(pa)[1], L.lcma_plan_info(pp)[1]
    assert 0 < ws_a < ws_p
    p = L.lcma_plan_ex(500, 520, 260, "f16", force="l1", combine="at_load", num_cus=CUS)
    assert L.lcma_plan_info(p)[0] == "l1"
    with pytest.raises(L.LcmaError):
        L.lcma_plan_operand(p, 0, 0)


def test_combine_at_load_rejects_what_it_does_not_build():
    for kw in (dict(force="l2"), dict(force="l1", bf16_ops_f16=1)):
        with pytest.raises(L.LcmaError) as e:
            L.lcma_plan_ex(1024, 1024, 1024, "bf16", combine="at_load", num_cus=CUS, **kw)
        assert e.value.status == L.E_UNSUPPORTED, kw
    d = oracle.naive(2, 2, 2)
    with pytest.raises(L.LcmaError) as e:
        L.lcma_plan_ex(512, 512, 512, "f16", desc=L.Desc(2, 2, 2, d.U, d.V, d.W), force="l1", combine="at_load",
                       num_cus=CUS)
    assert e.value.status == L.E_UNSUPPORTED
    # binary16 inputs have binary16 operands either way
    p = L.lcma_plan_ex(512, 512, 512, "f16", force="l1", combine="at_load", bf16_ops_f16=1, num_cus=CUS)
    assert L.lcma_plan_info(p)[0] == "l1"


def test_combine_at_load_estimate_has_no_prepass():
    n = 4096
    pa = L.lcma_plan_ex(n, n, n, "bf16", force="l1", combine="at_load", num_cus=256, fused_eff=0.31)
    pp = L.lcma_plan_ex(n, n, n, "bf16", force="l1", combine="prepass", num_cus=256, fused_eff=0.31)
    # same kernel efficiency: dropping the pre-pass can only shorten the estimate
    assert L.lcma_plan_info(pa)[2] < L.lcma_plan_info(pp)[2]


# ---------------------------------------------------------------- accuracy gate, limits, header

def test_two_level_plans_beyond_the_accuracy_gate_need_an_opt_in():
    # Two levels with combined operands rounded to the input type carry about
    # 5.8-5.9x the classic kernel's normwise error (see
    # test_oracle.py::test_two_level_error_ratios_from_the_scheme_evaluation),
    # beyond the 4x the library promises: refused unless opted in.
    for kw in (dict(), dict(combine="l2_on_chip")):
        with pytest.raises(L.LcmaError) as e:
            L.lcma_plan_ex(1024, 1024, 1024, "f16", force="l2", num_cus=CUS, **kw)
        assert e.value.status == L.E_UNSUPPORTED, kw
        p = L.lcma_plan_ex(1024, 1024, 1024, "f16", force="l2", num_cus=CUS, accuracy_optin=1, **kw)
        assert L.lcma_plan_info(p)[0] == "l2"
    # a shape that is padded first is refused the same way
    with pytest.raises(L.LcmaError) as e:
        L.lcma_plan_ex(1000, 1032, 520, "f16", force="l2", num_cus=CUS)
    assert e.value.status == L.E_UNSUPPORTED
    # bfloat16 inputs: bfloat16 operands need the opt-in, binary16 operands (the default) do not
    with pytest.raises(L.LcmaError) as e:
        L.lcma_plan_ex(1024, 1024, 1024, "bf16", force="l2", bf16_ops_f16=-1, num_cus=CUS)
    assert e.value.status == L.E_UNSUPPORTED
    for kw in (dict(bf16_ops_f16=-1, accuracy_optin=1), dict(), dict(bf16_ops_f16=1)):
        assert L.lcma_plan_info(L.lcma_plan_ex(1024, 1024, 1024, "bf16", force="l2", num_cus=CUS, **kw))[0] == "l2"
    # one level (about 2.8x) never needs it
    for dt in ("f16", "bf16"):
        for ops in (-1, 0, 1):
            assert L.lcma_plan_info(L.lcma_plan_ex(1024, 1024, 1024, dt, force="l1", bf16_ops_f16=ops,
                                                   num_cus=CUS))[0] == "l1"
    with pytest.raises(L.LcmaError) as e:
        L.lcma_plan_ex(64, 64, 64, "f16", num_cus=CUS, accuracy_optin=2)
    assert e.value.status == L.E_INVALID
    # the planner never picks a gated form by itself, even when it estimates it fastest
    for (M, N, K) in si.sweep_shapes() + [(16384, 16384, 16384)]:
        p = L.lcma_plan_ex(M, N, K, "f16", num_cus=CUS, classic_eff=0.01)
        assert L.lcma_plan_info(p)[0] != "l2", (M, N, K)


def test_leading_dimension_limits_are_refused_at_plan_time():
    big = 1 << 21
    for (M, N, K, algo) in [(8, big, 64, "auto"), (8, 64, big, "classic"),     # lda >= K, ldb >= N
                            (8, big - 3, 64, "auto"), (8, 64, big - 5, "auto"),  # classic padding to 8
                            (64, 64, big - 1, "l1"), (64, big - 30, 64, "l1"),    # L1 padding to 32
                            (64, 64, big - 60, "l2")]:                           # L2 padding to 64
        with pytest.raises(L.LcmaError) as e:
            L.lcma_plan_ex(M, N, K, "bf16", force=algo, num_cus=CUS)
        assert e.value.status == L.E_UNSUPPORTED, (M, N, K, algo)
    assert L.lcma_plan_info(L.lcma_plan_ex(8, big - 8, 64, "bf16", num_cus=CUS))[0] == "classic"
    # a split block's leading dimension must stay below the limit too: AUTO keeps classic
    p = L.lcma_plan_ex(1 << 20, 64, big - 64, "bf16", num_cus=CUS)
    assert L.lcma_plan_info(p)[0] == "classic"


def test_noalloc_entry_point_refuses_before_any_device_call():
    assert L._lib_gemm_noalloc(None, 4096, 64, 4096, 64, 4096, 64, None) == L.E_INVALID
    p = L.lcma_plan_ex(8192, 8192, 8192, "bf16", force="l1", combine="prepass", num_cus=CUS)
    assert L.lcma_plan_info(p)[1] > L.SCRATCH_BYTES
    # fake addresses: the call must return before touching them
    assert L._lib_gemm_noalloc(p.handle, 4096, 8192, 8192, 8192, 16384, 8192, None) == L.E_WORKSPACE
    text = open(os.path.join(ROOT, "include", "lcma.h")).read()
    assert re.search(r"#define LCMA_SCRATCH_BYTES \(\(size_t\)64 << 20\)", text) and L.SCRATCH_BYTES == 64 << 20


# The calls the boundary exports and the passage each is defined by.
SOURCED = ["lcma_desc_builtin", "lcma_desc_validate", "lcma_plan", "lcma_plan_info", "lcma_plan_estimate",
           "lcma_gemm", "lcma_prepass", "lcma_plan_operand", "lcma_plan_schedule", "gemm_classic",
           "lcma_plan_destroy", "lcma_status_str"]


def test_each_boundary_declaration_cites_its_source():
    text = open(os.path.join(ROOT, "include", "lcma.h")).read()
    for name in SOURCED:
        m = re.search(r"^[a-z_ ]+\*?\s*\b" + name + r"\(", text, flags=re.M)
        assert m, name
        # the comment block that ends right above the declaration (or above its group)
        before = text[:m.start()]
        end = before.rfind("*/")
        start = before.rfind("/*", 0, end)
        between = before[end + 2:]
        assert between.count(";") <= 1, (name, "comment is not next to the declaration")
        block = before[start:end]
        src = re.search(r"Source:(.*)", block, flags=re.S)
        assert src, name
        cited = src.group(1)
        assert re.search(r"\[(FG|CL2|KP)\] \"[^\"]+\"", cited) or "none on the pages" in cited, name


def test_binding_refuses_host_tensors_and_short_buffers():
    import torch
    p = L.lcma_plan_ex(64, 64, 64, "f16", force="classic", num_cus=CUS)
    A = torch.zeros((64, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="device tensor"):
        L.lcma_gemm(p, A, A, A)
    with pytest.raises(ValueError, match="device tensor"):
        L.gemm_classic(A, A, A)
    with pytest.raises(ValueError, match="device tensor"):
        L.lcma_gemm_noalloc(p, A, A, A)
    with pytest.raises(ValueError, match="device tensor"):
        L.lcma_gemm_prepared(p, A, A, A)        # checked once, when the call is prepared


def test_measurement_entry_points_check_arguments_first():
    assert L._lib_measure_mfma(None, 1, 1, L.BF16, None) == L.E_INVALID
    assert L._lib_measure_mfma(4096, 0, 1, L.BF16, None) == L.E_INVALID
    assert L._lib_measure_mfma(4096, 1, 0, L.BF16, None) == L.E_INVALID
    assert L._lib_measure_mfma(4096, 1, 1, 7, None) == L.E_INVALID
    assert L._lib_measure_copy(None, None, 0, None) == L.OK            # nothing to copy
    assert L._lib_measure_copy(None, 4096, 16, None) == L.E_INVALID
    assert L._lib_measure_copy(4104, 8192, 16, None) == L.E_UNSUPPORTED   # misaligned source
    assert L._lib_measure_copy(4096, 8192, 24, None) == L.E_UNSUPPORTED   # not a multiple of 16 bytes
    assert L._lib_measure_read(None, 0, None, None) == L.OK               # nothing to read
    assert L._lib_measure_read(None, 16, 4096, None) == L.E_INVALID
    assert L._lib_measure_read(4096, 16, None, None) == L.E_INVALID
    assert L._lib_measure_read(4104, 16, 4096, None) == L.E_UNSUPPORTED   # misaligned source
    assert L._lib_measure_read(4096, 24, 4096, None) == L.E_UNSUPPORTED   # not a multiple of 16 bytes
    import torch
    with pytest.raises(ValueError, match="device tensors"):
        L.lcma_measure_read(torch.zeros(16, dtype=torch.uint8), torch.zeros(1, dtype=torch.int32))
