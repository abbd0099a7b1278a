"""The roofline cost model pinned to values computed by hand.

The model (FalconGEMM write-up, section "从缓存重排到 Cost Model": a
roofline-like estimate from FLOPs, bytes and the device's peak and bandwidth;
"Kernel 与性能" notes, section "Roofline") is written out here from its
definition in ``include/lcma.h`` (lcma_plan_estimate), independently of the
library's code:

  per kernel: max(F / (eta * peak * q), B / (0.8 * bw), F / (I_tile * bw_L2 * q)) + 4 us
  bw_L2 = 8 * 2048 B * 2.4 GHz, I_tile = BM * BN / (BM + BN), q = wave-quantisation
  efficiency (work units / P) / (rounds needed); a split tail counts as half a round.

Each case fixes peak, bandwidth and efficiencies, so a wrong byte term (for
example 7 written blocks instead of 5), a wrong tile, a wrong quantisation or
a wrong efficiency changes the estimate and fails the test.
"""
import math

import pytest

import complexity_half_precision_amd as L
import descriptors as D

P = 256
PEAK = 2000e12          # peak_tflops = 2000
BW = 6000e9             # hbm_gbps = 6000
ETA_C, ETA_F = 0.5, 0.25
BW_L2 = 8 * 2048 * 2.4e9
LAUNCH = 4e-6
OPTS = dict(num_cus=P, peak_tflops=2000.0, hbm_gbps=6000.0, classic_eff=ETA_C, fused_eff=ETA_F)


def kernel(F, B, itile, q, eta):
    return max(F / (eta * PEAK * q), B / (0.8 * BW), F / (itile * BW_L2 * q)) + LAUNCH


def close(a, b):
    return math.isclose(a, b, rel_tol=1e-9)


def test_classic_4096_cubed():
    # 256 x 256 tiles: 256 tiles on 256 CUs, one full round (q = 1)
    n = 4096
    F, B = 2.0 * n ** 3, 2.0 * 3 * n * n
    want = kernel(F, B, 256 * 256 / 512, 1.0, ETA_C)
    assert close(want, 137.438953472e-6 + 4e-6)          # compute-bound: F / (0.5 * 2 PFLOP/s)
    p = L.lcma_plan_ex(n, n, n, "bf16", force="classic", **OPTS)
    assert close(L.lcma_plan_estimate(p, "classic"), want)


def test_classic_2560_cubed_takes_the_128_tile():
    # 100 tiles of 256^2 need one round, 400 tiles of 128^2 two rounds; a round
    # of 128^2 tiles counts 0.4 of a 256^2 round, so 0.8 < 1 picks 128 x 128,
    # which sustains 0.7 of the classic efficiency; q = 400 / (2 * 256)
    n = 2560
    F, B = 2.0 * n ** 3, 2.0 * 3 * n * n
    q = 400 / (2 * 256)
    want = kernel(F, B, 128 * 128 / 256, q, 0.7 * ETA_C)
    p = L.lcma_plan_ex(n, n, n, "bf16", force="classic", **OPTS)
    assert close(L.lcma_plan_estimate(p, "classic"), want)


def test_one_level_with_prepass_4096_cubed():
    # pre-pass: read A and B once, write 5 combined operands per side (the two
    # single-block operands per side are read in place: bfloat16 operands)
    n, h = 4096, 2048
    pre_bytes = 2.0 * (n * n + n * n) + 2.0 * (5 * h * h + 5 * h * h)
    assert pre_bytes == 150994944.0
    t_pre = pre_bytes / (0.8 * BW) + LAUNCH
    # group kernel: 7 products of 2048^3; reads 7 operands per side, writes C;
    # 128 x 128 group tiles: 256 groups on 256 CUs (no tail, q = 1), I_tile = 64
    F = 2.0 * 7 * h ** 3
    Bf = 2.0 * (7 * h * h + 7 * h * h) + 2.0 * n * n
    want = t_pre + kernel(F, Bf, 64.0, 1.0, ETA_F)
    p = L.lcma_plan_ex(n, n, n, "bf16", force="l1", combine="prepass", **OPTS)
    assert close(L.lcma_plan_estimate(p, "l1"), want)
    # 31.46 us of pre-pass bandwidth + 240.52 us of MFMA work at 0.25 of peak + two launches
    assert abs(want - 279.98e-6) < 0.01e-6


def test_one_level_split_tail_2560_cubed():
    # 100 groups of 128 x 128 on 256 CUs: the partial round is split two ways
    # (2 * 100 <= 256), which counts as half a round: q = (100 / 256) / 0.5
    n, h = 2560, 1280
    pre_bytes = 2.0 * 2 * n * n + 2.0 * 10 * h * h
    t_pre = pre_bytes / (0.8 * BW) + LAUNCH
    F = 2.0 * 7 * h ** 3
    Bf = 2.0 * 14 * h * h + 2.0 * n * n
    q = (100 / 256) / 0.5
    want = t_pre + kernel(F, Bf, 64.0, q, ETA_F)
    p = L.lcma_plan_ex(n, n, n, "bf16", force="l1", combine="prepass", **OPTS)
    assert close(L.lcma_plan_estimate(p, "l1"), want)
    # without the split the tail is a whole round (q = 100 / 256)
    p = L.lcma_plan_ex(n, n, n, "bf16", force="l1", combine="prepass", split="none", **OPTS)
    assert close(L.lcma_plan_estimate(p, "l1"), t_pre + kernel(F, Bf, 64.0, 100 / 256, ETA_F))


def test_one_level_combined_at_load_4096_cubed():
    # no pre-pass; the group kernel reads every nonzero block of U and V
    # (12 per side) instead of one operand per product
    n, h = 4096, 2048
    F = 2.0 * 7 * h ** 3
    Bf = 2.0 * (12 * h * h + 12 * h * h) + 2.0 * n * n
    want = kernel(F, Bf, 64.0, 1.0, ETA_F)
    p = L.lcma_plan_ex(n, n, n, "bf16", force="l1", combine="at_load", **OPTS)
    assert close(L.lcma_plan_estimate(p, "l1"), want)


def test_one_level_unfused_16384_cubed():
    # pre-pass writing all 7 operands per side, 7 classic products of 8192^3,
    # and the fp32 folds: 8c - 6 bytes per element of an output block that
    # takes c folds (2 for one).  C11 (P1, P4, P5, P7) and C22 (P1, P2, P3, P6)
    # are fed by four products, C12 and C21 by two; in one persistent launch
    # P6 continues P1's accumulators and P7 continues P4's, one fold less in
    # C22 and in C11: 2 * (8 * 3 - 6) + 2 * (8 * 2 - 6) = 56 bytes per Mb Nb
    n, h = 16384, 8192
    pre = 2.0 * 2 * n * n + 2.0 * 7 * 2 * h * h
    comb = 56.0 * h * h
    Fh = 2.0 * h ** 3
    prod = kernel(Fh, 2.0 * 3 * h * h, 128.0, 1.0, ETA_C)      # 1024 tiles of 256^2: 4 full rounds
    want = (pre + comb) / (0.8 * BW) + 7 * prod + 2 * LAUNCH
    p = L.lcma_plan_ex(n, n, n, "bf16", force="l1", combine="unfused", **OPTS)
    assert close(L.lcma_plan_estimate(p, "l1"), want)


def test_one_level_unfused_per_product_2048_cubed():
    # 1024^2 blocks hold 16 positions of 256^2, too few for one persistent
    # launch: each product folds on its own, every nonzero of W is a fold:
    # (8 * 4 - 6) * 2 + (8 * 2 - 6) * 2 = 8 * 12 - 6 * 4 = 72 bytes per Mb Nb;
    # the 1024^3 products run on 128^2 tiles (64 of them, a quarter round)
    n, h = 2048, 1024
    pre = 2.0 * 2 * n * n + 2.0 * 7 * 2 * h * h
    comb = 72.0 * h * h
    prod = kernel(2.0 * h ** 3, 2.0 * 3 * h * h, 64.0, 0.25, 0.7 * ETA_C)
    want = (pre + comb) / (0.8 * BW) + 7 * prod + 2 * LAUNCH
    p = L.lcma_plan_ex(n, n, n, "bf16", force="l1", combine="unfused", **OPTS)
    assert close(L.lcma_plan_estimate(p, "l1"), want)


def test_one_level_unfused_winograd_16384_cubed():
    # Winograd's variant in one persistent launch: its searched schedule
    # writes one block with a single fold (2 bytes) and the other three with
    # two folds each (10 bytes): 32 per Mb Nb
    n, h = 16384, 8192
    pre = 2.0 * 2 * n * n + 2.0 * 7 * 2 * h * h
    comb = 32.0 * h * h
    prod = kernel(2.0 * h ** 3, 2.0 * 3 * h * h, 128.0, 1.0, ETA_C)
    want = (pre + comb) / (0.8 * BW) + 7 * prod + 2 * LAUNCH
    d = L.Desc(2, 2, 2, D.WINOGRAD_U, D.WINOGRAD_V, D.WINOGRAD_W)
    p = L.lcma_plan_ex(n, n, n, "bf16", desc=d, force="l1", **OPTS)
    assert close(L.lcma_plan_estimate(p, "l1"), want)


@pytest.mark.parametrize("n", [4096, 2560])
def test_auto_pick_follows_the_estimates(n):
    p = L.lcma_plan_ex(n, n, n, "bf16", **OPTS)
    est = {a: L.lcma_plan_estimate(p, a) for a in ("classic", "l1", "l2")}
    best = min((v, a) for a, v in est.items() if v > 0)[1]
    chosen = L.lcma_plan_info(p)[0]
    # ties within 2% go to classic
    assert chosen == best or (chosen == "classic" and est["classic"] <= est[best] / 0.98)
