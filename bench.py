#!/usr/bin/env python3
"""Benchmark: effective TFLOP/s (2MNK / t) of half-precision GEMM on one MI355X.

One step = one pass of the hot path on the 4096^3 bfloat16 workload (A, B
i.i.d. N(0,1)/sqrt(K), fp32 accumulate, bfloat16 out): plan with the roofline
cost model (which picks classic, one-level or two-level), then run the planned
product (for an LCMA plan: combine pre-pass + persistent fused group kernel).
Inputs are resident in HBM before timing starts.

Besides the step, every algorithm is timed kernel by kernel with HIP events
on the stream the kernels run on, so the JSON line also reports the classic
and LCMA rates, the pre-pass bandwidth, the roofline of the dominant kernel
and the CPU oracle's rate on a bounded sample.

Also in the default line: the measured machine references (an MFMA loop
and an HBM stream kernel of the library; socket power and the shader clock
held while the classic kernel, the MFMA loop and the vendor GEMM each run
back to back, from amd-smi), the 16384^3 comparison of classic,
one level (unfused and fused) and two levels, decode-shaped products (M = 1
to 64 against N = 14336, K = 4096 and against N = 4096, K = 14336), cold-cache
and server-mode timings, the cold pre-pass bandwidth, and the performance
targets with whether each is met.

Prints ONE JSON line.  Single GPU only.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA, published
HBM_GBPS = 8000.0      # MI355X HBM3E, published
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILE = os.path.join(ROOT, "profiles", "gemm_4096_bf16_bench.md")


def recorded_traffic(kernel_prefix):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, calibrated against a copy of known size), or None
    when the kernel source changed since the counters were taken."""
    import hashlib
    try:
        text = open(PROFILE).read()
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        src = open(os.path.join(ROOT, "complexity_half_precision_amd", "csrc", "kernels.hip"), "rb").read()
        if hashlib.sha256(src).hexdigest()[:16] != blob["kernels_hip_sha256_16"]:
            return None
        for name, mb in blob["traffic_mb_per_launch"].items():
            if name.startswith(kernel_prefix):
                return mb * 1e6
    except (OSError, ValueError, KeyError, IndexError):
        return None
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--only", default="", help="time only these algorithms (comma list), for profiling runs")
    ap.add_argument("--size", type=int, default=0,
                    help="time the algorithms on an n^3 bfloat16 product instead of the 4096^3 workload "
                         "(detail only; the headline workload is fixed)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode-shape bandwidth measurement (one JSON line), for profiling runs")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the decode-shape bandwidth, 24-shape sweep, 16384^3 and machine measurements")
    ap.add_argument("--no-large", action="store_true", help="skip the 16384^3 and 32768^3 comparisons")
    ap.add_argument("--cold", action="store_true",
                    help="also time every kernel with the caches flushed before each call (writes a 512 MiB "
                         "buffer between calls, outside the timed region)")
    ap.add_argument("--server", action="store_true",
                    help="also time every algorithm in server mode: single calls separated by seeded random "
                         "host-side gaps of 0.2-2 ms (mean and median of the per-call event times)")
    ap.add_argument("--study", action="store_true",
                    help="only the schedule ablation of the one-level fused kernel (one JSON line): tail split "
                         "none/auto and locality/plain order on a tail shape, an all-split shape and 4096^3")
    ap.add_argument("--study-case", default="",
                    help="with --study: run only the case named 'MxNxK:split:order' (for counter runs)")
    ap.add_argument("--crossover", action="store_true",
                    help="only the classic / unfused one level comparison on n^3 bfloat16 for n from 8192 to "
                         "32768 (one JSON line)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="first run 3 device copies of this many MiB (reference for HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import complexity_half_precision_amd as L
    import seeded_inputs as si

    if args.copy_calib_mib:
        # reference for the HBM byte counters: device copies of known size
        src = torch.ones(args.copy_calib_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.crossover:
        print(json.dumps({"crossover": crossover(L, torch)}), flush=True)
        return

    if args.decode_only:
        def tc(fn, reps, warm):
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps
        print(json.dumps({"decode": decode_bandwidth(L, si, torch, tc),
                          "decode_long_k": decode_bandwidth(L, si, torch, tc, si.decode_long_k_shape)}), flush=True)
        return

    if args.study:
        def tc(fn, reps, warm):
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps
        print(json.dumps({"schedule_study": schedule_study(L, si, torch, tc, args.study_case,
                                                           max(args.steps, 10), args.warmup)}), flush=True)
        return

    wl = dict(si.SQUARE_4096_BF16)
    if args.size:
        wl.update(M=args.size, N=args.size, K=args.size)
    M, N, K, dtype = wl["M"], wl["N"], wl["K"], wl["dtype"]
    dev = "cuda"
    A, B = si.gen(**wl)
    Ad, Bd = A.to(dev), B.to(dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    flops = 2.0 * M * N * K

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def warm_clocks(seconds=0.5):
        # Bring clocks and power state to steady load before any timing.
        p = L.lcma_plan_ex(M, N, K, dtype, force="classic")
        ws = L.workspace_for(p)
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            for _ in range(20):
                L.lcma_gemm(p, Ad, Bd, C, ws)
            torch.cuda.synchronize()

    def time_calls(fn, reps, warm):
        """Mean ms per call over `reps` back-to-back calls, HIP events on the kernels' stream."""
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def time_cold(fn, reps):
        """Mean ms of fn with L2 and the last-level cache flushed before each call:
        a 512 MiB write (twice the MI355X last-level cache) between calls; only fn
        is inside the events."""
        tot = 0.0
        for _ in range(reps):
            flush_buf.fill_(1)
            e0, e1 = ev(), ev()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
        return tot / reps

    def time_gapped(fn, reps, seed=1234):
        """Per-call event times of fn, each call issued after the device went idle and
        the host slept a seeded random gap of 0.2-2 ms: the clock and cache state a
        server sees between requests, rather than back-to-back."""
        import random
        import time as _time
        rng = random.Random(seed)
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            _time.sleep(rng.uniform(0.2e-3, 2e-3))
            e0, e1 = ev(), ev()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        return sum(ts) / len(ts), ts[len(ts) // 2]

    # normwise error of each plan against the float64 product of the same
    # (already rounded) inputs, formed by torch on the device
    Cref = torch.matmul(Ad.double(), Bd.double())
    ref_norm = Cref.norm().item()

    def rel_err():
        torch.cuda.synchronize()
        return ((C.double() - Cref).norm() / ref_norm).item()

    detail = {}
    only = set(a for a in args.only.split(",") if a)
    plans = {}
    for algo in ("classic", "l1", "l1_f16_operands", "l2", "l2_bf16_operands", "l1_unfused", "l1_winograd",
                 "l1_at_load"):
        if only and algo not in only:
            continue
        try:
            if algo == "l1_unfused":
                p = L.lcma_plan_ex(M, N, K, dtype, force="l1", combine="unfused")
            elif algo == "l1_at_load":
                # one launch: the group kernel combines the input blocks itself
                p = L.lcma_plan_ex(M, N, K, dtype, force="l1", combine="at_load")
            elif algo == "l1":
                # the fused group kernel after a pre-pass (the planner itself
                # takes the unfused path for large blocks)
                p = L.lcma_plan_ex(M, N, K, dtype, force="l1", combine="prepass")
            elif algo == "l1_f16_operands":
                # one level with the combined operands rounded to binary16
                # (the default keeps bfloat16 operands at one level)
                p = L.lcma_plan_ex(M, N, K, dtype, force="l1", combine="prepass", bf16_ops_f16=1)
            elif algo == "l1_winograd":
                # Winograd's variant: the unfused path (any description)
                p = L.lcma_plan_ex(M, N, K, dtype, desc=L.winograd_desc(), force="l1")
            elif algo == "l2_bf16_operands":
                # two levels with the combined operands rounded to bfloat16
                # (the default rounds them to binary16 for bfloat16 inputs);
                # outside the 4x error band, so it needs the opt-in
                p = L.lcma_plan_ex(M, N, K, dtype, force="l2", bf16_ops_f16=-1, accuracy_optin=1)
            else:
                p = L.lcma_plan_ex(M, N, K, dtype, force=algo)
        except L.LcmaError:
            continue
        plans[algo] = (p, L.workspace_for(p))
    reps = max(args.steps, 10)
    warm_clocks()
    for algo, (p, ws) in plans.items():
        t_all = time_calls(lambda: L.lcma_gemm(p, Ad, Bd, C, ws), reps, args.warmup)
        d = {"ms": t_all, "eff_tflops": flops / (t_all * 1e-3) / 1e12, "est_ms": L.lcma_plan_info(p)[2] * 1e3}
        L.lcma_gemm(p, Ad, Bd, C, ws)
        d["rel_err"] = float("%.4g" % rel_err())
        if algo == "l1_at_load":
            mfma_flops = 2.0 * 7 * (M // 2) * (N // 2) * (K // 2)
            d.update({"fused_mfma_tflop": mfma_flops / 1e12, "fused_tflops_actual": mfma_flops / (t_all * 1e-3) / 1e12})
        elif algo != "classic":
            t_pre = time_calls(lambda: L.lcma_prepass(p, Ad, Bd, ws), reps, args.warmup)
            L.lcma_prepass(p, Ad, Bd, ws)
            t_fu = time_calls(lambda: L.lcma_fused(p, Ad, Bd, C, ws), reps, args.warmup)
            R = 49 if algo.startswith("l2") else 7
            S = 4 if algo.startswith("l2") else 2
            mfma_flops = 2.0 * R * (M // S) * (N // S) * (K // S)
            # bytes the pre-pass must move: read A and B once, write the combined operands
            written = sum(1 for r in range(R) if L.lcma_plan_operand(p, 0, r)[0] >= 0) * (M // S) * (K // S) \
                + sum(1 for r in range(R) if L.lcma_plan_operand(p, 1, r)[0] >= 0) * (K // S) * (N // S)
            pre_bytes = 2.0 * (M * K + K * N) + 2.0 * written
            d.update({"prepass_ms": t_pre, "fused_ms": t_fu, "fused_mfma_tflop": mfma_flops / 1e12,
                      "fused_tflops_actual": mfma_flops / (t_fu * 1e-3) / 1e12,
                      "prepass_bytes": pre_bytes, "prepass_gbps": pre_bytes / (t_pre * 1e-3) / 1e9})
        if args.cold or algo in ("classic", "l1", "l2", "l1_unfused"):
            reps_c = min(reps, 20)
            d["cold_ms"] = time_cold(lambda: L.lcma_gemm(p, Ad, Bd, C, ws), reps_c)
            if algo not in ("classic", "l1_at_load"):
                t_pre_c = time_cold(lambda: L.lcma_prepass(p, Ad, Bd, ws), reps_c)
                d.update({"cold_prepass_ms": t_pre_c, "cold_prepass_gbps": d["prepass_bytes"] / (t_pre_c * 1e-3) / 1e9})
        if args.server or algo in ("classic", "l1", "l2", "l1_unfused"):
            d["server_mean_ms"], d["server_p50_ms"] = time_gapped(lambda: L.lcma_gemm(p, Ad, Bd, C, ws), 50)
        detail[algo] = d
    if "classic" in detail:
        for d in detail.values():
            d["err_over_classic"] = d["rel_err"] / detail["classic"]["rel_err"]
    del Cref

    # ---- the step: plan + planned product on the workload
    auto = L.lcma_plan(M, N, K, dtype)
    chosen = L.lcma_plan_info(auto)[0]
    ws_auto = L.workspace_for(auto)

    def step():
        p = L.lcma_plan(M, N, K, dtype)
        L.lcma_gemm(p, Ad, Bd, C, ws_auto)

    if chosen not in plans:
        plans[chosen] = (auto, ws_auto)
    warm_clocks(0.2)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = max(e0.elapsed_time(e1), 0.0) / args.steps
    ms_step = max(ms_step, wall * 1e3 / args.steps)
    value = flops / (ms_step * 1e-3) / 1e12

    # ---- per-call distribution of the chosen path (a separate pass after the
    # timed steps: each call bracketed by its own events)
    p_dist, ws_dist = plans[chosen]
    per = []
    for _ in range(max(args.steps, 20)):
        a0, a1 = ev(), ev()
        a0.record(stream)
        L.lcma_gemm(p_dist, Ad, Bd, C, ws_dist)
        a1.record(stream)
        per.append((a0, a1))
    torch.cuda.synchronize()
    per = sorted(a0.elapsed_time(a1) for a0, a1 in per)
    q = lambda f: per[min(len(per) - 1, int(f * len(per)))]
    dist = {"calls": len(per), "median_ms": round(q(0.5), 4), "p10_ms": round(q(0.1), 4),
            "p90_ms": round(q(0.9), 4), "min_ms": round(per[0], 4),
            "median_tflops": round(flops / (q(0.5) * 1e-3) / 1e12, 1)}

    # ---- roofline of the dominant kernel of the chosen path
    if chosen == "classic":
        # (an --only run without the classic leg takes the per-call median)
        t_k = detail["classic"]["ms"] if "classic" in detail else dist["median_ms"]
        achieved = flops / (t_k * 1e-3) / 1e12
        kname, kprefix = "k_classic_m16 (256x256 tile, 8 waves, 16x16x32 MFMA; 2MNK flops per launch)", "k_classic_m16"
    else:
        # two levels: the 7 launches of the outer level together
        t_k = detail[chosen]["fused_ms"]
        achieved = detail[chosen]["fused_mfma_tflop"] * 1e12 / (t_k * 1e-3) / 1e12
        kname = "k_fused1_m16 (MFMA flops of the LCMA products per launch)"
        kprefix = "k_fused1_m16<true, true, false>" if chosen == "l1" else "k_fused1_m16<false, true, true>"
    traffic = recorded_traffic(kprefix)
    roofline = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 1), "peak": PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                "traffic": None if traffic is None else round(traffic),
                "traffic_note": "HBM bytes per launch, FETCH_SIZE + WRITE_SIZE calibrated by a 256 MiB copy; "
                                "algorithmic minimum %d" % int(2 * (M * K + K * N + M * N)),
                "kernel_ms": round(t_k, 4)}

    out = {
        "metric": "effective TFLOP/s (2MNK/t) FP16/BF16 GEMM at 1 GPU; % of MFMA peak",
        "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"square GEMM M=N=K={M}, bf16 A,B ~ N(0,1)/sqrt(K), fp32 accumulate, bf16 out",
                   "M": M, "N": N, "K": K, "algo_chosen": chosen},
        "pct_of_peak": round(100.0 * value / PEAK_TFLOPS, 2),
        "roofline": roofline,
        "dist": dist,
        "detail": {k: {kk: (round(vv, 4) if isinstance(vv, float) and kk != "rel_err" else vv) for kk, vv in v.items()}
                   for k, v in detail.items()},
    }
    if "l1" in detail and "classic" in detail:
        out["l1_over_classic"] = round(detail["classic"]["ms"] / detail["l1"]["ms"], 4)
    if "l1_at_load" in detail and "classic" in detail:
        out["l1_at_load_over_classic"] = round(detail["classic"]["ms"] / detail["l1_at_load"]["ms"], 4)
    if "l1_unfused" in detail and "classic" in detail:
        out["l1_unfused_over_classic"] = round(detail["classic"]["ms"] / detail["l1_unfused"]["ms"], 4)
    if "l1" in detail and "l1_unfused" in detail:
        # the fusion gain: same scheme, products folded on chip vs through fp32 blocks in HBM
        out["fused_over_unfused"] = round(detail["l1_unfused"]["ms"] / detail["l1"]["ms"], 4)

    out["modes"] = {a: {k: round(d[k], 4) for k in ("ms", "cold_ms", "server_p50_ms", "server_mean_ms") if k in d}
                    for a, d in detail.items() if "cold_ms" in d}
    if not args.no_extra and not args.size:
        del Ad, Bd, C, plans
        torch.cuda.empty_cache()
        out["machine"] = machine_refs(L, torch, time_calls)
        roofline["measured_peak_tflops"] = out["machine"]["mfma_bf16_tflops"]
        roofline["frac_of_measured_peak"] = round(roofline["achieved"] / out["machine"]["mfma_bf16_tflops"], 4)
        out["machine"]["power"] = power_and_clock(L, torch)
        held = out["machine"]["power"].get("classic_4096_bf16", {})
        if "gfx_clock_mhz" in held:
            roofline["held_clock_mhz"] = held["gfx_clock_mhz"]
            roofline["socket_power_w"] = held["socket_power_w"]
            roofline["frac_at_held_clock"] = round(roofline["achieved"] / held["peak_at_clock_tflops"], 4)
        if not args.no_large:
            out["large"] = large_square(L, si, torch, time_calls, time_cold)
            out["huge"] = huge_square(L, si, torch)
        out["square_512_f16"] = small_square(L, si, torch, time_calls)
        out["decode"] = decode_bandwidth(L, si, torch, time_calls)
        out["decode_long_k"] = decode_bandwidth(L, si, torch, time_calls, si.decode_long_k_shape)
        for leg in (out["decode"], out["decode_long_k"]):       # against the measured read-only stream
            for v in leg.values():
                v["frac_of_read_ref"] = round(v["hbm_gbps"] / out["machine"]["hbm_read_gbps"], 3)
        out["sweep"] = sweep_picks(L, si, torch, time_calls)
        out["k_split"] = k_split_gains(L, si, torch, time_calls)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(A, B, args.cpu_seconds)
        out["cpu_baseline"]["one_core"] = cpu_baseline_one_core(A, B, args.cpu_seconds)
    out["targets"] = targets(out)
    print(json.dumps(out), flush=True)


def targets(out):
    """The throughput targets against what this run measured (reported
    as they stand, met or not)."""
    t = {"classic_frac_of_peak": {"target": 0.70, "measured": out["roofline"]["frac"]}}
    if "l1_over_classic" in out:
        best = max(out.get("l1_over_classic", 0), out.get("l1_at_load_over_classic", 0),
                   out.get("l1_unfused_over_classic", 0))
        t["lcma_over_classic_4096"] = {"target": 1.08, "measured": round(best, 4)}
    if "large" in out:
        lg = out["large"]
        forms = [a for a in ("l1", "l1_fused", "l1_winograd", "l2") if a in lg]
        best = max(forms, key=lambda a: lg[a]["over_classic"])
        t["lcma_over_classic_16384"] = {"target": 1.08, "measured": lg[best]["over_classic"], "form": best}
    if "huge" in out:
        hg = out["huge"]
        best = max(("l1", "l1_winograd"), key=lambda a: hg[a]["over_classic"])
        t["lcma_over_classic_32768"] = {"target": 1.08, "measured": hg[best]["over_classic"], "form": best}
    for v in t.values():
        v["met"] = v["measured"] >= v["target"]
    return t


def machine_refs(L, torch, time_calls):
    """Measured references beside the published peaks: the library's MFMA loop
    (16x16x32, random operands, 2 workgroups of 8 waves per compute unit), its
    HBM stream kernels (1 GiB copied, read + write counted; 1 GiB read), plus
    torch's device copy of the same buffers."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {}
    wg, iters = 2 * cus, 20000
    out = torch.empty(wg * 512, dtype=torch.float32, device="cuda")
    for dt in ("bf16", "f16"):
        flops = [0.0]

        def call():
            flops[0] = L.lcma_measure_mfma(out, wg, iters, dt)
        t = time_calls(call, 5, 2)
        res[f"mfma_{dt}_tflops"] = round(flops[0] / (t * 1e-3) / 1e12, 1)
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    t = time_calls(lambda: L.lcma_measure_copy(src, dst), 10, 3)
    res["hbm_stream_gbps"] = round(2.0 * n / (t * 1e-3) / 1e9, 1)
    t = time_calls(lambda: dst.copy_(src), 10, 3)
    res["torch_copy_gbps"] = round(2.0 * n / (t * 1e-3) / 1e9, 1)
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    t = time_calls(lambda: L.lcma_measure_read(src, word), 10, 3)
    res["hbm_read_gbps"] = round(n / (t * 1e-3) / 1e9, 1)
    del src, dst, word
    # the vendor library's GEMM on the headline shape, as context for the classic kernel
    g = torch.Generator(device="cuda").manual_seed(7)
    a = (torch.randn(4096, 4096, device="cuda", generator=g) / 64).to(torch.bfloat16)
    b = (torch.randn(4096, 4096, device="cuda", generator=g) / 64).to(torch.bfloat16)
    c = torch.empty(4096, 4096, device="cuda", dtype=torch.bfloat16)
    t = time_calls(lambda: torch.matmul(a, b, out=c), 200, 200)     # its first calls run slower: warm it up well
    res["torch_matmul_4096_bf16_tflops"] = round(2.0 * 4096 ** 3 / (t * 1e-3) / 1e12, 1)
    res["note"] = ("mfma: %d workgroups x 8 waves x %d x 16 MFMAs per launch; stream: %d bytes read and written "
                   "(copy) or read (read); "
                   "torch.matmul: the vendor BLAS on 4096^3 bfloat16, context only" % (wg, iters, n))
    del out, a, b, c
    torch.cuda.empty_cache()
    return res


def power_and_clock(L, torch, seconds=2.0):
    """Socket power and shader clock while one workload at a time runs back to
    back for `seconds`: the classic kernel on a 4096^3 bfloat16 product, the
    library's MFMA loop and the vendor GEMM.  amd-smi (a child process)
    samples every ~0.1 s; the medians over the second half of each run are
    reported (its readings update about once a second).  peak_at_clock =
    1024 SIMDs x 1024 flop/clk x the clock held; frac_at_clock = achieved /
    peak_at_clock."""
    import shutil
    import subprocess
    import threading
    import time
    smi = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(smi):
        return {"note": "amd-smi not found"}

    def sample():
        r = subprocess.run([smi, "metric", "-p", "-c", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)["gpu_data"][0]
        clk = [v["clk"]["value"] for k, v in d["clock"].items() if k.startswith("gfx_")]
        return float(d["power"]["socket_power"]["value"]), sum(clk) / len(clk)

    def run(fn, flops_per_call, batch):
        samples, stop = [], threading.Event()

        def loop():
            while not stop.is_set():
                try:
                    samples.append((time.time(),) + sample())
                except (OSError, ValueError, KeyError, IndexError, subprocess.SubprocessError):
                    time.sleep(0.1)
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
        th = threading.Thread(target=loop, daemon=True)
        t0 = time.time()
        th.start()
        calls = 0
        while time.time() - t0 < seconds:
            for _ in range(batch):
                fn()
            calls += batch
            torch.cuda.synchronize()
        el = time.time() - t0
        stop.set()
        th.join()
        late = sorted(x for x in samples if x[0] >= t0 + seconds / 2) or samples
        if not late:
            return {"note": "no amd-smi samples"}
        pw = sorted(x[1] for x in late)[len(late) // 2]
        ck = sorted(x[2] for x in late)[len(late) // 2]
        achieved = calls * flops_per_call / el / 1e12
        peak = 1024 * 1024 * ck * 1e6 / 1e12
        return {"tflops": round(achieved, 1), "socket_power_w": pw, "gfx_clock_mhz": round(ck, 1),
                "peak_at_clock_tflops": round(peak, 1), "frac_at_clock": round(achieved / peak, 4),
                "samples": len(late)}

    n = 4096
    g = torch.Generator(device="cuda").manual_seed(7)
    a = (torch.randn(n, n, device="cuda", generator=g) / 64).to(torch.bfloat16)
    b = (torch.randn(n, n, device="cuda", generator=g) / 64).to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    plan = L.lcma_plan(n, n, n, "bf16")
    res = {"classic_4096_bf16": run(L.lcma_gemm_prepared(plan, a, b, c, L.workspace_for(plan)), 2.0 * n ** 3, 100)}
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(2 * cus * 512, dtype=torch.float32, device="cuda")
    mflops = [0.0]

    def mfma():
        mflops[0] = L.lcma_measure_mfma(out, 2 * cus, 2000, "bf16")
    mfma()
    res["mfma_loop_bf16"] = run(mfma, mflops[0], 2)
    res["torch_matmul_4096_bf16"] = run(lambda: torch.matmul(a, b, out=c), 2.0 * n ** 3, 100)
    del a, b, c, out
    torch.cuda.empty_cache()
    return res


def large_square(L, si, torch, time_calls, time_cold):
    """16384^3 bfloat16, A, B ~ N(0,1)/sqrt(K): classic against one level (the
    planner's unfused form and the fused group kernel after a pre-pass) and
    Winograd's variant on the unfused path (its run schedule moves the fewest
    fold bytes), two levels (binary16 combined operands, the default for bfloat16, and
    bfloat16 operands under the accuracy opt-in), each timed back to back on
    resident inputs; effective TFLOP/s = 2 n^3 / t.  Each plan's normwise
    error is taken against the float64 product of the same inputs."""
    w = si.SQUARE_16384_BF16
    n = w["M"]
    A, B = si.gen(**w)
    Ad, Bd = A.to("cuda"), B.to("cuda")
    del A, B
    C = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    flops = 2.0 * n ** 3
    res = {"workload": f"square GEMM M=N=K={n}, bf16 A,B ~ N(0,1)/sqrt(K), fp32 accumulate, bf16 out"}
    Cref = torch.matmul(Ad.double(), Bd.double())
    ref_norm = Cref.norm().item()
    for name, kw in (("classic", dict(force="classic")), ("l1", dict(force="l1")),
                     ("l1_fused", dict(force="l1", combine="prepass")),
                     ("l1_winograd", dict(force="l1", desc=L.winograd_desc())), ("l2", dict(force="l2")),
                     ("l2_bf16_operands", dict(force="l2", bf16_ops_f16=-1, accuracy_optin=1))):
        p = L.lcma_plan_ex(n, n, n, "bf16", **kw)
        ws = L.workspace_for(p)
        t = time_calls(lambda: L.lcma_gemm(p, Ad, Bd, C, ws), 6, 2)
        d = {"ms": round(t, 4), "eff_tflops": round(flops / (t * 1e-3) / 1e12, 1)}
        L.lcma_gemm(p, Ad, Bd, C, ws)
        torch.cuda.synchronize()
        d["rel_err"] = float("%.4g" % ((C.double() - Cref).norm() / ref_norm).item())
        if name != "classic":
            t_pre = time_calls(lambda: L.lcma_prepass(p, Ad, Bd, ws), 6, 1)
            R = 49 if name.startswith("l2") else 7
            S = 4 if name.startswith("l2") else 2
            nw = sum(1 for r in range(R) for side in (0, 1) if L.lcma_plan_operand(p, side, r)[0] >= 0)
            pre_bytes = 2.0 * 2 * n * n + 2.0 * nw * (n // S) ** 2
            d.update({"prepass_ms": round(t_pre, 4), "prepass_gbps": round(pre_bytes / (t_pre * 1e-3) / 1e9, 1),
                      "cold_prepass_gbps": round(pre_bytes / (time_cold(lambda: L.lcma_prepass(p, Ad, Bd, ws), 3)
                                                              * 1e-3) / 1e9, 1),
                      "mfma_tflop": round(2.0 * R * (n // S) ** 3 / 1e12, 3)})
        res[name] = d
        del ws
        torch.cuda.empty_cache()
    for name in ("l1", "l1_fused", "l1_winograd", "l2", "l2_bf16_operands"):
        res[name]["over_classic"] = round(res["classic"]["ms"] / res[name]["ms"], 4)
        res[name]["err_over_classic"] = round(res[name]["rel_err"] / res["classic"]["rel_err"], 3)
    del Cref
    del Ad, Bd, C
    torch.cuda.empty_cache()
    return res


def huge_square(L, si, torch):
    """32768^3 bfloat16, A, B ~ N(0,1)/sqrt(K): classic against one level on the
    unfused path, Strassen's scheme and Winograd's variant (each run schedule
    the planner's), timed in alternating rounds on resident inputs; each
    plan's normwise error against the float64 product of the same inputs."""
    w = si.SQUARE_32768_BF16
    n = w["M"]
    A, B = si.gen(**w)
    Ad, Bd = A.to("cuda"), B.to("cuda")
    del A, B
    C = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    flops = 2.0 * n ** 3
    res = {"workload": f"square GEMM M=N=K={n}, bf16 A,B ~ N(0,1)/sqrt(K), fp32 accumulate, bf16 out"}
    plans = {}
    for name, kw in (("classic", dict(force="classic")), ("l1", dict(force="l1")),
                     ("l1_winograd", dict(force="l1", desc=L.winograd_desc()))):
        p = L.lcma_plan_ex(n, n, n, "bf16", **kw)
        plans[name] = (p, L.workspace_for(p))
    ts = {k: [] for k in plans}
    for rnd in range(4):
        for k in (list(plans) if rnd % 2 == 0 else list(plans)[::-1]):
            p, ws = plans[k]
            L.lcma_gemm(p, Ad, Bd, C, ws)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(2):
                L.lcma_gemm(p, Ad, Bd, C, ws)
            e1.record()
            torch.cuda.synchronize()
            ts[k].append(e0.elapsed_time(e1) / 2)
    Cref = torch.matmul(Ad.double(), Bd.double())
    ref_norm = Cref.norm().item()
    for k, (p, ws) in plans.items():
        t = sorted(ts[k])[len(ts[k]) // 2]
        L.lcma_gemm(p, Ad, Bd, C, ws)
        torch.cuda.synchronize()
        res[k] = {"ms": round(t, 4), "eff_tflops": round(flops / (t * 1e-3) / 1e12, 1),
                  "rel_err": float("%.4g" % ((C.double() - Cref).norm() / ref_norm).item())}
    for k in ("l1", "l1_winograd"):
        res[k]["over_classic"] = round(res["classic"]["ms"] / res[k]["ms"], 4)
        res[k]["err_over_classic"] = round(res[k]["rel_err"] / res["classic"]["rel_err"], 3)
    # the planner's own pick (built-in scheme) against the faster of the two it chooses from
    res["auto_pick"] = L.lcma_plan_info(L.lcma_plan(n, n, n, "bf16"))[0]
    res["auto_agrees"] = res["auto_pick"] == min(("classic", "l1"), key=lambda a: res[a]["ms"])
    del Ad, Bd, C, Cref, plans
    torch.cuda.empty_cache()
    return res


def crossover(L, torch, sizes=(8192, 12288, 16384, 20480, 24576, 28672, 32768)):
    """Where the unfused one level overtakes the classic kernel: n^3 bfloat16
    with A, B ~ N(0,1)/sqrt(n) drawn on the device (torch's seeded Philox
    generator; timing only), classic against Strassen and Winograd on the
    unfused path, timed in alternating rounds (median of 4 rounds of 2 calls),
    plus the planner's AUTO pick."""
    g = torch.Generator(device="cuda").manual_seed(0)
    out = {}
    for n in sizes:
        A = (torch.randn(n, n, device="cuda", generator=g) / n ** 0.5).to(torch.bfloat16)
        B = (torch.randn(n, n, device="cuda", generator=g) / n ** 0.5).to(torch.bfloat16)
        C = torch.empty(n, n, dtype=torch.bfloat16, device="cuda")
        plans = {}
        for name, kw in (("classic", dict(force="classic")), ("strassen", dict(force="l1", combine="unfused")),
                         ("winograd", dict(force="l1", desc=L.winograd_desc()))):
            p = L.lcma_plan_ex(n, n, n, "bf16", **kw)
            plans[name] = (p, L.workspace_for(p))
        ts = {k: [] for k in plans}
        for rnd in range(4):
            for k in (list(plans) if rnd % 2 == 0 else list(plans)[::-1]):
                p, ws = plans[k]
                L.lcma_gemm(p, A, B, C, ws)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(2):
                    L.lcma_gemm(p, A, B, C, ws)
                e1.record()
                torch.cuda.synchronize()
                ts[k].append(e0.elapsed_time(e1) / 2)
        med = {k: sorted(v)[len(v) // 2] for k, v in ts.items()}
        row = {k: round(v, 4) for k, v in med.items()}
        row["strassen_over_classic"] = round(med["classic"] / med["strassen"], 4)
        row["winograd_over_classic"] = round(med["classic"] / med["winograd"], 4)
        row["auto_pick"] = L.lcma_plan_info(L.lcma_plan(n, n, n, "bf16"))[0]
        out[str(n)] = row
        print(json.dumps({"n": n, **row}), file=sys.stderr, flush=True)
        del A, B, C, plans
        torch.cuda.empty_cache()
    return out


def small_square(L, si, torch, time_calls):
    """512^3 binary16 product, A, B ~ U(-1, 1): classic against one level (7
    products of 256^3 blocks).  Launch- and latency-bound: the operands sit in
    the caches and the MFMA work is a fraction of a microsecond."""
    A, B = si.gen(512, 512, 512, "f16", "uniform", 0)
    Ad, Bd = A.to("cuda"), B.to("cuda")
    Cd = torch.empty((512, 512), dtype=torch.float16, device="cuda")
    res = {}
    for algo in ("classic", "l1"):
        p = L.lcma_plan_ex(512, 512, 512, "f16", force=algo)
        # prepared once: the binding's per-call checks take longer than these kernels
        t = time_calls(L.lcma_gemm_prepared(p, Ad, Bd, Cd, L.workspace_for(p)), 200, 20)
        res[algo] = {"us": round(t * 1e3, 2), "eff_tflops": round(2.0 * 512 ** 3 / (t * 1e-3) / 1e12, 1)}
    res["pick"] = L.lcma_plan_info(L.lcma_plan(512, 512, 512, "f16"))[0]
    del Ad, Bd, Cd
    torch.cuda.empty_cache()
    return res


def decode_bandwidth(L, si, torch, time_calls, shape=None):
    """Decode-shaped products (M in 1, 4, 16, 64, bfloat16; K=4096, N=14336 by
    default, or `shape(m)`, e.g. K=14336, N=4096, which the K split serves):
    the planned path (the cost model must pick classic), HBM GB/s of the
    algorithmic bytes 2(MK + KN + MN).  B rotates over 4 resident copies (470
    MB, more than the 256 MB last-level cache), so every call streams its B
    from HBM.  The calls are prepared once (lcma_gemm_prepared) and issued
    back to back."""
    res = {}
    for m in si.DECODE_MS:
        w = (shape or si.decode_shape)(m)
        A, B = si.gen(**w)
        Ad = A.to("cuda")
        Bs = [B.to("cuda")] + [None] * 3
        for i in range(1, 4):
            Bs[i] = Bs[0].clone()
        Cd = torch.empty((m, w["N"]), dtype=torch.bfloat16, device="cuda")
        p = L.lcma_plan(m, w["N"], w["K"], "bf16")
        algo = L.lcma_plan_info(p)[0]
        # arguments checked once per B copy: the per-call checks of the binding
        # take about as long as these kernels run
        ws = L.workspace_for(p)      # the K split's partials, if the plan splits
        calls = [L.lcma_gemm_prepared(p, Ad, Bs[i], Cd, ws) for i in range(4)]
        k = [0]

        def call():
            calls[k[0] & 3]()
            k[0] += 1
        t = time_calls(call, 200, 20)
        byts = 2.0 * (m * w["K"] + w["K"] * w["N"] + m * w["N"])
        res[f"M={m}"] = {"algo": algo, "us": round(t * 1e3, 2), "hbm_gbps": round(byts / (t * 1e-3) / 1e9, 1),
                         "tflops": round(2.0 * m * w["N"] * w["K"] / (t * 1e-3) / 1e12, 2)}
        del calls, ws, Ad, Bs, Cd
    torch.cuda.empty_cache()
    return res


K_SPLIT_SHAPES = ((1, 4096, 14336), (64, 4096, 14336), (4096, 256, 8192), (512, 2048, 16384), (256, 256, 16384),
                  (3328, 5120, 8192), (4104, 4104, 4104), (7168, 7168, 7168))


def k_split_gains(L, si, torch, time_calls):
    """Classic plans whose K is split (decode strips, few tiles, the last
    partial round of a multi-round grid) against the same product planned
    with split="none" (the unsplit kernels): bfloat16, A ~ N(0,1)/sqrt(K),
    prepared calls on resident operands."""
    rows = []
    for i, (M, N, K) in enumerate(K_SPLIT_SHAPES):
        A, B = si.gen(M, N, K, "bf16", "normal_sqrtk", 500 + i)
        Ad, Bd = A.to("cuda"), B.to("cuda")
        Cd = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        calls = {mode: L.lcma_gemm_prepared(p, Ad, Bd, Cd, L.workspace_for(p))
                 for mode in ("auto", "none")
                 for p in [L.lcma_plan_ex(M, N, K, "bf16", force="classic", split=mode)]}
        reps = 20 if 2.0 * M * N * K > 1e11 else 100
        ts = {"auto": [], "none": []}
        for rnd in range(4):                  # alternating order, median of the rounds
            for mode in (("auto", "none") if rnd % 2 == 0 else ("none", "auto")):
                ts[mode].append(time_calls(calls[mode], reps, 5))
        t = {mode: sorted(v)[len(v) // 2] for mode, v in ts.items()}
        rows.append({"shape": [M, N, K], "split_us": round(t["auto"] * 1e3, 2), "unsplit_us": round(t["none"] * 1e3, 2),
                     "speedup": round(t["none"] / t["auto"], 3),
                     "split_tflops": round(2.0 * M * N * K / (t["auto"] * 1e-3) / 1e12, 1)})
        del Ad, Bd, Cd
    torch.cuda.empty_cache()
    return rows


def sweep_picks(L, si, torch, time_calls):
    """The 24 seeded sweep shapes (binary16): the cost model's pick against the
    measured fastest admissible algorithm; agreement rate over the shapes."""
    rows, agree = [], 0
    for w in si.sweep_workloads():
        M, N, K = w["M"], w["N"], w["K"]
        A, B = si.gen(**w)
        Ad, Bd = A.to("cuda"), B.to("cuda")
        Cd = torch.empty((M, N), dtype=torch.float16, device="cuda")
        pick = L.lcma_plan_info(L.lcma_plan(M, N, K, "f16"))[0]
        times = {}
        for algo in ("classic", "l1", "l2"):
            try:
                p = L.lcma_plan_ex(M, N, K, "f16", force=algo)
            except L.LcmaError:
                continue
            # prepared once: the per-call argument checks of the binding would
            # otherwise set the pace for the small shapes
            times[algo] = time_calls(L.lcma_gemm_prepared(p, Ad, Bd, Cd, L.workspace_for(p)), 20, 3)
        best = min(times, key=times.get)
        agree += pick == best
        rows.append({"shape": [M, N, K], "pick": pick, "best": best,
                     "ms": {a: round(t, 4) for a, t in times.items()}})
        del Ad, Bd, Cd
    torch.cuda.empty_cache()
    return {"agreement": round(agree / len(rows), 3), "shapes": rows}


STUDY_SHAPES = ((4096, 5120, 4096), (2560, 2560, 2560), (4096, 4096, 4096))


def schedule_mix(L, plan):
    """From the planned schedule: split groups, the makespan in products, and the
    fraction of XCDs (worker w runs on XCD w % 8) whose workers run both halves
    of split groups at once (product-type mixing in one L2)."""
    items, _ = L.lcma_plan_schedule(plan)
    load, halves = {}, {}
    split = set()
    for (w, g, p0, p1, slot) in items:
        load[w] = load.get(w, 0) + (p1 - p0)
        if slot >= 0:
            split.add(g)
            halves.setdefault(w % 8, set()).add(p0 == 0)
    mixed = sum(1 for h in halves.values() if len(h) == 2)
    return {"split_groups": len(split), "makespan_products": max(load.values()),
            "xcds_mixing_halves": round(mixed / 8, 3)}


def schedule_study(L, si, torch, time_calls, case, reps, warm):
    """Schedule ablation of the one-level fused kernel on bfloat16 N(0,1)/sqrt(K)
    inputs: tail split (none / auto) x order (locality / plain), timed kernel by
    kernel (the pre-pass is identical across variants and excluded), with the
    classic product of the same shape beside it.  4096 x 5120 x 4096 has 320
    groups of 128 x 128 (one full round plus a tail of 64 on 256 compute units);
    2560^3 has 100 groups, all split; 4096^3 has 256, no tail."""
    res = []
    for (M, N, K) in STUDY_SHAPES:
        shape = f"{M}x{N}x{K}"
        variants = [(sp, od) for sp in ("none", "auto") for od in ("auto", "plain")]
        variants = [v for v in variants if not case or case == f"{shape}:{v[0]}:{v[1]}"]
        if not variants:
            continue
        A, B = si.gen(M, N, K, "bf16", "normal_sqrtk", 0)
        Ad, Bd = A.to("cuda"), B.to("cuda")
        Cd = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        row = {"shape": [M, N, K]}
        calls = {}
        if not case:
            pc = L.lcma_plan_ex(M, N, K, "bf16", force="classic")
            wsc = L.workspace_for(pc)
            calls["classic"] = (None, lambda pc=pc, wsc=wsc: L.lcma_gemm(pc, Ad, Bd, Cd, wsc))
        for sp, od in variants:
            p = L.lcma_plan_ex(M, N, K, "bf16", force="l1", split=sp, order=od)
            ws = L.workspace_for(p)
            L.lcma_prepass(p, Ad, Bd, ws)
            calls[f"split={sp},order={od}"] = (p, lambda p=p, ws=ws: L.lcma_fused(p, Ad, Bd, Cd, ws))
        # rounds in rotated order, median per variant: clock drift over the
        # run then favours no variant
        names = list(calls)
        times = {n: [] for n in names}
        for rnd in range(5):
            for i in range(len(names)):
                n = names[(i + rnd) % len(names)]
                times[n].append(time_calls(calls[n][1], reps, warm))
        flops = 2.0 * 7 * (M // 2) * (N // 2) * (K // 2)
        for n in names:
            t = sorted(times[n])[len(times[n]) // 2]
            if n == "classic":
                row["classic_ms"] = round(t, 4)
            else:
                row[n] = dict(schedule_mix(L, calls[n][0]), fused_ms=round(t, 4),
                              fused_tflops_actual=round(flops / (t * 1e-3) / 1e12, 1))
        res.append(row)
        del Ad, Bd, Cd
        torch.cuda.empty_cache()
    return res


def cpu_baseline(A, B, target_s):
    """The fp64 oracle on a row slice of the same product (all host threads)."""
    import numpy as np
    import oracle
    import seeded_inputs as si
    A64, B64 = si.f64(A), si.f64(B)
    M, K = A64.shape
    N = B64.shape[1]
    cores = oracle.max_threads()
    rows = 64
    t0 = time.perf_counter()
    oracle.gemm_rows(A64, B64, 0, rows)
    dt = time.perf_counter() - t0
    rows = int(min(M, max(64, rows * target_s / max(dt, 1e-6))))
    # the whole product may take less than the target: repeat it
    reps = max(1, int(target_s / max(dt * rows / 64, 1e-6))) if rows == M else 1
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.gemm_rows(A64, B64, 0, rows)
    dt = time.perf_counter() - t0
    tflops = 2.0 * reps * rows * N * K / dt / 1e12
    return {"value": round(tflops, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"rows 0..{rows} of the {M}x{N}x{K} product (fp64, k ascending), {reps} time(s), {dt:.1f} s"}


def cpu_baseline_one_core(A, B, target_s):
    """The same oracle on one host thread, on a row slice of the same workload
    sized for about a third of target_s."""
    import oracle
    import seeded_inputs as si
    A64, B64 = si.f64(A), si.f64(B)
    M, K = A64.shape
    N = B64.shape[1]
    before = oracle.max_threads()
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.gemm_rows(A64, B64, 0, 8)
        dt = time.perf_counter() - t0
        rows = int(min(M, max(8, 8 * (target_s / 3) / max(dt, 1e-6))))
        t0 = time.perf_counter()
        oracle.gemm_rows(A64, B64, 0, rows)
        dt = time.perf_counter() - t0
        used = oracle.max_threads()
    finally:
        oracle.set_threads(before)
    return {"value": round(2.0 * rows * N * K / dt / 1e12, 6), "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "sample": f"rows 0..{rows} of the {M}x{N}x{K} product (fp64, k ascending), {dt:.1f} s"}

if __name__ == "__main__":
    main()
