#!/usr/bin/env python3
"""Benchmark of the two-sided rounding solver (bakron_quantize) on one MI355X.

One step = one bakron_quantize call over the 4096 x 4096 INT4 workload (the
pages' benchmark size): quantizer parameters, relayout, every leaf and band
GEMM of the recursion, and the e^2 reduction.  The inputs (W, LA, LB) are
resident in HBM before timing; LA and LB come from bakron_hessian and
bakron_factor on the synthetic samples (untimed preparation).

Prints one JSON line.  Besides the contract fields it carries
  roofline      for the band GEMM (fp32 MFMA peak), the kernel the metric's
                "% of fp32 MFMA peak" names, with algorithmic flops / average
                launch duration from HIP events recorded inside the library on
                the solver's stream, and the MFMA utilisation from the committed
                counter summary (fp32 MFMA flops counted per dispatch over that
                same duration).  The leaf kernel takes about as long in total
                (dominant_kernel names the longer phase) but is bound by its
                chain of dependent steps, not by a throughput roofline
  gemm_phase    the whole band phase (critical and deferred products): useful
                flops over the kernel time of the two band replays, against the
                fp32 MFMA peak
  leaf          the leaf phase: HBM bytes per launch, launches, in-kernel steps,
                and its in-tile flops against the fp32 vector peak
  prep          bakron_hessian and bakron_factor for both Kronecker factors,
                each timed on its own (they sit on either side of the solve and
                are not part of a step)
  cpu_baseline  the fp64 oracle (BaKron-naive) on a bounded leading block of
                the same problem, on this host's cores
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP32_MFMA_PEAK_TFLOPS = 157.3
# MI355X's published fp32 vector peak; it counts packed two-wide fp32 FMAs,
# which this library's kernels do not use (scalar FMAs reach half of it)
FP32_VALU_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
# committed rocprofv3 summaries, per workload, of this command's default launch
# configuration (graph replay, automatic product order)
PROFILES = {"c3": os.path.join(ROOT, "profiles", "band_gemm_leaf_4096x4096_int4.md"),
            "c5": os.path.join(ROOT, "profiles", "band_gemm_leaf_4096x14336_int2asym.md")}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="c3")
    p.add_argument("--cpu-sample", type=int, default=1024,
                   help="edge of the leading block timed with the CPU oracle (0 = skip)")
    p.add_argument("--order", type=int, default=0)
    p.add_argument("--antidiag", action="store_true",
                   help="also time BaKron-antidiagonal once on the same inputs and report the ratio")
    p.add_argument("--split", choices=["cols", "rows", "both"], default=None,
                   help="also time the hybrid schedule (one top-level column / row split, "
                        "BAKRON_FLAG_SPLIT_*) on the same inputs and report its time")
    p.add_argument("--eager", action="store_true",
                   help="launch kernel by kernel instead of replaying the solve's graph")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a 1 GiB device copy (reference for HBM byte counters)")
    return p.parse_args()


def cpu_baseline(W, LA, LB, w, k):
    """Time BaKron-naive (fp64, OpenMP) on the leading k x k block of the
    workload: the entries of that block only receive updates from inside it,
    so it is an exact sub-problem of the same solve."""
    import oracle
    Wk = np.ascontiguousarray(W[:k, :k])
    LAk = np.ascontiguousarray(LA[:k, :k])
    LBk = np.ascontiguousarray(LB[:k, :k])
    s, z = oracle.qparams(Wk, w.qkind, w.qbits)
    oracle._load()
    t0 = time.perf_counter()
    oracle.naive(Wk, LAk, LBk, s, z, w.qkind, w.qbits)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    rate = k * k / dt
    # the naive solver's work grows as (m(m+1)/2)(n(n+1)/2): its rate on the
    # whole problem is the sample rate scaled by the work per entry
    work = lambda a, b: (a * (a + 1) / 2) * (b * (b + 1) / 2)
    full = (w.m * w.n) / (dt * work(w.m, w.n) / work(k, k))
    return {"value": rate, "unit": "entries/s", "cores": min(cores, threads), "kind": "oracle",
            "sample": f"leading {k}x{k} block of the {w.m}x{w.n} solve (BaKron-naive fp64, "
                      f"{dt:.2f} s); full-size rate by the naive work ratio: {full:.4g} entries/s",
            "seconds": dt, "full_size_rate_estimate": full}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    from two_sided_gptq_amd import bakron, synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    bakron.load()

    # ---- synthetic inputs and factors (outside the timed steps; each hessian
    # and factor call is timed on its own after one warm-up call)
    W_h = synth.weights(w)
    X = torch.from_numpy(synth.input_samples(w)).to(dev)
    Y_h = synth.output_samples(w)
    prep = {}

    def timed(label, fn, flops):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        r = fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        prep[label] = {"ms": ms, "tflops": flops / (ms / 1e3) / 1e12 if flops else None}
        return r

    # Gram product: 2 N d^2 flops for the full product (N d (d + 1) for one
    # triangle); factor: Cholesky plus triangular inverse, d^3 flops
    HA = timed("hessian_A", lambda: bakron.hessian(X, synth.DAMP), 2.0 * X.shape[0] * w.n ** 2)
    prep["hessian_A"].update(N=int(X.shape[0]), d=w.n)
    LA = timed("factor_A", lambda: bakron.factor(HA), float(w.n) ** 3)
    prep["factor_A"].update(d=w.n)
    if Y_h is None:
        LB = torch.eye(w.m, dtype=torch.float32, device=dev)
    else:
        Y = torch.from_numpy(Y_h).to(dev)
        HB = timed("hessian_B", lambda: bakron.hessian(Y, synth.DAMP), 2.0 * Y.shape[0] * w.m ** 2)
        prep["hessian_B"].update(N=int(Y.shape[0]), d=w.m)
        LB = timed("factor_B", lambda: bakron.factor(HB), float(w.m) ** 3)
        prep["factor_B"].update(d=w.m)
        del Y, HB
    del X, HA
    W = torch.from_numpy(W_h).to(dev)
    m, n = w.m, w.n
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(bakron.quantize_workspace_size(m, n, w.qkind, w.qbits), dtype=torch.uint8,
                     device=dev)
    out = dict(codes=torch.empty((m, n), dtype=torch.int8, device=dev),
               scales=torch.empty(m, dtype=torch.float32, device=dev),
               zeros=torch.empty(m, dtype=torch.float32, device=dev) if w.qkind == 1 else None,
               V=torch.empty((m, n), dtype=torch.float32, device=dev),
               E=None,
               sum_e2=torch.empty(1, dtype=torch.float64, device=dev))
    torch.cuda.synchronize()
    print(f"[bench] prepared {w.name} {m}x{n}", file=sys.stderr, flush=True)

    def step():
        bakron.quantize(W, LA, LB, kind=w.qkind, bits=w.qbits, order=args.order,
                        dev_status=status, workspace=ws, out=out, graph=not args.eager)

    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed / args.steps * 1e3
    value = m * n * args.steps / elapsed
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)
    if int(status.item()) != 0:
        raise SystemExit(f"device status {int(status.item())}")

    # ---- per-phase times from HIP events on the solver's stream
    bakron.quantize(W, LA, LB, kind=w.qkind, bits=w.qbits, order=args.order, dev_status=status,
                    workspace=ws, out=out, timing=True)
    ph = bakron.last_phase_ms()
    sched = bakron.schedule_info(m, n, args.order)
    # the band-GEMM kernel on the critical stream (the deferred products run in
    # band_side_kernel, reported apart).  Its average launch duration comes from
    # the timing call's replay of the critical band launches alone, as a graph
    # whose kernels start back to back, between two HIP events on the stream
    band_launches = ph["band_launches"]
    # a single tile diagonal (64 x 64) has no band launch: the band figures are null
    gemm_avg_s = ph["band_replay_ms"] / 1e3 / band_launches if band_launches else None
    # algorithmic flops of the band-GEMM launches: the useful multiply-adds of
    # their tiles (the zero halves of triangular diagonal factor blocks left
    # out); the two-diagonal nodes run inside the leaves and are not counted
    crit_useful = sched["useful_band_flops"] - sched["side_useful_flops"]
    assert band_launches == sched["band_launches"] - sched["side_launches"]
    gemm_alg_per_launch = crit_useful / band_launches if band_launches else None
    gemm_tflops = gemm_alg_per_launch / gemm_avg_s / 1e12 if band_launches else None
    side_tflops = (sched["side_useful_flops"] / (ph["side_replay_ms"] / 1e3) / 1e12
                   if ph["side_launches"] else None)
    leaf_avg_s = ph["leaf_ms"] / 1e3 / sched["leaf_launches"]
    # leaf algorithmic HBM bytes per entry: W tile in (4), E out (4), codes (1),
    # V (4), and the lower triangles of the two diagonal 64 x 64 factor blocks of
    # each tile (2 x 64 x 65 / 2 floats per 4096 entries, about 4)
    leaf_bytes = m * n * (4 + 4 + 1 + 4 + 2 * 4.0 * (64 * 65 / 2) / (64 * 64))
    leaf_gbs = leaf_bytes / sched["leaf_launches"] / leaf_avg_s / 1e9
    dominant = "band_gemm" if ph["band_ms"] >= ph["leaf_ms"] else "leaf"
    # HBM bytes per band-GEMM dispatch from the committed rocprofv3 counter
    # summary of this workload, null for workloads without one and unless it was
    # taken from the current kernel source
    from two_sided_gptq_amd import profsum
    profile_md = PROFILES.get(args.workload)
    profiled = profile_md is not None and args.order == 0 and not args.eager
    traffic = profsum.read_traffic(profile_md, "band_gemm_kernel") if profiled else None
    # MFMA utilisation from the same summary's counters: fp32 MFMA flops the
    # hardware counted per dispatch (executed, so the zero halves of triangular
    # blocks included) over this run's average launch duration, against the peak
    counted = (profsum.read_figure(profile_md, "mfma_flops_per_dispatch", "band_gemm_kernel")
               if profiled else None)
    mfma_util = counted / gemm_avg_s / 1e12 / FP32_MFMA_PEAK_TFLOPS if counted and gemm_avg_s else None
    roofline = {"kernel": "band_gemm_kernel", "bound": "mfma", "achieved": gemm_tflops,
                "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": gemm_tflops / FP32_MFMA_PEAK_TFLOPS if gemm_tflops else None,
                "traffic": traffic, "alg_flops_per_launch": gemm_alg_per_launch,
                "avg_launch_ms": gemm_avg_s * 1e3 if gemm_avg_s else None,
                "launches": band_launches, "counted_mfma_flops_per_launch": counted,
                "mfma_util_counted": mfma_util}

    phase_ms = ph["band_replay_ms"] + ph["side_replay_ms"]
    # null for a single tile diagonal, which has no band product
    phase_tflops = (sched["useful_band_flops"] / (phase_ms / 1e3) / 1e12
                    if band_launches and phase_ms > 0 else None)
    gemm_phase = {"useful_flops": sched["useful_band_flops"],
                  "critical_replay_ms": ph["band_replay_ms"], "deferred_replay_ms": ph["side_replay_ms"],
                  "tflops": phase_tflops,
                  "frac": phase_tflops / FP32_MFMA_PEAK_TFLOPS if phase_tflops else None}
    result = {
        "metric": "weight entries quantized/sec at 4096x4096 INT4; % of fp32 MFMA peak",
        "value": value, "unit": "entries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: {m}x{n} W, "
                               f"{['INT%d sym' % w.qbits, 'INT%d asym' % w.qbits, 'unit'][w.qkind]}, "
                               f"A from {w.n_x} samples, B from {w.n_y} samples",
                   "m": m, "n": n, "qkind": w.qkind, "qbits": w.qbits,
                   "order": int(sched["order"]), "tile": int(sched["tile"]),
                   "launch": "eager" if args.eager else "graph"},
        "roofline": roofline,
        "dominant_kernel": dominant,
        "gemm_pct_fp32_mfma_peak": 100.0 * gemm_tflops / FP32_MFMA_PEAK_TFLOPS if gemm_tflops else None,
        "whole_solve_tflops_alg": sched["alg_band_flops"] / (ms / 1e3) / 1e12,
        # phase times come from a separate timing pass that runs the same plan in
        # order on one stream; the timed graph overlaps the deferred products
        # (side_ms) with the leaves, so the phases add up to more than ms_per_step
        "phases_ms": {k: ph[k] for k in ("prep_ms", "leaf_ms", "band_ms", "side_ms", "final_ms")},
        # the whole band phase: every band product's useful flops (critical and
        # deferred) over the two replays' kernel time (critical launches back to
        # back, then the deferred launches alone on their capped CU share)
        "gemm_phase": gemm_phase,
        "side": {"kernel": "band_side_kernel", "launches": int(sched["side_launches"]),
                 "useful_flops": sched["side_useful_flops"],
                 "replay_ms": ph["side_replay_ms"], "tflops_alone": side_tflops},
        "leaf": {"launches": int(sched["leaf_launches"]), "in_kernel_steps": int(sched["leaf_steps"]),
                 "in_tile_flops": sched["leaf_flops"],
                 "valu_tflops": sched["leaf_flops"] / (ph["leaf_ms"] / 1e3) / 1e12,
                 "valu_frac": sched["leaf_flops"] / (ph["leaf_ms"] / 1e3) / 1e12 / FP32_VALU_PEAK_TFLOPS,
                 "avg_launch_ms": leaf_avg_s * 1e3, "alg_bytes": leaf_bytes,
                 "achieved_GBs": leaf_gbs, "hbm_frac": leaf_gbs / HBM_PEAK_GBS},
        "schedule": sched,
        "prep": prep,
        "hessian_ms": sum(v["ms"] for k, v in prep.items() if k.startswith("hessian")),
        "factor_ms": sum(v["ms"] for k, v in prep.items() if k.startswith("factor")),
    }
    if args.antidiag:
        # the pages' comparison (review page, "If this is right": BaKron about 27x
        # faster than BaKron-antidiagonal at 4096 x 4096): one antidiagonal solve
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        bakron.quantize_antidiag(W, LA, LB, kind=w.qkind, bits=w.qbits, dev_status=status)
        torch.cuda.synchronize()
        ad_ms = (time.perf_counter() - t0) * 1e3
        result["antidiag"] = {"ms": ad_ms, "ratio_vs_bakron": ad_ms / ms, "pages_ratio": 27}
        print(f"[bench] BaKron-antidiagonal: {ad_ms:.1f} ms ({ad_ms / ms:.0f}x)", file=sys.stderr, flush=True)
    if args.split:
        # the hybrid schedule (review page, "Circularity Check": BaKron-recursive's
        # split, Appendix C), timed like the main line
        result["split"] = {}
        for sp in (["cols", "rows"] if args.split == "both" else [args.split]):
            def split_step():
                bakron.quantize(W, LA, LB, kind=w.qkind, bits=w.qbits, order=args.order,
                                dev_status=status, workspace=ws, out=out, split=sp)
            for _ in range(args.warmup):
                split_step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                split_step()
            torch.cuda.synchronize()
            sp_ms = (time.perf_counter() - t0) / args.steps * 1e3
            result["split"][sp] = {"ms_per_step": sp_ms, "ratio_vs_bakron": sp_ms / ms}
            print(f"[bench] split {sp}: {sp_ms:.3f} ms/step ({sp_ms / ms:.2f}x)", file=sys.stderr, flush=True)
        if int(status.item()) != 0:
            raise SystemExit(f"device status {int(status.item())}")
    if args.cpu_sample > 0:
        LA_h = LA.cpu().numpy()
        LB_h = LB.cpu().numpy()
        result["cpu_baseline"] = cpu_baseline(W_h, LA_h, LB_h, w, min(args.cpu_sample, m, n))
    print(json.dumps(result))


if __name__ == "__main__":
    main()
