#!/usr/bin/env python3
"""Benchmark of the fp16 NT GEMM (D = A * B^T) on one MI355X.

One step = one call of the library on one batch of synthetic operands
(inputs generated from the workload's seed and already resident in HBM when
the timed region starts).  Prints one JSON line:

  value       whole-run throughput, TFLOP/s = 2*M*N*K*steps / timed seconds
              (K host launches; --launch graph captures the K steps once
              into a HIP graph and times its replay)
  roofline    the GEMM kernel against the dense-fp16 MFMA peak: achieved =
              2*M*N*K / mean launch duration (HIP events bracketing the timed
              region on the launch stream, divided by the number of
              back-to-back launches), traffic = HBM bytes per launch from the
              committed rocprofv3 counter summary when it matches the
              current kernel sources, else null; counters = the committed
              matrix-core, LDS and HBM figures under the same condition
              (mfma_busy_pct: the kernel's own busy fraction, its MFMA
              cycles over the traced duration at the shader clock of a long
              run of the same box)
  cpu_baseline  the CPU oracle timed on the host cores on a bounded sample
              (a block of full output rows), scaled to TFLOP/s

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload NAME] [--rung R] [--no-cpu-baseline]
       python bench.py --suite [--only NAME,...] [--seconds S] [--rung R]
                                      (one JSON line per product beyond the
                                       five fixed workloads: ragged and
                                       unaligned shapes, batches, attention
                                       scores; each against its own roofline)
       python bench.py --copy-calib   (a plain device copy of known size, for
                                       scaling the HBM byte counters)
       python bench.py --library-gemm [--workload NAME] [--steps K]
                                      (context: the platform's GEMM on the
                                       same inputs; one JSON line)
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2516.6   # MI355X dense fp16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/CU/clk
HBM_PEAK_GBS = 8000.0
METRIC = "fp16 GEMM TFLOP/s at M=N=K=4096 (+ % of MI355X dense-fp16 peak)"
RUNG_NAMES = {0: "auto", 1: "r1_single_tile", 2: "r2_kloop", 3: "r3_grid", 4: "r4_ring",
              5: "r5_persistent_ws", 8: "r8_ring4_gap", 9: "r9_ring_small", 10: "r10_ring4_paired",
              11: "r11_wide", 12: "r12_skinny", 13: "r13_ksplit"}


def kernel_source_hash() -> str:
    from dense_fp16_gemm_nt_amd.profiling import kernel_source_hash as h

    return h()


def traffic_record(workload: str, rung_name: str):
    """HBM bytes per launch from profiles/traffic_<rung>_<workload>.txt (a
    JSON record written by dense_fp16_gemm_nt_amd.profiling from two
    rocprofv3 counter passes) if it was taken on the current kernel
    sources, else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{rung_name}_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha") != kernel_source_hash() or rec.get("rung") != rung_name:
        return None
    return rec.get("hbm_bytes_per_launch")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="square_4096")
    p.add_argument("--rung", type=int, default=0, choices=sorted(RUNG_NAMES), help="0 = library choice, else a ladder rung")
    p.add_argument("--splitk", type=int, default=-1,
                   help="time gemm_f16_nt_splitk with this many K slices (0 = library choice)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU sample")
    p.add_argument("--copy-calib", action="store_true", help="run only a plain device copy (counter scaling)")
    p.add_argument("--library-gemm", action="store_true",
                   help="context only: time torch.matmul (hipBLASLt) on the workload (a fixed workload or a "
                        "single extra product) instead of this library")
    p.add_argument("--launch", choices=("graph", "host"), default="host",
                   help="time the K steps as K host launches (default) or as one captured HIP graph")
    p.add_argument("--suite", action="store_true", help="time the extra products (general shapes, attention scores)")
    p.add_argument("--only", default="", help="comma-separated extra product names for --suite")
    p.add_argument("--seconds", type=float, default=0.3, help="timed seconds per extra product")
    return p.parse_args()


def copy_calib():
    import torch

    n = 256 << 20  # bytes
    src = torch.empty(n // 2, dtype=torch.float16, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes_read": n, "copy_calib_bytes_written": n, "launches": 5}), flush=True)


def library_gemm(args):
    """Context only: the platform's GEMM (torch.matmul -> hipBLASLt) on the
    same workload, inputs and launch pattern (warm-up launches, then the
    timed launches bracketed by events on the launch stream).  Its output is
    compared with this library's, which is not timed here."""
    import numpy as np
    import torch

    import dense_fp16_gemm_nt_amd as g
    from dense_fp16_gemm_nt_amd import inputs, workloads

    w = workloads.BY_NAME.get(args.workload) or workloads.EXTRA_BY_NAME[args.workload]
    if getattr(w, "kind", "gemm") != "gemm":
        raise SystemExit(f"{w.name}: --library-gemm takes a single product")
    M, N, K, seed, dist = w.M, w.N, w.K, w.seed, w.dist
    dev = torch.device("cuda:0")
    A_np, B_np = inputs.operands(M, N, K, seed, dist)
    A, B = torch.from_numpy(A_np).to(dev), torch.from_numpy(B_np).to(dev)
    stream = torch.cuda.current_stream(dev)
    Bt = B.t()
    out = torch.empty((M, N), dtype=torch.float16, device=dev)
    for _ in range(args.warmup):
        torch.matmul(A, Bt, out=out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        torch.matmul(A, Bt, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    mine = g.gemm_f16_nt(A, B)
    torch.cuda.synchronize()
    diff = (mine.float() - out.float()).abs()
    flop = 2.0 * M * N * K
    print(json.dumps({
        "context": "torch.matmul (hipBLASLt), not this library", "workload": args.workload, "M": M, "N": N, "K": K,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "value": round(flop / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "outputs_bitwise_equal_to_this_library": bool(torch.equal(mine.view(torch.int16), out.view(torch.int16))),
        "max_abs_diff": float(diff.max().item()), "outputs_differing": int((diff > 0).sum().item()),
    }), flush=True)


def cpu_baseline(A, B, D_gpu_bits, w, target_s):
    """Time the oracle on the first R full output rows (R sized to about
    target_s seconds of work on the host's cores) and check those rows of
    the GPU result against it."""
    import numpy as np

    import oracle
    from tests.parity import compare

    rows = 8
    t0 = time.perf_counter()
    _, threads = oracle.gemm_nt(A[:rows], B)
    dt = time.perf_counter() - t0
    rows = int(max(8, min(w.M, rows * target_s / max(dt, 1e-6))))
    t0 = time.perf_counter()
    ref, threads = oracle.gemm_nt(A[:rows], B)
    dt = time.perf_counter() - t0
    ok, worst, nbad, _ = compare(D_gpu_bits[:rows], ref, w.K)
    flop = 2.0 * rows * w.N * w.K
    return {
        "value": round(flop / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"first {rows} of {w.M} output rows x all {w.N} columns, K={w.K} "
                  f"({rows * w.N} dot products, fp64 accumulation), {dt:.1f} s",
        "seconds": round(dt, 3),
        "gpu_rows_match_oracle": bool(ok),
        "gpu_rows_worst_err_over_tol": round(worst, 4),
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def counter_record(workload: str, rung_name: str):
    """Matrix-core, LDS and HBM figures from profiles/counters_<rung>_<workload>.txt
    (dense_fp16_gemm_nt_amd.profiling counters) if taken on the current
    kernel sources, else None."""
    path = os.path.join(ROOT, "profiles", f"counters_{rung_name}_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha") != kernel_source_hash() or rec.get("rung") != rung_name:
        return None
    out = {"mfma_flop_counted": rec["mfma_flop_counted"], "lds_bank_conflict_pct": round(rec["lds_bank_conflict_pct"], 3),
           "hbm_gbs": round(rec["hbm_gbs"], 1),
           # the clock at which the counted MFMA cycles alone fill the traced
           # kernel time; over the shader clock of a long run of the same
           # box (profiles/power_clock_*), the kernel's own busy fraction
           "mfma_floor_clock_ghz": round(rec["mfma_floor_clock_ghz"], 4),
           # busy cycles over the graphics engine's active window, which is
           # longer than the kernel: a lower bound
           "mfma_busy_pct_lower_bound": round(rec["mfma_busy_pct"], 2)}
    ppath = os.path.join(ROOT, "profiles", f"power_clock_{rung_name}_{workload}.txt")
    if os.path.exists(ppath):
        with open(ppath) as f:
            pw = json.load(f)
        if pw.get("kernel_src_sha") == kernel_source_hash() and pw.get("clock_mhz_mean_all_xcds"):
            clk = pw["clock_mhz_mean_all_xcds"] / 1e3
            out["long_run_clock_ghz"] = round(clk, 4)
            out["mfma_busy_pct"] = round(100.0 * rec["mfma_floor_clock_ghz"] / clk, 2)
    return out


def suite(args):
    """One JSON line per extra product.  Each is timed like the headline
    (warm-up launches, then back-to-back launches bracketed by events on
    the launch stream) and placed against the roofline its arithmetic
    intensity selects: 2*b*M*N*K FLOPs over the compulsory bytes
    2*b*(MK + NK + MN); below the ridge (peak FLOP/s over 8 TB/s) the
    bound is HBM."""
    import numpy as np
    import torch

    import dense_fp16_gemm_nt_amd as g
    from dense_fp16_gemm_nt_amd import inputs, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    s_ptr = ctypes.c_void_p(stream.cuda_stream)
    L = g.lib()
    ridge = PEAK_FP16_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    chosen = [n for n in args.only.split(",") if n] or [w.name for w in workloads.EXTRA_WORKLOADS]
    for name in chosen:
        w = workloads.EXTRA_BY_NAME[name]
        print(f"[bench] {w.describe()}", file=sys.stderr, flush=True)
        A3, B3 = inputs.batched_operands(w.batch, w.M, w.N, w.K, w.seed, w.dist)
        if w.kind == "heads_rows":
            # (S, H, d) storage: row s of head h starts at (s*H + h)*d
            A = torch.from_numpy(np.ascontiguousarray(A3.transpose(1, 0, 2))).to(dev)
            B = torch.from_numpy(np.ascontiguousarray(B3.transpose(1, 0, 2))).to(dev)
            lda, sa, ldb, sb = w.batch * w.K, w.K, w.batch * w.K, w.K
        else:
            A = torch.from_numpy(A3).to(dev)
            B = torch.from_numpy(B3).to(dev)
            lda, sa, ldb, sb = w.K, w.M * w.K, w.K, w.N * w.K
        D = torch.empty((w.batch, w.M, w.N), dtype=torch.float16, device=dev)
        a, b, d = A.data_ptr(), B.data_ptr(), D.data_ptr()
        if w.kind == "gemm" and args.rung:
            def step():
                return L.gemm_f16_nt_rung(args.rung, w.M, w.N, w.K, a, b, d, s_ptr)
        elif args.rung:
            raise SystemExit(f"{name}: --rung applies to the single products (kind gemm), not to {w.kind}")
        elif w.kind == "gemm":
            def step():
                return L.gemm_f16_nt(w.M, w.N, w.K, a, b, d, s_ptr)
        elif w.kind == "splitk":
            ws_bytes = max(16, g.splitk_workspace_bytes(w.M, w.N, w.K, 0))
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

            def step():
                return L.gemm_f16_nt_splitk(w.M, w.N, w.K, a, b, d, 0, ws.data_ptr(), ws_bytes, s_ptr)
        else:
            def step():
                return L.gemm_f16_nt_strided_batched(w.M, w.N, w.K, a, lda, sa, b, ldb, sb, d, w.N, w.M * w.N,
                                                     w.batch, s_ptr)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        bad = 0
        for _ in range(10):
            bad |= step()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(10):
            bad |= step()
        e1.record(stream)
        torch.cuda.synchronize()
        est = e0.elapsed_time(e1) / 10 * 1e-3
        steps = int(min(1_000_000, max(20, args.seconds / max(est, 1e-6))))
        for _ in range(steps // 4):
            bad |= step()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            bad |= step()
        e1.record(stream)
        torch.cuda.synchronize()
        if bad:
            raise SystemExit(f"{name}: the library returned an error")
        launch_s = e0.elapsed_time(e1) * 1e-3 / steps
        tflops = w.flop / launch_s / 1e12
        gbs = w.min_bytes / launch_s / 1e9
        if w.flop / w.min_bytes < ridge:
            roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4)}
            # context: the same output written by torch's fill kernel (a
            # plain store stream, no reads), as a practical write ceiling
            reps = max(5, steps // 4)
            for _ in range(reps // 2):
                D.fill_(0.0)
            e0.record(stream)
            for _ in range(reps):
                D.fill_(0.0)
            e1.record(stream)
            torch.cuda.synchronize()
            fill_gbs = D.numel() * 2 / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e9
            roof["fill_gbs_same_output"] = round(fill_gbs, 1)
        else:
            roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / PEAK_FP16_TFLOPS, 4)}
        roof["traffic"] = None
        roof["kernel_src_sha"] = kernel_source_hash()
        extra = {}
        if w.kind == "splitk":
            # context: the same product on gemm_f16_nt (no split)
            def plain():
                return L.gemm_f16_nt(w.M, w.N, w.K, a, b, d, s_ptr)
            for _ in range(max(3, steps // 10)):
                bad |= plain()
            e0.record(stream)
            for _ in range(steps):
                bad |= plain()
            e1.record(stream)
            torch.cuda.synchronize()
            if bad:
                raise SystemExit(f"{name}: gemm_f16_nt returned an error")
            m_top, sl = g.splitk_plan(w.M, w.N, w.K, torch.cuda.get_device_properties(dev).multi_processor_count)
            extra = {"plain_us_per_launch": round(e0.elapsed_time(e1) * 1e3 / steps, 3), "rows_unsplit": m_top,
                     "slices": sl}
        print(json.dumps({
            "suite": "extra", "workload": w.name, "kind": w.kind, "batch": w.batch, "M": w.M, "N": w.N, "K": w.K,
            "kernel": RUNG_NAMES[args.rung],
            "value": round(tflops, 2), "unit": "TFLOP/s", "us_per_launch": round(launch_s * 1e6, 3),
            "steps": steps, "compulsory_bytes": w.min_bytes, "compulsory_gbs": round(gbs, 1),
            "flop_per_byte": round(w.flop / w.min_bytes, 2), "roofline": roof, "dtype": "f16",
            "data": "synthetic", **extra}), flush=True)
        del A, B, D
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on exactly one GPU (got --gpus {args.gpus}); "
              "it does not shard a GEMM across GPUs.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calib:
        copy_calib()
        return
    if args.suite:
        suite(args)
        return
    if args.library_gemm:
        library_gemm(args)
        return

    import numpy as np
    import torch

    import dense_fp16_gemm_nt_amd as g
    from dense_fp16_gemm_nt_amd import inputs, workloads

    w = workloads.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] {w.describe()} rung={RUNG_NAMES[args.rung]} splitk={args.splitk} warmup={args.warmup} "
          f"steps={args.steps}",
          file=sys.stderr, flush=True)
    A_np, B_np = inputs.operands(w.M, w.N, w.K, w.seed, w.dist)
    A = torch.from_numpy(A_np).to(dev)
    B = torch.from_numpy(B_np).to(dev)
    D = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)

    L = g.lib()
    a_ptr, b_ptr, d_ptr = A.data_ptr(), B.data_ptr(), D.data_ptr()
    s_ptr = ctypes.c_void_p(stream.cuda_stream)
    if args.splitk >= 0:
        ws_bytes = max(16, g.splitk_workspace_bytes(w.M, w.N, w.K, args.splitk))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def step(sp):
            return L.gemm_f16_nt_splitk(w.M, w.N, w.K, a_ptr, b_ptr, d_ptr, args.splitk, ws.data_ptr(), ws_bytes, sp)
    elif args.rung == 0:
        def step(sp):
            return L.gemm_f16_nt(w.M, w.N, w.K, a_ptr, b_ptr, d_ptr, sp)
    else:
        def step(sp):
            return L.gemm_f16_nt_rung(args.rung, w.M, w.N, w.K, a_ptr, b_ptr, d_ptr, sp)

    for _ in range(args.warmup):
        if step(s_ptr) != 0:
            raise SystemExit("gemm_f16_nt returned an error")
    torch.cuda.synchronize()

    bad = 0
    graph = None
    if args.launch == "graph":
        # the K timed steps, captured once into one HIP graph (the same
        # launches, replayed without a host call per step)
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            bad |= step(ctypes.c_void_p(side.cuda_stream))
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
            for _ in range(args.steps):
                bad |= step(cap)
        torch.cuda.synchronize()
        if bad:
            raise SystemExit("gemm_f16_nt returned an error while captured")

    # timed region: bracketed by events on the launch stream, with the
    # device synchronised on both sides
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            bad |= step(s_ptr)
    region1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if bad:
        raise SystemExit("gemm_f16_nt returned an error")
    region_ms = region0.elapsed_time(region1)
    kernel_ms = region_ms / args.steps      # mean launch duration over the region

    flop = float(w.flop)
    value = flop * args.steps / (region_ms * 1e-3) / 1e12
    achieved = flop / (kernel_ms * 1e-3) / 1e12
    rung_name = RUNG_NAMES[args.rung] if args.splitk < 0 else f"splitk{args.splitk}"
    traffic = traffic_record(w.name, rung_name)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(region_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "M": w.M, "N": w.N, "K": w.K, "seed": w.seed,
            "dist": w.dist, "layout": "A MxK row-major, B NxK row-major, D MxN row-major",
            "accumulate": "f32", "kernel": rung_name,
            "launch": "one HIP graph of the K steps" if graph is not None else "K host launches",
        },
        "pct_of_peak": round(100.0 * value / PEAK_FP16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_FP16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
            "traffic": traffic,
            "counters": counter_record(w.name, rung_name),
            "kernel_mean_ms": round(kernel_ms, 5),
            "kernel_src_sha": kernel_source_hash(),
        },
        "wall_s": round(wall, 4),
    }
    props = torch.cuda.get_device_properties(dev)
    out["device"] = {"name": props.name, "cus": props.multi_processor_count,
                     "arch": getattr(props, "gcnArchName", "?")}
    if not args.no_cpu_baseline:
        D_bits = D.cpu().view(torch.int16).numpy().view(np.uint16)
        out["cpu_baseline"] = cpu_baseline(A_np, B_np, D_bits, w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
