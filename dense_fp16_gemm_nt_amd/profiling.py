"""Summaries of rocprofv3 output for the GEMM kernels (short text files).

  python -m dense_fp16_gemm_nt_amd.profiling stats  --dir D --kernel SUBSTR --command CMD --out FILE
      per-kernel dispatch count and mean/median/min/max duration (one block
      per kernel name) from a `rocprofv3 --kernel-trace --stats
      --output-format csv` run
  python -m dense_fp16_gemm_nt_amd.profiling traffic --fetch D1 --write D2 --copy-fetch D3 --copy-write D4
      --copy-bytes N --kernel SUBSTR --workload NAME --rung NAME --command CMD --out FILE
      HBM bytes per dispatch of the kernel from FETCH_SIZE / WRITE_SIZE
      passes (KiB per dispatch), each scaled by what the same counter reads
      for a device copy of known size
  python -m dense_fp16_gemm_nt_amd.profiling power --steps N --workload NAME --command CMD --out FILE [--raw F]
      socket power and per-XCD shader clocks (amd-smi) sampled while
      bench.py runs N back-to-back launches in a child process (summary in
      FILE, the raw samples in F)
  python -m dense_fp16_gemm_nt_amd.profiling timeline --dir D --kernel SUBSTR --timed K --command CMD --out FILE
      per-dispatch durations and gaps of one kernel over a traced bench run
      whose last K dispatches are the timed region
  python -m dense_fp16_gemm_nt_amd.profiling counters --dir D --trace T --traffic F --flop X --kernel SUBSTR
      --workload NAME --rung NAME --cus N --command CMD --out FILE
      matrix-core and LDS figures per dispatch from one counter pass
      (SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_F16,
      SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE, SQ_BUSY_CU_CYCLES,
      GRBM_GUI_ACTIVE), the kernel's mean duration from a kernel trace
      and its HBM bytes from a traffic record
  python -m dense_fp16_gemm_nt_amd.profiling calib-run --out STAMPS.npy [--iters N] [--launches L]
      (on the GPU, under rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
      --kernel-trace) L launches of the MFMA-only calibration kernel
      (csrc/mfma_calib.hip) on every SIMD, saving each wave's shader-cycle
      and reference-clock counts
  python -m dense_fp16_gemm_nt_amd.profiling calib --dir D --stamps STAMPS.npy --command CMD --out FILE
      the busy fraction the GEMM summaries use (matrix-core cycles per SIMD
      over shader clock x traced duration) evaluated on that kernel, whose
      true busy fraction is ~1
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ["common.hpp", "sched.hpp", "ladder.hpp", "ring.hpp", "ring4.hpp", "ring4_sched.inc",
                  "ring_wide.hpp", "wide_sched.inc", "persistent_ws.hpp", "skinny.hpp", "gemm_f16_nt.hip"]


def _code_only(text: str) -> str:
    """Source text without comments and blank lines (the kernels' sources
    hold no comment markers inside string literals)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.split("\n") if ln.strip())


def kernel_source_hash() -> str:
    """Hash of the code (comments aside) of the sources the kernels are
    built from: a profile summary is current when it carries this hash."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dense_fp16_gemm_nt_amd", "csrc", name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _find(d: str, pattern: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return hits[0]


def kernel_stats(d: str, substr: str):
    rows = list(csv.DictReader(open(_find(d, "*kernel_trace.csv"))))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows if substr in r["Kernel_Name"]]
    names = sorted({r["Kernel_Name"] for r in rows if substr in r["Kernel_Name"]})
    return names, durs


def counter_per_dispatch(d: str, counter: str, substr: str) -> float:
    rows = list(csv.DictReader(open(_find(d, "*counter_collection.csv"))))
    per = {}
    for r in rows:
        if substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per.setdefault(r["Dispatch_Id"], 0.0)
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise ValueError(f"{counter} for {substr!r} not found in {d}")
    return statistics.mean(per.values())


def per_kernel(d: str, substr: str):
    """{kernel name: [durations in us, dispatch order]} for the kernels whose
    name contains substr."""
    rows = list(csv.DictReader(open(_find(d, "*kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    out = {}
    for r in rows:
        if substr in r["Kernel_Name"]:
            out.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return out


def split_products(d: str, substr: str, products: list):
    """{(kernel name, product): durations} for a run that timed several
    products one after another with the same kernel: each kernel's
    dispatches, in time order, are cut at its len(products) - 1 longest
    gaps (the host work between two products) and the runs are named in
    order."""
    rows = list(csv.DictReader(open(_find(d, "*kernel_trace.csv"))))
    rows = sorted((r for r in rows if substr in r["Kernel_Name"]), key=lambda r: int(r["Start_Timestamp"]))
    out = {}
    for name in sorted({r["Kernel_Name"] for r in rows}):
        rs = [r for r in rows if r["Kernel_Name"] == name]
        gaps = sorted(range(1, len(rs)), key=lambda i: int(rs[i - 1]["End_Timestamp"]) - int(rs[i]["Start_Timestamp"]))
        cuts = sorted(gaps[:len(products) - 1]) if len(rs) >= len(products) else []
        bounds = [0] + cuts + [len(rs)]
        for k, prod in enumerate(products[:len(bounds) - 1]):
            out[(name, prod)] = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                                 for r in rs[bounds[k]:bounds[k + 1]]]
    return out


def cmd_stats(a):
    """One block of figures per kernel name (never one mean over different
    kernels), and per product when --products names the products a run
    timed in turn."""
    if a.products:
        groups = {f"{name}\nproduct: {prod}": durs
                  for (name, prod), durs in split_products(a.dir, a.kernel, a.products.split(",")).items()}
    else:
        groups = per_kernel(a.dir, a.kernel)
    if not groups:
        raise SystemExit(f"no dispatch of a kernel matching {a.kernel!r} in {a.dir}")
    lines = [f"# rocprofv3 kernel trace summary: kernels matching {a.kernel!r}",
             f"command: {a.command}",
             f"kernel_src_sha: {kernel_source_hash()}"]
    for name, durs in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines += ["",
                  f"kernel: {name}",
                  f"dispatches: {len(durs)}",
                  f"mean_us: {statistics.mean(durs):.3f}",
                  f"median_us: {statistics.median(durs):.3f}",
                  f"min_us: {min(durs):.3f}",
                  f"max_us: {max(durs):.3f}"]
    stats_csv = glob.glob(os.path.join(a.dir, "**", "*kernel_stats.csv"), recursive=True)
    if stats_csv:
        lines.append("")
        lines.append("## rocprofv3 --stats (kernel_stats.csv rows" +
                     (", rocprofv3's own per-kernel totals over every product above)" if a.products else ")"))
        for r in csv.DictReader(open(stats_csv[0])):
            lines.append(", ".join(f"{k}={v}" for k, v in r.items()))
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines[:12]))


def cmd_timeline(a):
    """Per-dispatch durations and the gaps between dispatches of one kernel
    over a traced bench run: the last `timed` dispatches are the timed
    region, the ones before them the warm-up launches."""
    rows = list(csv.DictReader(open(_find(a.dir, "*kernel_trace.csv"))))
    rows = [r for r in rows if a.kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    if len(rows) < a.timed:
        raise SystemExit(f"{len(rows)} dispatches, fewer than the {a.timed} timed ones")
    t0 = int(rows[0]["Start_Timestamp"])
    lines = [f"# rocprofv3 per-dispatch timeline: {a.kernel}",
             f"command: {a.command}",
             f"kernel_src_sha: {kernel_source_hash()}",
             f"dispatches: {len(rows)} (the last {a.timed} are the timed region)",
             "",
             "index  start_us  duration_us  gap_before_us  region"]
    prev_end = None
    durs, gaps = [], []
    for i, r in enumerate(rows):
        st, en = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        gap = (st - prev_end) / 1e3 if prev_end is not None else 0.0
        timed = i >= len(rows) - a.timed
        lines.append(f"{i:5d}  {(st - t0) / 1e3:8.1f}  {(en - st) / 1e3:11.3f}  {gap:13.3f}  "
                     f"{'timed' if timed else 'warm-up'}")
        if timed:
            durs.append((en - st) / 1e3)
            if i > len(rows) - a.timed:
                gaps.append(gap)
        prev_end = en
    span = (int(rows[-1]["End_Timestamp"]) - int(rows[len(rows) - a.timed]["Start_Timestamp"])) / 1e3
    lines += ["",
              f"timed_mean_duration_us: {statistics.mean(durs):.3f}",
              f"timed_first_half_mean_us: {statistics.mean(durs[:len(durs) // 2]):.3f}",
              f"timed_second_half_mean_us: {statistics.mean(durs[len(durs) // 2:]):.3f}",
              f"timed_gap_total_us: {sum(gaps):.3f}",
              f"timed_span_first_start_to_last_end_us: {span:.3f}",
              f"timed_span_per_dispatch_us: {span / a.timed:.3f}"]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines[-7:]))


def counter_per_launch(d: str, counter: str, kernels: str) -> float:
    """A counter per library call whose launches are the kernels named by
    the comma-separated substrings (one dispatch of each per call): the
    sum of each kernel's mean per dispatch."""
    return sum(counter_per_dispatch(d, counter, k) for k in kernels.split(","))


def cmd_traffic(a):
    fetch_k = counter_per_launch(a.fetch, "FETCH_SIZE", a.kernel)
    write_k = counter_per_launch(a.write, "WRITE_SIZE", a.kernel)
    copy_fetch_k = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    copy_write_k = counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    f_scale = a.copy_bytes / (copy_fetch_k * 1024.0)
    w_scale = a.copy_bytes / (copy_write_k * 1024.0)
    rec = {
        "workload": a.workload, "rung": a.rung, "kernel": a.kernel,
        "fetch_kib_per_dispatch": fetch_k, "write_kib_per_dispatch": write_k,
        "copy_bytes": a.copy_bytes, "copy_fetch_kib": copy_fetch_k, "copy_write_kib": copy_write_k,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "hbm_bytes_per_launch": fetch_k * 1024.0 * f_scale + write_k * 1024.0 * w_scale,
        "kernel_src_sha": kernel_source_hash(),
        "command": a.command,
    }
    open(a.out, "w").write(json.dumps(rec, indent=1) + "\n")
    print(json.dumps(rec, indent=1))


COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
            "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"]
XCDS = 8            # GRBM_GUI_ACTIVE is summed over the 8 XCDs
SIMDS_PER_CU = 4


def cmd_counters(a):
    c = {name: counter_per_launch(a.dir, name, a.kernel) for name in COUNTERS}
    # one library call: the sum of its kernels' mean durations
    mean_s = sum(statistics.mean(kernel_stats(a.trace, k)[1]) for k in a.kernel.split(",")) * 1e-6
    gui = c["GRBM_GUI_ACTIVE"] / XCDS                 # shader-clock cycles of the dispatch
    simds = a.cus * SIMDS_PER_CU
    traffic = json.load(open(a.traffic))
    rec = {
        "workload": a.workload, "rung": a.rung, "kernel": a.kernel, "flop_per_dispatch": a.flop,
        "counters_per_dispatch": c,
        # matrix-core busy cycles over the SIMD-cycles the graphics engine
        # was active in the dispatch's counter window (GRBM_GUI_ACTIVE: its
        # cycles span more than the kernel's own duration, so this is a
        # lower bound on the busy fraction of the kernel itself)
        "mfma_busy_pct": 100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * simds),
        # MFMA FLOPs the hardware counted (equal to 2*M*N*K when every MFMA
        # of the product ran exactly once)
        "mfma_flop_counted": c["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512,
        "mfma_cycles_per_instruction": c["SQ_VALU_MFMA_BUSY_CYCLES"] / max(c["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512 / 16384, 1.0),
        "lds_bank_conflict_pct": 100.0 * c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_LDS_IDX_ACTIVE"], 1.0),
        # matrix-core cycles per SIMD over the traced kernel duration: the
        # shader clock at which the MFMAs alone would fill the kernel.  The
        # kernel's own busy fraction is this over the clock it ran at (the
        # counter is exactly 16 cycles per 16x16x32 MFMA, so the clock is the
        # only measured quantity in it)
        "mfma_cycles_per_simd": c["SQ_VALU_MFMA_BUSY_CYCLES"] / simds,
        "mfma_floor_clock_ghz": c["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / (mean_s * 1e9),
        "kernel_mean_us_trace": mean_s * 1e6,
        "hbm_bytes_per_launch": traffic["hbm_bytes_per_launch"],
        "hbm_gbs": traffic["hbm_bytes_per_launch"] / mean_s / 1e9,
        "kernel_src_sha": kernel_source_hash(),
        "command": a.command,
    }
    open(a.out, "w").write(json.dumps(rec, indent=1) + "\n")
    print(json.dumps(rec, indent=1))


def _smi_sample():
    """Socket power (W) and the per-XCD shader clocks (MHz) of GPU 0 from
    one `amd-smi metric -p -c --json` call."""
    out = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                         timeout=30).stdout
    d = json.loads(out)
    g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
    clocks = g["clock"]
    gfx = [clocks[f"gfx_{i}"]["clk"]["value"] for i in range(XCDS) if isinstance(clocks.get(f"gfx_{i}", {}).get("clk"), dict)]
    return g["power"]["socket_power"]["value"], gfx


def cmd_power(a):
    """Run the bench (a child process: this one never touches the GPU) and
    sample the board's socket power and per-XCD clocks while it runs."""
    if a.product:
        # one extra product, timed by the suite for about `seconds`
        cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--suite", "--only", a.product, "--rung", str(a.rung),
               "--seconds", str(a.seconds)]
    else:
        cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", str(a.steps), "--warmup", "100",
               "--no-cpu-baseline", "--workload", a.workload, "--rung", str(a.rung)]
    child = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    samples = []
    t0 = time.time()
    while child.poll() is None and len(samples) < a.samples + 64:
        try:
            samples.append((round(time.time() - t0, 2),) + _smi_sample())
        except (subprocess.SubprocessError, ValueError, KeyError, IndexError, TypeError):
            pass
        time.sleep(a.interval)
    out, err = child.communicate()
    if child.returncode != 0:
        raise SystemExit(f"bench failed ({child.returncode}): {err[-2000:]}")
    bench = json.loads(out.strip().splitlines()[-1])
    # samples taken under load: power within 25% of the highest sample
    top = max(p for _, p, _ in samples)
    busy = [x for x in samples if x[1] >= 0.75 * top]
    clocks = [statistics.mean(c[i] for _, _, c in busy) for i in range(len(busy[0][2]))] if busy else []
    ms = bench["ms_per_step"] if "ms_per_step" in bench else bench["us_per_launch"] / 1e3
    rec = {
        "workload": a.product or a.workload, "rung": a.rung, "bench_value_tflops": bench["value"],
        "bench_ms_per_step": ms, "bench_steps": bench["steps"],
        "samples_under_load": len(busy), "samples_total": len(samples),
        "socket_power_w_mean": round(statistics.mean(p for _, p, _ in busy), 1),
        "socket_power_w_min": min(p for _, p, _ in busy), "socket_power_w_max": max(p for _, p, _ in busy),
        "xcd_clock_mhz_mean": [round(c) for c in clocks],
        "clock_mhz_mean_all_xcds": round(statistics.mean(clocks), 1) if clocks else None,
        "kernel_src_sha": kernel_source_hash(),
        "command": a.command,
    }
    open(a.out, "w").write(json.dumps(rec, indent=1) + "\n")
    if a.raw:
        # the raw samples (time s, socket power W, per-XCD clocks MHz) go
        # to a file of their own, outside the summaries
        open(a.raw, "w").write(json.dumps(samples) + "\n")
    print(json.dumps(rec, indent=1))


SIMDS = 1024            # 256 compute units x 4 SIMDs
CALIB_WAVES_PER_BLOCK = 4
CALIB_CYCLES_PER_TRIP = 128 * 16   # 128 v_mfma_f32_16x16x32_f16 of 16 cycles


def calib_source_hash() -> str:
    with open(os.path.join(ROOT, "dense_fp16_gemm_nt_amd", "csrc", "mfma_calib.hip")) as f:
        return hashlib.sha256(_code_only(f.read()).encode()).hexdigest()[:16]


def calib_lib():
    import ctypes

    path = os.path.join(ROOT, "dense_fp16_gemm_nt_amd", "libmfma_calib.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built: python -c 'import __graft_entry__ as g; g.build()'")
    L = ctypes.CDLL(path)
    L.mfma_calib_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return L


def cmd_calib_run(a):
    """Launch the calibration kernel on one workgroup of 4 waves per compute
    unit and save the per-wave stamps (launch, wave, [cycles, ticks, sum])."""
    import numpy as np
    import torch

    L = calib_lib()
    dev = torch.device("cuda:0")
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    waves = blocks * CALIB_WAVES_PER_BLOCK
    # random fp16 operands in [-1, 1): the matrix cores' power depends on the data
    rnd = (torch.rand(waves * 8192, device=dev) * 2 - 1).half()
    out = torch.zeros(a.launches * waves * 3, dtype=torch.int64, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    for i in range(a.launches):
        st = L.mfma_calib_launch(blocks, rnd.data_ptr(), out.data_ptr() + i * waves * 3 * 8, a.iters, s)
        if st != 0:
            raise SystemExit(f"mfma_calib_launch returned {st}")
    torch.cuda.synchronize()
    np.save(a.out, out.cpu().numpy().reshape(a.launches, waves, 3))
    print(f"[calib] {a.launches} launches of {blocks} x {CALIB_WAVES_PER_BLOCK} waves, {a.iters} trips", flush=True)


def cmd_calib(a):
    import numpy as np

    stamps = np.load(a.stamps).astype(np.float64)            # (launches, waves, 3)
    rows = list(csv.DictReader(open(_find(a.dir, "*counter_collection.csv"))))
    per = {}
    for r in rows:
        if "mfma_calib" in r["Kernel_Name"] and r["Counter_Name"] == "SQ_VALU_MFMA_BUSY_CYCLES":
            per.setdefault(int(r["Dispatch_Id"]), 0.0)
            per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    trace = sorted((r for r in csv.DictReader(open(_find(a.dir, "*kernel_trace.csv")))
                    if "mfma_calib" in r["Kernel_Name"]), key=lambda r: int(r["Start_Timestamp"]))
    busy_cycles = [per[k] for k in sorted(per)]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9 for r in trace]
    n = min(len(busy_cycles), len(durs), stamps.shape[0])
    if n == 0:
        raise SystemExit(f"no calibration dispatch with counters in {a.dir}")
    lines = ["# Matrix-core busy calibration: the MFMA-only kernel (csrc/mfma_calib.hip) on every SIMD",
             f"command: {a.command}", f"calib_src_sha: {calib_source_hash()}", "",
             "launch  duration_us  clock_ghz (waves' min-max)  busy_cycles_per_simd  busy_pct  loop_cycles_per_ideal"]
    fr = []
    for i in range(n):
        cyc, ticks = stamps[i, :, 0], stamps[i, :, 1]
        clock = float(np.median(cyc / (ticks * 10.0)))          # GHz: 100 MHz reference ticks
        per_simd = busy_cycles[i] / SIMDS
        busy = per_simd / (clock * 1e9 * durs[i])
        trips = per_simd / CALIB_CYCLES_PER_TRIP
        ideal = float(np.median(cyc)) / (trips * CALIB_CYCLES_PER_TRIP)
        fr.append(busy)
        ck = cyc / (ticks * 10.0)
        lines.append(f"{i:6d}  {durs[i] * 1e6:11.1f}  {clock:9.3f} ({ck.min():.3f}-{ck.max():.3f})"
                     f"  {per_simd:20.0f}  {100 * busy:8.2f}  {ideal:21.4f}")
    lines += ["", f"busy_pct_mean: {100 * statistics.mean(fr):.2f}",
              "(busy_pct = matrix-core cycles per SIMD / (the clock the waves measured x the traced duration);"
              " loop_cycles_per_ideal = the waves' own loop cycles over the MFMA cycles they issued)"]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--dir", required=True)
    s.add_argument("--kernel", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--products", default="", help="comma-separated names of the products the run timed in turn")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--kernel", required=True, help="comma-separated name substrings: the kernels one call launches")
    t.add_argument("--workload", required=True)
    t.add_argument("--rung", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--dir", required=True)
    c.add_argument("--trace", required=True)
    c.add_argument("--traffic", required=True)
    c.add_argument("--flop", type=float, required=True)
    c.add_argument("--cus", type=int, required=True)
    c.add_argument("--kernel", required=True, help="comma-separated name substrings: the kernels one call launches")
    c.add_argument("--workload", required=True)
    c.add_argument("--rung", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--out", required=True)
    w = sub.add_parser("power")
    w.add_argument("--steps", type=int, default=100000)
    w.add_argument("--workload", default="square_4096")
    w.add_argument("--rung", type=int, default=0, help="0 = the library's choice")
    w.add_argument("--product", default="", help="an extra product of bench.py --suite instead of a workload")
    w.add_argument("--seconds", type=float, default=12.0, help="suite seconds for --product")
    w.add_argument("--samples", type=int, default=16)
    w.add_argument("--interval", type=float, default=0.4)
    w.add_argument("--command", required=True)
    w.add_argument("--out", required=True)
    w.add_argument("--raw", default="", help="file for the raw amd-smi samples")
    tl = sub.add_parser("timeline")
    tl.add_argument("--dir", required=True)
    tl.add_argument("--kernel", required=True)
    tl.add_argument("--timed", type=int, required=True)
    tl.add_argument("--command", required=True)
    tl.add_argument("--out", required=True)
    cr = sub.add_parser("calib-run")
    cr.add_argument("--out", required=True)
    cr.add_argument("--iters", type=int, default=1000)
    cr.add_argument("--launches", type=int, default=12)
    cb = sub.add_parser("calib")
    cb.add_argument("--dir", required=True)
    cb.add_argument("--stamps", required=True)
    cb.add_argument("--command", required=True)
    cb.add_argument("--out", required=True)
    a = p.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters, "power": cmd_power,
     "timeline": cmd_timeline, "calib-run": cmd_calib_run, "calib": cmd_calib}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())
