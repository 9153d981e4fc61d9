"""Host checks of the profile-summary helpers (no GPU)."""
from dense_fp16_gemm_nt_amd import profiling


def test_code_only_drops_comments_and_blank_lines():
    src = "int a;  // trailing\n\n/* block\n comment */ int b;\n// whole line\nint c; /* x */\n"
    assert profiling._code_only(src) == "int a;\n int b;\nint c;"


def test_source_hash_is_stable_and_short():
    h = profiling.kernel_source_hash()
    assert h == profiling.kernel_source_hash() and len(h) == 16 and int(h, 16) >= 0


def _write_trace(d, rows):
    d.mkdir(parents=True, exist_ok=True)
    with open(d / "run_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for name, st, en in rows:
            f.write(f'"{name}",{st},{en}\n')


def test_split_products_cuts_at_the_longest_gaps(tmp_path):
    """Two products timed in turn with the same kernel: the dispatches are
    cut at the long host gap between them, not at the short launch gaps."""
    rows = [("k<1>", 1000 * i, 1000 * i + 900) for i in range(5)]                       # 0.9 us each
    rows += [("k<1>", 10_000_000 + 2000 * i, 10_000_000 + 2000 * i + 1800) for i in range(3)]  # 1.8 us each
    rows += [("other", 50, 60)]
    _write_trace(tmp_path / "t", rows)
    out = profiling.split_products(str(tmp_path / "t"), "k<", ["small", "large"])
    assert [round(x, 3) for x in out[("k<1>", "small")]] == [0.9] * 5
    assert [round(x, 3) for x in out[("k<1>", "large")]] == [1.8] * 3


def test_counter_per_launch_sums_the_kernels_of_one_call(tmp_path):
    d = tmp_path / "c"
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i in range(4):   # each call: one "wide" and one "ring4" dispatch; values summed over XCDs
            f.write(f'{2 * i},"wide_kernel",FETCH_SIZE,30\n{2 * i},"wide_kernel",FETCH_SIZE,70\n')
            f.write(f'{2 * i + 1},"ring4_kernel",FETCH_SIZE,40\n')
    assert profiling.counter_per_dispatch(str(d), "FETCH_SIZE", "wide") == 100
    assert profiling.counter_per_launch(str(d), "FETCH_SIZE", "wide,ring4") == 140


def test_calibration_summary_reads_full_busy_for_a_saturated_kernel(tmp_path):
    """Synthetic counters for a kernel whose matrix cores are busy for the
    whole traced duration at the clock its waves measured: the summary
    reports 100% and the loop at its ideal cycle count."""
    import numpy as np

    d = tmp_path / "pmc"
    d.mkdir()
    clock, dur_ns, waves = 2.0, 1_000_000, 1024     # 2 GHz, 1 ms: 2e6 cycles per SIMD
    cycles = 2_000_000
    with open(d / "run_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i in range(2):
            for x in range(8):   # one value per XCD, summed per dispatch
                f.write(f'{i},"mfma_calib_kernel",SQ_VALU_MFMA_BUSY_CYCLES,{cycles * profiling.SIMDS / 8}\n')
    with open(d / "run_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for i in range(2):
            f.write(f'"mfma_calib_kernel",{10 * i * dur_ns},{10 * i * dur_ns + dur_ns}\n')
    stamps = np.zeros((2, waves, 3))
    stamps[:, :, 0] = cycles                       # shader cycles of the loop
    stamps[:, :, 1] = dur_ns / 10.0                # 100 MHz ticks
    np.save(tmp_path / "s.npy", stamps)
    out = tmp_path / "calib.txt"
    profiling.main(["calib", "--dir", str(d), "--stamps", str(tmp_path / "s.npy"), "--command", "x", "--out", str(out)])
    text = out.read_text()
    assert "busy_pct_mean: 100.00" in text
    assert " 1.0000" in text
