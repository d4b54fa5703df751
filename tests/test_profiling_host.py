"""Counter summaries of rocprofv3 CSV output (CPU only, synthetic files)."""

import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from block_sparse_video_fp32_amd import profiling  # noqa: E402

KERNEL = "void sa::(anonymous namespace)::attend_kernel<128, 2, false, false>(sa::Shape, unsigned short const*)"
COPY = "void at::native::elementwise_kernel<direct_copy>(int)"


def _write(tmp, rows):
    d = tmp / "run"
    d.mkdir()
    with open(d / "x_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        for r in rows:
            w.writerow(r)
    return str(tmp)


def test_mfma_summary(tmp_path):
    # two dispatches of 1 ms; 8 XCDs x 2e6 active cycles each = 2 GHz
    rows = []
    for disp, mf in ((1, 1000.0), (2, 3000.0)):
        t0 = 10_000_000 * disp
        for name, val in (("SQ_INSTS_VALU_MFMA_BF16", mf), ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 64.0 * mf),
                          ("SQ_VALU_MFMA_BUSY_CYCLES", 32.0 * mf), ("SQ_INSTS_VALU", 5.0 * mf),
                          ("SQ_INSTS_VALU_TRANS_F32", mf), ("SQ_INSTS_LDS", mf), ("SQ_BUSY_CYCLES", 1.0),
                          ("GRBM_GUI_ACTIVE", 16e6)):
            rows.append([disp, KERNEL, name, val, t0, t0 + 1_000_000])
        rows.append([disp + 10, COPY, "SQ_INSTS_VALU_MFMA_BF16", 7.0, t0, t0 + 5])
    d = _write(tmp_path, rows)
    res = profiling.mfma(d, {"selected_tflop_per_call": 4e-8, "attend_mfma_per_launch": 2000}, "attend_kernel<128")
    assert res["dispatches"] == 2
    assert res["mfma_instructions"] == pytest.approx(2000.0)          # the copy's counts are not mixed in
    assert res["mfma_instructions_ratio"] == pytest.approx(1.0)
    assert res["flop_per_mfma"] == pytest.approx(32768.0)             # 64 units of 512 FLOPs
    assert res["clock_ghz"] == pytest.approx(2.0)
    assert res["mfma_busy_cycles_per_mfma"] == pytest.approx(32.0)
    assert res["mfma_busy_frac"] == pytest.approx(32.0 * 2000 / (1024 * 2e6))
    assert res["executed_tflops"] == pytest.approx(2000 * 32768 / 1e-3 / 1e12)


def test_counters_resident_waves(tmp_path):
    # 12 resident waves on each of 256 CUs for 1e6 cycles = 3 quad-cycle units per CU-cycle
    rows = [[1, KERNEL, "GRBM_GUI_ACTIVE", 8e6, 0, 500_000],
            [1, KERNEL, "SQ_WAVE_CYCLES", 3.0 * 256 * 1e6, 0, 500_000]]
    res = profiling.counters(_write(tmp_path, rows), "attend_kernel<128")
    assert res["clock_ghz"] == pytest.approx(2.0)
    assert res["resident_waves_per_cu"] == pytest.approx(12.0)


def test_traffic_scales_by_the_copy(tmp_path):
    fetch = tmp_path / "f"
    write = tmp_path / "w"
    fetch.mkdir()
    write.mkdir()
    _write(fetch, [[1, KERNEL, "FETCH_SIZE", 100.0, 0, 1], [2, COPY, "FETCH_SIZE", 512.0, 0, 1]])
    _write(write, [[1, KERNEL, "WRITE_SIZE", 10.0, 0, 1], [2, COPY, "WRITE_SIZE", 1024.0, 0, 1]])
    res = profiling.traffic(str(fetch), str(write), "attend_kernel", 1024 * 1024)
    # the copy read 512 KiB for 1 MiB moved (scale 2) and wrote 1024 KiB (scale 1)
    assert res["FETCH_SIZE"]["bytes_per_launch"] == pytest.approx(100 * 1024 * 2.0)
    assert res["WRITE_SIZE"]["bytes_per_launch"] == pytest.approx(10 * 1024 * 1.0)


def test_kernel_stats_skip_warmup(tmp_path):
    """Averages over all calls and over the calls after the first N (in start
    order, whatever the order of the trace rows)."""
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "x_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for t0, dur in ((300, 10), (100, 40), (200, 20), (400, 30)):  # first two by start: 40, 20
            w.writerow([KERNEL, t0, t0 + dur])
    (name, n, tot, avg, mn, mx, rest), = profiling.kernel_stats(str(tmp_path), skip=2)
    assert n == 4 and tot == 100 and avg == 25 and mn == 10 and mx == 40
    assert rest == pytest.approx(20.0)  # (10 + 30) / 2
    assert profiling.kernel_stats(str(tmp_path))[0][6] is None


def test_launch_sequence_takes_the_last_stretch(tmp_path):
    """The launches from the last `first` kernel up to the next `stop`
    kernel, in start order, with their grids and durations."""
    d = tmp_path / "trace"
    d.mkdir()
    rows = [  # (name, start, duration, grid x)
        ("void sa::(anonymous namespace)::gram_kernel<128>(sa::Shape)", 0, 5, 64),
        ("void sa::(anonymous namespace)::split_kernel<128, 256, 8>(sa::Shape, int)", 10, 7, 256),
        ("void sa::(anonymous namespace)::pool_q_kernel<128>(sa::Shape)", 20, 3, 64),
        ("void sa::(anonymous namespace)::gram_kernel<128>(sa::Shape)", 100, 6, 64),
        ("void sa::(anonymous namespace)::wide_pass_kernel<128>(sa::Shape, int)", 110, 9, 1024),
        ("void sa::(anonymous namespace)::split_kernel<128, 256, 8>(sa::Shape, int)", 105, 8, 256),
        ("void sa::(anonymous namespace)::pool_q_kernel<128>(sa::Shape)", 130, 3, 64),
        ("void sa::(anonymous namespace)::attend_kernel<128, 2, false, false>(sa::Shape)", 140, 50, 256),
    ]
    with open(d / "x_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"])
        for name, t0, dur, gx in rows:
            w.writerow([name, t0, t0 + dur, gx, 56, 1])
    seq = profiling.launch_sequence(str(tmp_path), "gram_kernel", "pool_q_kernel")
    assert [(n, g, ns) for n, g, ns in seq] == [
        ("gram_kernel<128>", (64, 56, 1), 6),
        ("split_kernel<128, 256, 8>", (256, 56, 1), 8),
        ("wide_pass_kernel<128>", (1024, 56, 1), 9),
    ]
    with pytest.raises(RuntimeError):
        profiling.launch_sequence(str(tmp_path), "embed_kernel", "pool_q_kernel")
