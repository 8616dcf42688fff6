"""Host-side checks of bench.py (no GPU needed): the one-GPU contract and
the arithmetic of the rocprofv3 summaries, on small synthetic counter files."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_summary_per_wave_and_mfma_busy_fraction(tmp_path):
    # two passes over the same two dispatches of the streaming kernel; the
    # MFMA-busy fraction is busy SIMD-cycles over duration x 2.4 GHz x 1024
    k = "void swa::bwd_stream_kernel<__bf16, true>(swa::BwdArgs)"
    dur_ns = 100_000
    busy = 0.25 * dur_ns * bench.CLOCK_GHZ * bench.N_SIMD
    _write_counters(tmp_path / "p1", [
        (1, k, "SQ_WAVES", 2048, 0, dur_ns), (2, k, "SQ_WAVES", 2048, 0, dur_ns),
        (1, "other_kernel", "SQ_WAVES", 7, 0, 5)])
    _write_counters(tmp_path / "p2", [
        (1, k, "SQ_INSTS_MFMA", 2048 * 100, 0, dur_ns), (2, k, "SQ_INSTS_MFMA", 2048 * 300, 0, dur_ns),
        (1, k, "SQ_VALU_MFMA_BUSY_CYCLES", busy, 0, dur_ns), (2, k, "SQ_VALU_MFMA_BUSY_CYCLES", busy, 0, dur_ns)])
    out = tmp_path / "sq.txt"
    bench.summarize_counters([str(tmp_path / "p1"), str(tmp_path / "p2")], str(out), ["cmd1", "cmd2"], "c3")
    text = out.read_text()
    assert "bwd_stream_kernel: 4 dispatches" in text
    assert "MFMA 200" in text  # (100 + 300) / 2 per dispatch, per wave
    assert "MFMA busy / SIMD cycles    0.250" in text
    assert "other_kernel" not in text and "cmd2" in text


def test_traffic_summary_calibrates_each_counter_by_the_copy(tmp_path):
    # FETCH_SIZE reads half a KiB per KiB fetched, WRITE_SIZE one per KiB
    # written (as measured on MI355X); the kernel's bytes are scaled back
    kib = bench.COPY_BYTES / 1024
    main = "void swa::bwd_stream_kernel<__bf16, true>(swa::BwdArgs)"
    _write_counters(tmp_path / "f", [(1, bench.COPY_KERNEL, "FETCH_SIZE", 0.5 * kib, 0, 1),
                                     (2, main, "FETCH_SIZE", 1000.0, 0, 1), (3, main, "FETCH_SIZE", 3000.0, 0, 1)])
    _write_counters(tmp_path / "w", [(1, bench.COPY_KERNEL, "WRITE_SIZE", kib, 0, 1),
                                     (2, main, "WRITE_SIZE", 500.0, 0, 1)])
    out = tmp_path / "t.txt"
    bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(out), ["a", "b"], "c3")
    rec = json.loads(out.read_text().split("TRAFFIC ", 1)[1])
    assert rec["fetch_factor"] == pytest.approx(0.5) and rec["write_factor"] == pytest.approx(1.0)
    assert rec["traffic_bytes_per_launch"] == pytest.approx(2000.0 * 1024 / 0.5 + 500.0 * 1024)
