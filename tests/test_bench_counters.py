"""Host logic of bench.py's counter summary: the calibration copy is the run's
trailing dispatches, not whichever kernel's count lies nearest the copy size."""
import csv
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), ".."))
import bench  # noqa: E402


def _write(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, v) in enumerate(rows):
            w.writerow([i + 1, name, counter, v])


def test_calibration_copy_is_the_trailing_dispatches(tmp_path):
    dec = "void tq::(anonymous namespace)::decode_reg_kernel<3, true, 3, false>(tq::DecodeArgs)"
    # a decoy whose count lies nearer the 256 MiB copy size than the copy's own
    fetch = [("reduce_kernel", 163911.0)] + [(dec, 13824.0)] * 5 + [("copyBuffer", 131083.5)] * 3
    write = [("reduce_kernel", 9.0)] + [(dec, 632.25)] * 5 + [("copyBuffer", 262144.0)] * 3
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(f, "FETCH_SIZE", fetch)
    _write(w, "WRITE_SIZE", write)
    out = bench.summarize_counters(str(f), str(w), 256)
    assert out["fetch_copy_kib"] == 131083.5
    assert out["fetch_bytes_per_launch"] == round(13824.0 * 1024 / (131083.5 / 262144.0))
    assert out["write_bytes_per_launch"] == 632 * 1024 + 256
    assert out["fetch_dispatches"] == 5


def test_summary_refuses_a_run_without_trailing_copies(tmp_path):
    dec = "void tq::(anonymous namespace)::decode_reg_kernel<3, true, 3, false>(tq::DecodeArgs)"
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(f, "FETCH_SIZE", [(dec, 1.0)] * 4)
    _write(w, "WRITE_SIZE", [(dec, 1.0)] * 4)
    try:
        bench.summarize_counters(str(f), str(w), 256)
    except SystemExit:
        return
    raise AssertionError("a run whose last dispatches are the decode kernel was accepted")
