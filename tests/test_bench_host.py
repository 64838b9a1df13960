"""Host logic of bench.py that turns measurements into reported figures, on
synthetic inputs (no GPU): per-call percentiles, the kernel-trace summary's
average over the timed steps, the counter calibration of the traffic
summaries, the cold-rotation sizing and the algorithmic bytes."""
from __future__ import annotations

import csv
import json
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_spread_takes_nearest_ranks():
    s = bench.spread([float(x) for x in range(100, 0, -1)])  # 1..100, unsorted
    assert s == {"median": 51.0, "p10": 11.0, "p90": 90.0, "samples": 100}
    assert bench.spread([3.0]) == {"median": 3.0, "p10": 3.0, "p90": 3.0, "samples": 1}


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_ALL)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_averages_only_the_timed_steps(tmp_path):
    """The first group kernel of the run is the timed one; of its dispatches
    (in start order) the first `warmup` are skipped and the next `steps` are
    averaged.  Later launches of the same symbol (comparisons) and other
    group kernels do not enter the average."""
    warmup, steps = 3, 5
    g2 = "void rlscan::group_kernel<2, false>(rlscan::GroupArgs)"
    g1 = "void rlscan::group_kernel<1, false>(rlscan::GroupArgs)"
    rows, t = [], 1000
    durations = [50, 50, 50] + [10, 12, 14, 16, 18] + [99, 99, 99]  # warmup, timed, later
    for i, d in enumerate(durations):
        rows.append([i, g2, t, t + d * 1000])
        t += 100_000
    rows.append([99, g1, t, t + 7_000])  # another group kernel, later in the run
    rows = rows[::-1]  # file order is not start order
    trace = tmp_path / "trace.csv"
    _write_csv(trace, ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    stats = tmp_path / "stats.csv"
    _write_csv(stats, ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                       "MaxNs", "StdDev"],
               [[g2, 11, 0, 40_000.0, 90.0, 10_000, 99_000, 0.0]])
    log = tmp_path / "run.log"
    log.write_text("[bench] noise\n" + json.dumps({
        "metric": "m", "warmup": warmup, "steps": steps, "ms_per_step": 0.0151,
        "roofline": {"avg_launch_us": 14.9}, "kernel_source_hash": "abc"}) + "\n")
    out = tmp_path / "summary.md"
    bench.trace_summary(str(log), str(stats), str(trace), str(out), "the command")
    text = out.read_text()
    assert "average duration over the 5 timed steps: 14.00 µs (min 10.00, max 18.00)" in text
    assert "dispatches 4–8 of 11" in text
    assert "`group_kernel<2, false>` | 11 | 40.00 |" in text
    assert "the command" in text and "`abc`" in text


def test_traffic_summary_calibrates_against_the_copy(tmp_path, monkeypatch):
    """Counter KiB are scaled so that the calibration copy reads and writes
    exactly COPY_BYTES: here FETCH_SIZE reports half and WRITE_SIZE all of
    the copy's bytes, so the scan kernel's fetch KiB double."""
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    cb = 1 << 28
    scan = "void rlscan::scan_kernel<rlscan::Gae<true, float>, 4, 4, true, true, false>(x)"
    copy = "rlscan::copy_kernel(float __vector(4) const*, float __vector(4)*, long)"
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(tmp_path / "f.csv", hdr, [[scan, "FETCH_SIZE", 100.0], [scan, "FETCH_SIZE", 102.0],
                                         [copy, "FETCH_SIZE", cb / 2 / 1024]])
    _write_csv(tmp_path / "w.csv", hdr, [[scan, "WRITE_SIZE", 40.0], [scan, "WRITE_SIZE", 40.0],
                                         [copy, "WRITE_SIZE", cb / 1024]])
    _write_csv(tmp_path / "h.csv", hdr, [[scan, "TCC_HIT_sum", 30.0], [scan, "TCC_MISS_sum", 70.0]])
    log = tmp_path / "run.log"
    log.write_text(json.dumps({
        "pmc_run": "gae", "workload": "unit_workload", "byte_flags": False,
        "launches": {"gae": 2}, "algorithmic_bytes_per_launch": {"gae": 200 * 1024},
        "copy_bytes": cb, "kernel_source_hash": "h"}) + "\n")
    bench.traffic_summary(str(log), str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                          str(tmp_path / "h.csv"))
    kv = {}
    for line in open(tmp_path / "traffic_gae_unit_workload.txt"):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert int(kv["read_bytes_per_launch"]) == 2 * 101 * 1024
    assert int(kv["write_bytes_per_launch"]) == 40 * 1024
    assert int(kv["hbm_bytes_per_launch"]) == 242 * 1024
    assert "hit rate 0.300" in open(tmp_path / "traffic_gae_unit_workload.txt").read()


class _FakeSet:
    def __init__(self, tag):
        self.tag = tag

    def clone(self, stream, lib):
        return _FakeSet(self.tag + "'")


@pytest.mark.parametrize("per_set,seeded,want", [
    (88_145_920, 6, 25),          # the production step: 25 sets, 2.2 GB
    (bench.COLD_BYTES, 3, 3),     # one set already moves COLD_BYTES
    (6_291_456, 6, 342),          # a 6 MB call: 342 launches per pass
    (1024, 6, 512),               # capped
])
def test_cold_rotation_reaches_cold_bytes(per_set, seeded, want):
    sets = bench.cold_rotation([_FakeSet(str(i)) for i in range(seeded)], per_set, None, None)
    assert len(sets) == want
    assert [s.tag for s in sets[:seeded]] == [str(i) for i in range(seeded)]
    assert all(s.tag.endswith("'") for s in sets[seeded:])
    if want < 512:
        assert want * per_set >= bench.COLD_BYTES > (want - 1) * per_set or want == seeded


def test_algorithmic_bytes_counts_every_array_once():
    torch = pytest.importorskip("torch")
    ins = {"a": np.zeros((4, 8), np.float32), "b": None, "c": np.zeros(4, np.int32)}
    outs = {"o": torch.empty((4, 8), dtype=torch.int64)}
    assert bench.algorithmic_bytes(ins, outs) == 4 * 8 * 4 + 4 * 4 + 4 * 8 * 8
