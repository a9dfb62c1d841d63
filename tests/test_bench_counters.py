"""Host logic of bench.py's counter summaries: which dispatches make up the
measured prefill call of a --traffic-probe run, and the per-call sums."""
import csv
import os
import sys

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(__file__), ".."))
import bench  # noqa: E402


def _write(path, rows, counters):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (name, vals) in enumerate(rows):
            for c in counters:
                # two instances per counter, as the per-XCD rows of rocprofv3
                for part in (0.25, 0.75):
                    w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": c,
                                "Counter_Value": vals[c] * part})


PROBE = [
    ("void at::native::distribution_elementwise_grid_stride_kernel", 5.0),
    ("void kda::prep_kernel<false>(...)", 11.0),        # warm call
    ("void kda::k2_kernel<bf16, 0, 64, 1, 2, false>(...)", 12.0),
    ("void at::native::vectorized_elementwise_kernel<4, mul>", 100.0),  # calibration copy
    ("__amd_rocclr_copyBuffer", 0.5),                   # schedule upload of the call
    ("void kda::prep_kernel<false>(...)", 21.0),        # measured call
    ("void kda::k2_kernel<bf16, 0, 64, 1, 2, false>(...)", 22.0),
    ("void at::native::elementwise_kernel<128, 4>", 7.0),  # decode inputs
    ("void kda::decode_kernel<float, false>(...)", 30.0),
    ("void kda::decode_kernel<float, false>(...)", 31.0),
]


def test_probe_window_picks_the_call_after_the_copy(tmp_path):
    p = str(tmp_path / "c.csv")
    _write(p, [(n, {"FETCH_SIZE": v}) for n, v in PROBE], ["FETCH_SIZE"])
    disp = bench.probe_dispatches(p, ("FETCH_SIZE",))
    assert len(disp) == len(PROBE)
    assert disp[3][1]["FETCH_SIZE"] == pytest.approx(100.0)   # instances summed
    icopy, call = bench.probe_window(disp)
    assert icopy == 3
    assert [t for t, _ in call] == ["prep_kernel", "k2_kernel"]
    assert [c["FETCH_SIZE"] for _, c in call] == pytest.approx([21.0, 22.0])


def test_probe_window_keeps_repeated_kernels_of_one_call(tmp_path):
    rows = PROBE[:5] + [("void kda::prep_kernel<false>(...)", 1.0),
                        ("void kda::k2_kernel<bf16, 1, 64, 1, 1, false>(...)", 2.0),
                        ("void kda::scan_kernel<false>(...)", 3.0),
                        ("void kda::k2_kernel<bf16, 0, 128, 1, 2, false>(...)", 4.0)] + PROBE[7:]
    p = str(tmp_path / "c.csv")
    _write(p, [(n, {"FETCH_SIZE": v}) for n, v in rows], ["FETCH_SIZE"])
    _, call = bench.probe_window(bench.probe_dispatches(p, ("FETCH_SIZE",)))
    assert [t for t, _ in call] == ["prep_kernel", "k2_kernel", "scan_kernel", "k2_kernel"]
    assert sum(c["FETCH_SIZE"] for _, c in call) == pytest.approx(10.0)


def test_probe_window_refuses_a_run_without_the_copy(tmp_path):
    rows = [r for r in PROBE if "mul" not in r[0]]
    rows = [("void kda::k2_kernel<x>(...)", 1.0) if "distribution" in n else (n, v)
            for n, v in rows]
    p = str(tmp_path / "c.csv")
    _write(p, [(n, {"FETCH_SIZE": v}) for n, v in rows], ["FETCH_SIZE"])
    with pytest.raises((AssertionError, StopIteration, IndexError)):
        bench.probe_window(bench.probe_dispatches(p, ("FETCH_SIZE",)))


def test_probe_window_counts_the_bf16_planner_scan(tmp_path):
    # the bf16 planner's scan kernel has a name of its own
    rows = PROBE[:5] + [("void kda::prep_kernel<false>(...)", 1.0),
                        ("void kda::k2_kernel<bf16, 1, 64, 1, 1, false>(...)", 2.0),
                        ("kda::scan_bf16_kernel(kda::ScanDesc const*, ...)", 3.0),
                        ("void kda::k2_kernel<bf16, 0, 128, 1, 2, false>(...)", 4.0)] + PROBE[7:]
    p = str(tmp_path / "c.csv")
    _write(p, [(n, {"FETCH_SIZE": v}) for n, v in rows], ["FETCH_SIZE"])
    _, call = bench.probe_window(bench.probe_dispatches(p, ("FETCH_SIZE",)))
    assert [t for t, _ in call] == ["prep_kernel", "k2_kernel", "scan_bf16_kernel", "k2_kernel"]
    assert sum(c["FETCH_SIZE"] for _, c in call) == pytest.approx(10.0)


def test_traffic_probe_entry_exists():
    # --traffic-probe is the command every committed counter summary cites
    assert callable(bench.traffic_probe)


def test_source_hash_ignores_comments_only():
    code = "int a = 1;\nchar c = '\\\\'; // note\n/* block */ const char *s = \"// kept\";\n"
    assert bench.strip_c_comments(code) == \
        "int a = 1; char c = '\\\\'; const char *s = \"// kept\";"
    assert bench.strip_c_comments("x = 1; // a\n") == bench.strip_c_comments("x  =  1;\n// b")
    assert bench.strip_c_comments("x = 1;") != bench.strip_c_comments("x = 2;")
