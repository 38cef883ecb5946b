"""Host-side measurement helpers of bench.py (no GPU): the code-only source hash that ties the
committed profiles to the kernels, and the rocprofv3 summariser that turns counter CSVs into
per-launch traffic."""
import argparse
import csv
import json
import os
import shutil
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import bench  # noqa: E402


def test_code_only_strips_comments_and_blank_lines():
    src = "int a; // trailing\n/* block\n   comment */ int b;\n\n   // whole line\nint c;  \n"
    assert bench.code_only(src) == "int a;\n int b;\nint c;"


def _copy_sources(tmp_path):
    dst = tmp_path / "mla_prolog_amd" / "csrc"
    shutil.copytree(os.path.join(bench.ROOT, "mla_prolog_amd", "csrc"), dst)
    return dst


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    csrc = _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    f = csrc / "gemm_big.hpp"
    f.write_text(f.read_text() + "\n// a note added to a comment\n\n")
    assert bench.kernel_source_hash() == h0
    f.write_text(f.read_text() + "static_assert(true, \"a code change\");\n")
    assert bench.kernel_source_hash() != h0
    # the row kernels are outside the hash (the up projections only read their outputs)
    g = csrc / "row_kernels.hip"
    h1 = bench.kernel_source_hash()
    g.write_text(g.read_text() + "static_assert(true, \"row kernel change\");\n")
    assert bench.kernel_source_hash() == h1


def _write_csv(path, fields, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_scales_traffic_by_the_calibration_runs(tmp_path, monkeypatch):
    dom = "void mlap::gemm_big_kernel<unsigned short, 256, 256, 4, 2, 128, 2, (mlap::Epi)3>(mlap::GemmArgs)"
    other = "void mlap::quant_q_kernel<0>(mlap::QuantQArgs)"
    copy = "__amd_rocclr_copyBuffer"
    fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, x>(int, x)"
    # trace: 3 steps of the two kernels (dominant 100 us, quant 20 us) and one copy
    trace = tmp_path / "trace.csv"
    rows, t = [], 0
    for _ in range(3):
        for name, us in ((dom, 100.0), (other, 20.0)):
            rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + int(us * 1000)})
            t += int(us * 1000) + 1000
    rows.append({"Kernel_Name": copy, "Start_Timestamp": t, "End_Timestamp": t + 5000})
    _write_csv(trace, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    # FETCH pass: the copy of 64 MiB reads as half (32768 KiB: scale 2); WRITE pass: exact
    mib = 64
    fetch, write = tmp_path / "F.csv", tmp_path / "W.csv"
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(fetch, fields, [{"Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": mib * 512},
                               {"Kernel_Name": dom, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000},
                               {"Kernel_Name": dom, "Counter_Name": "FETCH_SIZE", "Counter_Value": 3000}])
    _write_csv(write, fields, [{"Kernel_Name": fill, "Counter_Name": "WRITE_SIZE", "Counter_Value": mib * 1024},
                               {"Kernel_Name": dom, "Counter_Name": "WRITE_SIZE", "Counter_Value": 500}])
    inputs = tmp_path / "roofline_inputs.json"
    monkeypatch.setattr(bench, "PROFILE_INPUTS", str(inputs))
    out = tmp_path / "summary.md"
    a = argparse.Namespace(title="t", command=["cmd one"], trace=str(trace), pmc=[str(fetch), str(write)],
                           calibrate_mib=mib, sclk_mhz=2000, dominant="(mlap::Epi)3", out=str(out),
                           workload="wl")
    bench.summarize(a)
    e = json.load(open(inputs))["wl"]
    assert e["launches_per_step"] == 1
    assert abs(e["trace_us_avg"] - 100.0) < 1e-6 and abs(e["trace_us_median"] - 100.0) < 1e-6
    # average FETCH 2000 KiB x 2 + WRITE 500 KiB x 1, in bytes
    assert e["hbm_bytes_per_launch"] == (2000 * 2 + 500) * 1024
    assert e["kernel_source_hash"] == bench.kernel_source_hash()
    text = out.read_text()
    assert "cmd one" in text and "scale 2.000" in text and "scale 1.000" in text
