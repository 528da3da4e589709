"""The traffic stamps bench.py reports: rocprofv3 counter files (FETCH_SIZE,
WRITE_SIZE per dispatch, plain-copy calibration) turned into bytes per call,
summed over the kernels of a call, and reported only while the stamp's
kernel-source hash matches the source. Synthetic counter files; no GPU."""
import csv
import json
import os

import pytest

import bench

COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(d, sub, rows):
    os.makedirs(os.path.join(d, sub), exist_ok=True)
    with open(os.path.join(d, sub, "c_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(COLS, r)))


def _runs(d, kernels):
    # the copy: 512 MiB each way; FETCH_SIZE counts half the bytes read
    _write(d, "cf", [(i, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 262144.0) for i in range(3)])
    _write(d, "cw", [(i, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 524288.0) for i in range(3)])
    for sub, scale in (("fs", 1.0), ("ws", 0.5), ("fd", 3.0), ("wd", 2.0)):
        rows = []
        for call in range(4):
            for k, (name, kib) in enumerate(kernels):
                did = 10 * call + k
                # two counter instances per dispatch, summed by the reader
                rows.append((did, name, "X", kib * scale / 2))
                rows.append((did, name, "X", kib * scale / 2))
        _write(d, sub, rows)


@pytest.mark.parametrize("workload,kernels", [
    ("long", [("void kvq::gqa_fused<1, 8, 0>(kvq::GqaArgs)", 1000.0)]),
    ("mla", [("void kvq::mla_scores<8>(kvq::MlaArgs)", 1000.0), ("kvq::mla_out(kvq::MlaArgs)", 30.0)]),
])
def test_stamp_bytes_and_hash(tmp_path, monkeypatch, workload, kernels):
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path / "profiles"))
    os.makedirs(bench.TRAFFIC_DIR)
    d = str(tmp_path / "runs")
    _runs(d, kernels)
    t = bench.write_traffic(d, workload)
    total = sum(k for _, k in kernels)
    # fetch factor 2 (the copy's FETCH_SIZE reads half of 512 MiB), write factor 1
    assert t["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert t["calibration"]["write_factor"] == pytest.approx(1.0)
    assert t["sparse"]["bytes_per_launch"] == round((total * 1.0 * 2 + total * 0.5) * 1024)
    assert t["dense"]["bytes_per_launch"] == round((total * 3.0 * 2 + total * 2.0) * 1024)
    assert bench.load_traffic("sparse", workload) == t["sparse"]["bytes_per_launch"]
    # a stamp taken on other kernel code is not reported
    path = bench.traffic_file(workload)
    with open(path) as f:
        j = json.load(f)
    j["kernel_sha256_16"] = "0" * 16
    with open(path, "w") as f:
        json.dump(j, f)
    assert bench.load_traffic("sparse", workload) is None


def test_hash_ignores_comments_and_blank_space(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SRCS, "long", "k.hip")
    src.write_text("int a = 1;  // one\n\nint b = 2;\n")
    h0 = bench.kernel_hash("long")
    src.write_text("int a = 1;   // a different comment\n   int b = 2;   \n\n")
    assert bench.kernel_hash("long") == h0
    src.write_text("int a = 1;\nint b = 3;\n")
    assert bench.kernel_hash("long") != h0
