"""bench.py's counter ingestion: FETCH_SIZE / WRITE_SIZE passes (KiB per
dispatch, rocprofv3 csv rows) become bytes per decode call, each counter
scaled by what it reads for a plain 1 GiB copy.  Synthetic csv files, no GPU."""

import csv
import json
import os

import pytest

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
DEC = "void pa::decode_balanced_kernel<pa::MfmaCore<pa::BF16, 128, 16, 4>, pa::BF16, 128, 4>(pa::DecodeArgs, int)"
MRG = "void pa::decode_merge_balanced_kernel<pa::BF16, 128, 4>(pa::DecodeArgs, int, int)"
COPY = "__amd_rocclr_copyBuffer"


def write_pass(d, counter, rows):
    os.makedirs(d)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for i, (k, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_ingest_scales_by_the_copy_calibration(tmp_path):
    gib_kib = (1 << 30) / 1024
    # decode dispatches read 1000 and 1002 KiB (mean 1001), merge 10; the copy
    # reads half its bytes by FETCH_SIZE (factor 2) and all by WRITE_SIZE
    write_pass(tmp_path / "fetch", "FETCH_SIZE", [(DEC, 1000.0), (MRG, 10.0), (DEC, 1002.0), (COPY, 7.0)])
    write_pass(tmp_path / "write", "WRITE_SIZE", [(DEC, 4.0), (MRG, 2.0), (DEC, 4.0)])
    write_pass(tmp_path / "calf", "FETCH_SIZE", [(COPY, gib_kib / 2)] * 5)
    write_pass(tmp_path / "calw", "WRITE_SIZE", [(COPY, gib_kib)] * 5)
    out_path = tmp_path / "counters.json"
    out = bench.ingest_counters(str(tmp_path), out_path=str(out_path))
    assert out["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert out["calibration"]["write_factor"] == pytest.approx(1.0)
    assert out["decode_kernel_bytes"] == pytest.approx((1001.0 * 2 + 4.0) * 1024)
    assert out["hbm_bytes_per_launch"] == pytest.approx((1001.0 * 2 + 4.0 + 10.0 * 2 + 2.0) * 1024)
    assert out["source_sha"] == bench.source_sha()
    assert json.loads(out_path.read_text()) == out


def test_ingest_refuses_ambiguous_kernels(tmp_path):
    write_pass(tmp_path / "fetch", "FETCH_SIZE", [(DEC, 1.0), (DEC.replace("128, 4>", "128, 8>"), 1.0), (MRG, 1.0)])
    write_pass(tmp_path / "write", "WRITE_SIZE", [(DEC, 1.0), (MRG, 1.0)])
    write_pass(tmp_path / "calf", "FETCH_SIZE", [(COPY, 1.0)])
    write_pass(tmp_path / "calw", "WRITE_SIZE", [(COPY, 1.0)])
    with pytest.raises(SystemExit):
        bench.ingest_counters(str(tmp_path), out_path=str(tmp_path / "c.json"))
