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


UNIT = "void pa::decode_unit_kernel<pa::MfmaCore<pa::BF16, 128, 16, 4>, pa::BF16, 128, 4>(pa::DecodeArgs, int)"
PARTS = "void pa::decode_merge_parts_kernel<pa::BF16, 128>(pa::DecodeArgs, int)"


def test_ingest_partition_modes_name_the_unit_kernels(tmp_path):
    gib_kib = (1 << 30) / 1024
    write_pass(tmp_path / "fetch", "FETCH_SIZE", [(UNIT, 100.0), (PARTS, 6.0), (COPY, 3.0)])
    write_pass(tmp_path / "write", "WRITE_SIZE", [(UNIT, 8.0), (PARTS, 1.0)])
    write_pass(tmp_path / "calf", "FETCH_SIZE", [(COPY, gib_kib / 2)])
    write_pass(tmp_path / "calw", "WRITE_SIZE", [(COPY, gib_kib)])
    out = bench.ingest_counters(str(tmp_path), config=5, partition=512, block_size=8,
                                out_path=str(tmp_path / "p.json"))
    assert out["kernel"] == UNIT and out["merge_kernel"]["name"] == PARTS
    assert out["fetch_bytes_per_launch"] == pytest.approx((100.0 + 6.0) * 2 * 1024)
    assert out["hbm_bytes_per_launch"] == pytest.approx(((100.0 + 6.0) * 2 + 8.0 + 1.0) * 1024)
    assert out["block_size"] == 8
    # no split: the unit kernel alone
    out0 = bench.ingest_counters(str(tmp_path), config=2, partition=0, out_path=str(tmp_path / "z.json"))
    assert out0["merge_kernel"] is None
    assert out0["hbm_bytes_per_launch"] == pytest.approx((100.0 * 2 + 8.0) * 1024)
    # up to 4096 sequences fixed partitions run on the resident grid
    RES = UNIT.replace("decode_unit_kernel", "decode_parts_resident_kernel")
    for d in ("fetch", "write"):
        import shutil
        shutil.rmtree(tmp_path / d)
    write_pass(tmp_path / "fetch", "FETCH_SIZE", [(RES, 50.0), (PARTS, 6.0)])
    write_pass(tmp_path / "write", "WRITE_SIZE", [(RES, 2.0), (PARTS, 1.0)])
    out2 = bench.ingest_counters(str(tmp_path), config=5, partition=512, out_path=str(tmp_path / "r.json"))
    assert out2["kernel"] == RES and out2["hbm_bytes_per_launch"] == pytest.approx(((50.0 + 6.0) * 2 + 3.0) * 1024)


GROUP = ("void pa::decode_group_kernel<pa::MfmaPvCore<pa::BF16, 128, 16, 4, 1>, pa::MfmaPvCore<pa::BF16, 128, 16, 4, "
         "4>, pa::BF16, 128, 4>(pa::DecodeArgs, pa::GroupArgs, int)")
FEW = "void pa::decode_merge_few_kernel<pa::BF16, 128>(pa::DecodeArgs, int)"


def test_ingest_grouped_counters_adds_the_group_kernel_and_its_merge(tmp_path):
    gib_kib = (1 << 30) / 1024
    # a run that also holds the step's balanced decode: only the grouped call counts
    write_pass(tmp_path / "fetch", "FETCH_SIZE", [(DEC, 999.0), (GROUP, 400.0), (FEW, 8.0), (GROUP, 402.0)])
    write_pass(tmp_path / "write", "WRITE_SIZE", [(DEC, 5.0), (GROUP, 17.0), (FEW, 4.0), (GROUP, 17.0)])
    write_pass(tmp_path / "calf", "FETCH_SIZE", [(COPY, gib_kib / 2)])
    write_pass(tmp_path / "calw", "WRITE_SIZE", [(COPY, gib_kib)])
    out = bench.ingest_grouped_counters(str(tmp_path), out_path=str(tmp_path / "g.json"))
    assert out["kernel"] == GROUP and out["merge_kernel"] == FEW
    assert out["fetch_bytes_per_call"] == pytest.approx((401.0 + 8.0) * 2 * 1024)
    assert out["hbm_bytes_per_call"] == pytest.approx(((401.0 + 8.0) * 2 + 17.0 + 4.0) * 1024)
    assert out["source_sha"] == bench.source_sha()


def test_counter_files_are_named_by_workload():
    assert bench.counters_file(3).endswith("profiles/decode_gqa_llama3_8b_counters.json")
    assert bench.counters_file(5, 8).endswith("profiles/decode_long_context_bs8_counters.json")
    assert bench.counters_file(5, 16, 512).endswith("profiles/decode_long_context_bs16_p512_counters.json")


def test_unique_kv_bytes_counts_each_physical_slot_once():
    # brute force: the distinct (physical block, slot) pairs that the valid
    # tokens of all sequences occupy, on a small prefix-shared batch
    from workloads import synth as W
    b = W.make_prefix_shared_batch(7, num_prompts=3, samples=4, prefix_len=40, suffix_len=20, num_q_heads=4,
                                   num_kv_heads=2, head_dim=64, block_size=16)
    slots = {(int(b.block_tables[s, t // 16]), t % 16) for s in range(b.num_seqs)
             for t in range(int(b.context_lens[s]))}
    per_token = b.num_kv_heads * b.head_dim * 2 * b.elt_bytes
    assert bench.unique_kv_bytes(b) == len(slots) * per_token
    assert bench.unique_kv_bytes(b) < b.kv_bytes()
    # no sharing: unique equals logical
    c = W.make_decode_batch(5, num_seqs=3, num_q_heads=4, num_kv_heads=2, head_dim=64, dtype="bf16",
                            block_size=16, context_lens=[1, 17, 40])
    assert bench.unique_kv_bytes(c) == c.kv_bytes()


def test_cpu_share_respects_affinity_and_omp(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    cores, share = bench.cpu_share()
    assert cores == 1 and share["affinity_cpus"] >= 1
    monkeypatch.delenv("OMP_NUM_THREADS")
    cores, share = bench.cpu_share()
    import os
    assert 1 <= cores <= len(os.sched_getaffinity(0))
    assert isinstance(bench.cpu_model(), str)
