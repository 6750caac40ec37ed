"""Host logic of bench.py (no GPU): the one-GPU contract, the arithmetic of the
counter and traffic records written from rocprofv3 CSVs, the freshness check
that ties a record to the sources it was measured on, and the committed
records' own consistency."""
import csv
import glob
import json
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)
import bench  # noqa: E402

COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(COLS, r)))


@pytest.fixture
def sandbox(tmp_path, monkeypatch):
    """bench.py writing into a scratch copy of the profiles folder."""
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda kernel: "h-" + kernel)
    return tmp_path


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_record_fractions(sandbox):
    # two dispatches of the kernel, one of another kernel that must be ignored
    k = "void mla::gemm_bf16_ring<2, 4>(mla::GemmParams)"
    rows = []
    for d, (gui, mfma, ta, lds, bank) in enumerate([(8.0e6, 2.048e8, 1.28e8, 1.024e8, 1.024e7),
                                                    (8.4e6, 2.152e8, 1.344e8, 1.076e8, 1.076e7)]):
        for name, v in [("GRBM_GUI_ACTIVE", gui), ("SQ_VALU_MFMA_BUSY_CYCLES", mfma), ("TA_TA_BUSY_sum", ta),
                        ("SQ_LDS_IDX_ACTIVE", lds), ("SQ_LDS_BANK_CONFLICT", bank)]:
            rows.append([d, k, name, v, 1000, 1000 + 600000])
    rows.append([9, "other_kernel", "GRBM_GUI_ACTIVE", 1.0, 0, 10])
    p = sandbox / "c.csv"
    _csv(p, rows)
    bench.write_counter_record("c1_product", [str(p)], ["cmd"])
    rec = json.load(open(sandbox / "profiles" / "gemm_bf16_ring_c1_product_counters.json"))
    cycles = (8.0e6 + 8.4e6) / 2 / 8          # GRBM_GUI_ACTIVE is summed over the 8 XCDs
    assert rec["cycles_per_xcd"] == round(cycles)
    assert rec["mfma_busy_frac"] == round((2.048e8 + 2.152e8) / 2 / 1024 / cycles, 4)
    assert rec["ta_busy_frac"] == round((1.28e8 + 1.344e8) / 2 / 256 / cycles, 4)
    assert rec["lds_busy_frac"] == round((1.024e8 + 1.076e8) / 2 / 256 / cycles, 4)
    assert rec["lds_bank_conflict_frac"] == round(((1.024e7 + 1.076e7) / 2) / ((1.024e8 + 1.076e8) / 2), 4)
    assert rec["clock_ghz"] == round(cycles / 600000, 3)
    assert rec["source_hash"] == "h-gemm_bf16_ring" and rec["commands"] == ["cmd"]


def test_traffic_record_scaled_by_the_copy_calibration(sandbox):
    copy = "__amd_rocclr_copyBuffer_aligned"
    f, w = sandbox / "f.csv", sandbox / "w.csv"
    # a 1 GiB copy whose FETCH_SIZE reads half the bytes and WRITE_SIZE all of them (KiB)
    _csv(f, [[0, copy, "FETCH_SIZE", 524288.0, 0, 1], [1, copy, "FETCH_SIZE", 524288.0, 0, 1]])
    _csv(w, [[0, copy, "WRITE_SIZE", 1048576.0, 0, 1]])
    bench.write_traffic_record("copy", str(f), str(w), ["c1", "c2"], 0)
    cal = json.load(open(sandbox / "profiles" / "copy_probe_hbm_calibration.json"))
    assert cal["fetch_scale"] == 2.0 and cal["write_scale"] == 1.0
    k = "mla::gather_rows_kernel(mla::DecompressArgs, int)"
    _csv(f, [[0, k, "FETCH_SIZE", 1000.0, 0, 1], [1, k, "FETCH_SIZE", 3000.0, 0, 1]])
    _csv(w, [[0, k, "WRITE_SIZE", 4096.0, 0, 1]])
    bench.write_traffic_record("c1_gather", str(f), str(w), ["c1", "c2"], 123)
    rec = json.load(open(sandbox / "profiles" / "gather_rows_kernel_c1_gather_hbm_traffic.json"))
    assert rec["hbm_read_bytes_per_launch"] == 2000 * 1024 * 2
    assert rec["hbm_write_bytes_per_launch"] == 4096 * 1024
    assert rec["hbm_bytes_per_launch"] == rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    assert rec["algorithmic_bytes_per_launch"] == 123 and rec["dispatches_averaged"] == [2, 1]


def test_a_record_is_used_only_while_its_sources_are_unchanged(sandbox, monkeypatch):
    rec = {"kernel": "gather_rows_kernel", "workload": "c1_gather", "source_hash": "h-gather_rows_kernel",
           "hbm_bytes_per_launch": 7}
    with open(sandbox / "profiles" / "gather_rows_kernel_c1_gather_hbm_traffic.json", "w") as f:
        json.dump(rec, f)
    assert bench.traffic_from_profile("gather_rows_kernel", "c1_gather") == 7
    monkeypatch.setattr(bench, "source_hash", lambda kernel: "edited")
    assert bench.traffic_from_profile("gather_rows_kernel", "c1_gather") is None


def test_committed_records_are_consistent():
    recs = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.json")))
    assert recs, "no records under profiles/"
    for path in recs:
        rec = json.load(open(path))
        name = os.path.basename(path)
        assert rec.get("commands"), name
        for c in rec["commands"]:
            assert "_work" not in c and "bench.py" in c, (name, c)
        if name.endswith("_hbm_traffic.json"):
            assert rec["hbm_bytes_per_launch"] == rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
            assert rec["kernel"] in bench.KERNEL_SOURCES, name
        if name.endswith("_counters.json"):
            for k in ("mfma_busy_frac", "ta_busy_frac", "lds_busy_frac", "lds_bank_conflict_frac"):
                if k in rec:
                    assert 0.0 <= rec[k] <= 1.0, (name, k, rec[k])
