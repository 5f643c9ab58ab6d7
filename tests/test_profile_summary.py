"""The counter summaries' copy calibration (CPU only): the scale comes from
the run's largest device copies (the 1 GiB calibration copies), not from a
mean that smaller copies in the same run would pull down; written from a
synthetic rocprofv3 CSV in the tool's column layout."""
import argparse
import csv

from dropless_moe_expert_amd import profile_summary as ps

COLS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp", "Counter_Name", "Counter_Value"]


def _write(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=COLS)
        w.writeheader()
        for i, (name, counter, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": 256, "Start_Timestamp": 0,
                        "End_Timestamp": 1000, "Counter_Name": counter, "Counter_Value": kib})


def test_copy_scale_uses_the_largest_copies(tmp_path):
    gib = ps.COPY_KIB
    p = tmp_path / "fetch.csv"
    # three 1 GiB calibration copies (FETCH_SIZE reads half the bytes), two
    # 512 MiB copies and a small one in the same run, and a kernel
    _write(p, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", gib / 2)] * 3
           + [("__amd_rocclr_copyBuffer", "FETCH_SIZE", gib / 4 * 1.01)] * 2   # a little over a quarter
           + [("__amd_rocclr_copyBuffer", "FETCH_SIZE", gib / 64),
              ("some_kernel", "FETCH_SIZE", 12345.0)])
    assert ps._copy_scale(ps._dispatches(str(p)), "FETCH_SIZE") == 2.0


def test_copy_scale_absent_without_copies(tmp_path):
    p = tmp_path / "write.csv"
    _write(p, [("some_kernel", "WRITE_SIZE", 100.0)])
    assert ps._copy_scale(ps._dispatches(str(p)), "WRITE_SIZE") is None


def test_counters_table_lds_figures(tmp_path):
    # one kernel, two dispatches with the same counters: LDS utilisation is
    # SQ_LDS_IDX_ACTIVE over (GRBM_GUI_ACTIVE / 8 XCCs) x 256 CUs, conflicts
    # per active cycle, and LDS issue waits (units of 4 cycles) per wave cycle
    rows = []
    for _ in range(2):
        rows += [("k", "GRBM_GUI_ACTIVE", 8 * 1000.0), ("k", "SQ_LDS_IDX_ACTIVE", 256 * 250.0),
                 ("k", "SQ_LDS_BANK_CONFLICT", 640.0), ("k", "SQ_WAIT_INST_LDS", 50.0),
                 ("k", "SQ_WAVE_CYCLES", 800.0)]
    p = tmp_path / "lds.csv"
    with open(p, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=COLS)
        w.writeheader()
        for i, (name, counter, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i // 5, "Kernel_Name": name, "Grid_Size": 256, "Start_Timestamp": 0,
                        "End_Timestamp": 2000, "Counter_Name": counter, "Counter_Value": v})
    args = argparse.Namespace(
        title="t", source=[], command=["c"], counters=str(p), kernel_filter=None)
    out = ps.counters_table(args)
    row = [ln for ln in out.splitlines() if ln.startswith("| `k`")][0].split("|")
    assert row[2].strip() == "2"
    assert row[4].strip() == "25.0 %"
    assert row[5].strip() == "0.010"
    assert row[6].strip() == "0.25"
