"""The counter summaries' copy calibration (CPU only): the scale comes from
the run's largest device copies (the 1 GiB calibration copies), not from a
mean that smaller copies in the same run would pull down; written from a
synthetic rocprofv3 CSV in the tool's column layout."""
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
