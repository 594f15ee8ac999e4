"""bench.py's counter summary (--pmc-summary): HBM bytes per dispatch of the
grouped GEMM1 from rocprofv3 FETCH_SIZE / WRITE_SIZE rows, scaled by the
dispatches of known bytes in the same run (the plain device copy, and the
direct-to-LDS calibration tile when the run had one).  Synthetic counter files
with known values; no GPU."""
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size", "Kernel_Id",
        "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
        "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
COPY = "__amd_rocclr_copyBuffer"
DOWN = "void moe::gemm::grouped_gemm_bf16<false, 0, 0, 0>(moe::gemm::Args)"
GEMM1 = "void moe::gemm::grouped_gemm_bf16<true, 0, 0, 0>(moe::gemm::Args)"


def _write(path, counter, rows, reverse=False):
    """rows in dispatch order (ids 1, 2, ...); written to the file reversed if asked"""
    recs = []
    for i, (name, v) in enumerate(rows):
        r = dict.fromkeys(COLS, "0")
        r.update(Dispatch_Id=str(i + 1), Kernel_Name=name, Counter_Name=counter, Counter_Value=f"{v:.6f}")
        recs.append(r)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=COLS)
        w.writeheader()
        w.writerows(recs[::-1] if reverse else recs)


def _run(tmp_path, fetch_rows, write_rows, lds_mib, reverse=False):
    f, w, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _write(f, "FETCH_SIZE", fetch_rows, reverse)
    _write(w, "WRITE_SIZE", write_rows, reverse)
    bench.pmc_summary(str(f), str(w), "mixtral_bf16", str(out), lds_mib)
    return json.loads(out.read_text())


def test_copy_factor_without_calibration_tile(tmp_path):
    # a 1 GiB copy reading 0.5 GiB of FETCH_SIZE: fetch x2; GEMM1 averaged over its dispatches
    fetch = [(COPY, 524288.0), (GEMM1, 1000.0), (GEMM1, 3000.0), (DOWN, 777.0)]
    write = [(COPY, 1048576.0), (GEMM1, 50.0), (GEMM1, 70.0), (DOWN, 1.0)]
    d = _run(tmp_path, fetch, write, 0)
    assert d["fetch_scale"] == 2.0 and d["copy_fetch_scale"] == 2.0 and d["write_scale"] == 1.0
    assert d["fetch_bytes"] == round(2000.0 * 2.0 * 1024) and d["write_bytes"] == round(60.0 * 1024)
    assert d["bytes_per_dispatch"] == d["fetch_bytes"] + d["write_bytes"]
    assert d["lds_calibration_mib"] == 0
    assert d["source_hash"] == bench.kernel_source_hash("bf16")


def test_calibration_tile_sets_the_fetch_factor_and_is_not_a_down_gemm(tmp_path):
    # The first bf16 down-GEMM dispatch is the 256 MiB calibration tile; here it
    # reads 64 MiB of FETCH_SIZE (x4), which must scale GEMM1's fetch, while the
    # copy says x2.  Dispatch order, not file order, decides which one it is.
    fetch = [(GEMM1, 1000.0), (DOWN, 65536.0), (COPY, 524288.0), (DOWN, 5.0)]
    write = [(GEMM1, 10.0), (DOWN, 2.0), (COPY, 1048576.0), (DOWN, 3.0)]
    d = _run(tmp_path, fetch, write, 256, reverse=True)
    assert d["fetch_scale"] == 4.0 and d["copy_fetch_scale"] == 2.0
    assert d["fetch_bytes"] == round(1000.0 * 4.0 * 1024)
    assert d["lds_calibration_mib"] == 256
