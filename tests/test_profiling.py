"""Host logic of the profile summaries (gguf_block_quant_qmm_amd/profiling.py)
and of bench.py's counter lookup, on synthetic rocprofv3 CSV files whose
answers are worked out by hand.  No GPU."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from gguf_block_quant_qmm_amd import profiling  # noqa: E402
import bench  # noqa: E402

COUNTER_FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
                  "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
                  "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
                  "End_Timestamp"]


def write_counters(path, rows):
    """rows: (dispatch, kernel, grid, wg, counter, value, start_ns, end_ns)"""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, COUNTER_FIELDS, quoting=csv.QUOTE_NONNUMERIC)
        w.writeheader()
        for d, k, grid, wg, name, val, t0, t1 in rows:
            w.writerow({"Correlation_Id": d, "Dispatch_Id": d, "Agent_Id": "Agent 1", "Queue_Id": 1,
                        "Process_Id": 1, "Thread_Id": 1, "Grid_Size": grid, "Kernel_Id": 1, "Kernel_Name": k,
                        "Workgroup_Size": wg, "LDS_Block_Size": 0, "Scratch_Size": 0, "VGPR_Count": 64,
                        "Accum_VGPR_Count": 0, "SGPR_Count": 32, "Counter_Name": name, "Counter_Value": val,
                        "Start_Timestamp": t0, "End_Timestamp": t1})


def test_stats_groups_are_total_time_over_total_calls(tmp_path, capsys):
    p = tmp_path / "k.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["void qmm::gemv_kernel<2, 2, 0>(...)", 3, 30000, 10000, 50.0, 9000, 11000, 0])
        w.writerow(["void qmm::gemv_kernel<2, 2, 3>(...)", 1, 14000, 14000, 23.3, 14000, 14000, 0])
        w.writerow(["void qmm::gemm_wb_kernel<12, 32>(...)", 2, 16000, 8000, 26.7, 8000, 8000, 0])
    out = tmp_path / "s.md"
    profiling.main(["stats", "--csv", str(p), "--cmd", "cmd", "--group", "gemv=gemv_kernel<2,",
                    "--group", "gemm=gemm_wb_kernel<12,", "--out", str(out)])
    text = out.read_text()
    assert "| gemv | 4 | 11.000 |" in text  # (30000 + 14000) ns / 4 calls
    assert "| gemm | 2 | 8.000 |" in text
    # sorted by total time
    assert text.index("gemv_kernel<2, 2, 0>") < text.index("gemm_wb_kernel") < text.index("gemv_kernel<2, 2, 3>")


def test_traffic_scales_by_the_calibration_copy(tmp_path):
    mib512 = 512 << 20
    cf, cw, kf, kw = (tmp_path / n for n in ("cf.csv", "cw.csv", "kf.csv", "kw.csv"))
    # the copy reads 512 MiB; FETCH_SIZE reads 262144 units -> 2048 bytes per unit, WRITE_SIZE 524288 -> 1024
    write_counters(cf, [(1, "__amd_rocclr_copyBuffer", 1024, 512, "FETCH_SIZE", 999.0, 0, 1),
                        (2, "__amd_rocclr_copyBuffer", 1024, 512, "FETCH_SIZE", 262144.0, 0, 1)])
    write_counters(cw, [(1, "__amd_rocclr_copyBuffer", 1024, 512, "WRITE_SIZE", 524288.0, 0, 1)])
    # two dispatches of the kernel (one reading split over two rows, as for several dies) and one other kernel
    write_counters(kf, [(5, "qmm::gemv_kernel<2, 2>", 256, 256, "FETCH_SIZE", 100.0, 0, 1),
                        (5, "qmm::gemv_kernel<2, 2>", 256, 256, "FETCH_SIZE", 50.0, 0, 1),
                        (6, "qmm::gemv_kernel<2, 2>", 256, 256, "FETCH_SIZE", 250.0, 0, 1),
                        (7, "qmm::other", 256, 256, "FETCH_SIZE", 1e6, 0, 1)])
    write_counters(kw, [(5, "qmm::gemv_kernel<2, 2>", 256, 256, "WRITE_SIZE", 4.0, 0, 1),
                        (6, "qmm::gemv_kernel<2, 2>", 256, 256, "WRITE_SIZE", 6.0, 0, 1)])
    out = tmp_path / "c.json"
    profiling.main(["traffic", "--fetch", str(kf), "--write", str(kw), "--calib-fetch", str(cf), "--calib-write",
                    str(cw), "--calib-bytes", str(mib512), "--key", "g=gemv_kernel<2,", "--out", str(out)])
    db = json.loads(out.read_text())
    assert db["_calibration"]["bytes_per_fetch_unit"] == 2048.0  # the copy's last dispatch
    assert db["_calibration"]["bytes_per_write_unit"] == 1024.0
    g = db["g"]
    assert g["dispatches"] == 2
    assert g["fetch_bytes_per_launch"] == 2048 * 200  # mean of 150 and 250 units
    assert g["write_bytes_per_launch"] == 1024 * 5
    assert g["hbm_bytes_per_launch"] == 2048 * 200 + 1024 * 5
    assert g["source_hash"] == profiling.kernel_source_hash()


def test_mfma_busy_clock_and_flops(tmp_path, capsys):
    p = tmp_path / "m.csv"
    # one dispatch of 100 us: GUI-active 8 dies x 200000 cycles -> 2.0 GHz; busy cycles summed over
    # 1024 SIMDs = 0.25 x 200000 x 1024; MOPS x 512 = the algorithmic 1e12 FLOPs
    k = "qmm::gemm_wb_kernel<12, 32>"
    write_counters(p, [(3, k, 1, 1, "GRBM_GUI_ACTIVE", 8 * 200000.0, 0, 100000),
                       (3, k, 1, 1, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 200000 * 1024, 0, 100000),
                       (3, k, 1, 1, "SQ_INSTS_VALU_MFMA_MOPS_F16", 1e12 / 512, 0, 100000)])
    profiling.main(["mfma", "--csv", str(p), "--key", "gemm_wb_kernel<12,", "--flops", "1e12"])
    line = [l for l in capsys.readouterr().out.splitlines() if l.startswith("| 3 |")][0]
    assert line == "| 3 | 25.0 % | 2.00 | 1.000 | 10000.0 | 100.0 |"


def test_valu_issue_per_launch_shape(tmp_path, capsys):
    p = tmp_path / "v.csv"
    k = "qmm::gemv_kernel<2, 2, 0>"
    # two shapes: 2048 wavefronts issuing 424 VALU each (10 us), and 7168 wavefronts issuing 424 each
    # (one dispatch 10 us, one 12 us); VALU cycles per SIMD = instructions x 4 / 1024
    write_counters(p, [(1, k, 131072, 256, "SQ_INSTS_VALU", 424.0 * 2048, 0, 10000),
                       (1, k, 131072, 256, "GRBM_GUI_ACTIVE", 1.0, 0, 10000),
                       (2, k, 458752, 256, "SQ_INSTS_VALU", 424.0 * 7168, 0, 10000),
                       (3, k, 458752, 256, "SQ_INSTS_VALU", 424.0 * 7168, 0, 12000)])
    profiling.main(["valu", "--csv", str(p), "--key", "gemv_kernel<2, 2, 0>", "--name", "131072=q_proj",
                    "--ghz", "2.0", "2.4"])
    rows = [l for l in capsys.readouterr().out.splitlines() if l.startswith("| q_proj") or l.startswith("| 458752")]
    c1 = 424 * 2048 * 4 / 1024  # 3392 cycles: 1.41 us at 2.4 GHz, 1.70 at 2.0
    assert rows[0] == f"| q_proj | 512 x 256 | 1 | 424 | {c1:.0f} | 1.41 / 1.70 | 10.00 | 14-17 % |"
    c2 = 424 * 7168 * 4 / 1024  # 11872 cycles: 4.95 us at 2.4 GHz, 5.94 at 2.0; mean duration 11 us
    assert rows[1] == f"| 458752 | 1792 x 256 | 2 | 424 | {c2:.0f} | 4.95 / 5.94 | 11.00 | 45-54 % |"


def test_bench_and_profiling_hash_the_same_sources():
    assert bench.kernel_source_hash() == profiling.kernel_source_hash()


def test_bench_traffic_lookup_requires_the_current_sources(tmp_path, monkeypatch):
    (tmp_path / "gguf_block_quant_qmm_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "gguf_block_quant_qmm_amd" / "csrc" / "k.hip").write_text("kernel v1\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.kernel_source_hash()
    rec = {"g": {"source_hash": h, "hbm_bytes_per_launch": 1234}}
    (tmp_path / "profiles" / "counters.json").write_text(json.dumps(rec))
    assert bench.load_traffic("g") == 1234
    assert bench.load_traffic("missing") is None
    # any edit of a kernel source makes the stored counters stale
    (tmp_path / "gguf_block_quant_qmm_amd" / "csrc" / "k.hip").write_text("kernel v2\n")
    assert bench.load_traffic("g") is None
    (tmp_path / "profiles" / "counters.json").write_text("not json")
    assert bench.load_traffic("g") is None


def test_counters_table_is_the_mean_per_dispatch(tmp_path):
    p = tmp_path / "c.csv"
    # two matching dispatches; each counter reported in two instances that sum per dispatch
    write_counters(p, [(1, "qmm::gemm_sk_kernel<12>", 64, 256, "SQ_WAVES", 100.0, 0, 10000),
                       (1, "qmm::gemm_sk_kernel<12>", 64, 256, "SQ_WAVES", 50.0, 0, 10000),
                       (2, "qmm::gemm_sk_kernel<12>", 64, 256, "SQ_WAVES", 250.0, 0, 30000),
                       (1, "qmm::gemm_sk_kernel<12>", 64, 256, "TCP_TCC_READ_REQ_sum", 4000.0, 0, 10000),
                       (2, "qmm::gemm_sk_kernel<12>", 64, 256, "TCP_TCC_READ_REQ_sum", 6000.0, 0, 30000),
                       (3, "other_kernel", 64, 256, "SQ_WAVES", 1e9, 0, 1)])
    out = tmp_path / "c.md"
    profiling.main(["counters", "--csv", str(p), "--key", "gemm_sk_kernel<12>", "--cmd", "cmd", "--out", str(out)])
    text = out.read_text()
    assert "| SQ_WAVES | 200 |" in text  # (150 + 250) / 2
    assert "| TCP_TCC_READ_REQ_sum | 5,000 |" in text
    assert "2 dispatches, mean duration 20.00 us" in text
