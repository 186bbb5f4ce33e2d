"""Host checks of the rocprofv3 summary tool on small synthetic CSV files
(the column names rocprofv3 writes with --output-format csv)."""
import csv
import json
import os

from deformable_convolution_vision_dcnv4_amd import build, rocprof_summary
from deformable_convolution_vision_dcnv4_amd.workloads import WORKLOADS

OP = "void dcnv4::(anonymous namespace)::k_window<1, 2, 1, 0, 1024>(dcnv4::KArgs, unsigned int, unsigned int)"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def _counters(path, counter, copy_kib, op_kib):
    hdr = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
           "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
           "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows, d = [], 0
    for v in copy_kib:
        d += 1
        rows.append([d, d, "Agent 1", 1, 1, 1, 131072, 5, "__amd_rocclr_copyBuffer", 512, 0, 0, 8, 0, 32,
                     counter, v, 0, 1])
    for v in op_kib:
        d += 1
        rows.append([d, d, "Agent 1", 1, 1, 1, 262144, 7, OP, 1024, 0, 0, 128, 0, 64, counter, v, 0, 1])
    _write(path, hdr, rows)


def test_summary_scales_counters_by_copy_calibration(tmp_path):
    wl = WORKLOADS["fiit_stage1"]
    s = 2
    Ho, Wo = wl.out_hw()
    x_b = wl.N * wl.H * wl.W * wl.C * s
    off_b = wl.N * Ho * Wo * wl.G * 2 * wl.P * s
    m_b = wl.N * Ho * Wo * wl.G * wl.P * s
    # FETCH_SIZE reads half of a copy's bytes, WRITE_SIZE all of them
    fetch_copies = [x_b / 2048, off_b / 2048, m_b / 2048] * 2
    write_copies = [x_b / 1024, off_b / 1024, m_b / 1024] * 2
    op_fetch_kib = (x_b + off_b + m_b) / 2048 * 1.1     # 10% above algorithmic reads
    op_write_kib = x_b / 1024
    _counters(str(tmp_path / "f" / "pmc" / "pmc_counter_collection.csv"), "FETCH_SIZE", fetch_copies,
              [op_fetch_kib] * 3)
    _counters(str(tmp_path / "w" / "pmc" / "pmc_counter_collection.csv"), "WRITE_SIZE", write_copies,
              [op_write_kib] * 3)
    _write(str(tmp_path / "k" / "kt_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
           [[OP, 10, 500000, 50000.0, 99.0, 49000, 51000, 100.0],
            ["__amd_rocclr_copyBuffer", 6, 6000, 1000.0, 1.0, 900, 1100, 10.0]])
    out = str(tmp_path / "prof" / "fiit_stage1_f16")
    os.makedirs(os.path.dirname(out))
    rc = rocprof_summary.main(["--workload", "fiit_stage1", "--dtype", "f16", "--stats", str(tmp_path / "k"),
                               "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"),
                               "--command", "CMD", "--counter-command", "CCMD", "--out", out])
    assert rc == 0
    rec = json.load(open(out + "_hbm_counters.json"))
    assert abs(rec["fetch_factor"] - 2.0) < 1e-9 and abs(rec["write_factor"] - 1.0) < 1e-9
    assert abs(rec["hbm_read_bytes_per_launch"] - 1.1 * (x_b + off_b + m_b)) <= 2
    assert abs(rec["hbm_write_bytes_per_launch"] - x_b) <= 2
    assert rec["algorithmic_bytes_per_launch"] == wl.algorithmic_bytes("f16")
    assert rec["kernel_source_hash"] == build.source_hash("forward")
    assert rec["command"] == "CCMD"
    txt = open(out + "_kernel_trace.txt").read()
    assert "command: CMD" in txt and "50.000" in txt
    gbs = wl.algorithmic_bytes("f16") / 50e-6 / 1e9
    assert f"{gbs:.1f} GB/s" in txt


def test_summary_reports_l2_hit_rate_and_per_unit_counts(tmp_path):
    """Counters collected beside FETCH_SIZE / WRITE_SIZE in the same runs:
    L2 hit rate = hits / (hits + misses); wave instructions x 64 / units;
    bank-conflict cycles / LDS-busy cycles."""
    import csv as _csv
    wl = WORKLOADS["fiit_stage1"]
    units = wl.units()

    def multi(path, entries):
        hdr = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
               "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
               "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w", newline="") as fh:
            w = _csv.writer(fh, quoting=_csv.QUOTE_NONNUMERIC)
            w.writerow(hdr)
            d = 0
            for name, counter, v in entries:
                d += 1
                w.writerow([d, d, "Agent 1", 1, 1, 1, 1, 1, name, 1024, 0, 0, 128, 0, 64, counter, v, 0, 1])

    copy = "__amd_rocclr_copyBuffer"
    f_entries = [(copy, "FETCH_SIZE", 1.0)] * 3 + [(OP, "FETCH_SIZE", 2.0)]
    f_entries += [(OP, "SQ_INSTS_VALU", units * 1000 / 64), (OP, "SQ_INSTS_LDS", units * 80 / 64),
                  (OP, "SQ_LDS_BANK_CONFLICT", 30.0), (OP, "SQ_LDS_IDX_ACTIVE", 120.0),
                  (copy, "SQ_INSTS_VALU", 5.0)]
    w_entries = [(copy, "WRITE_SIZE", 1.0)] * 3 + [(OP, "WRITE_SIZE", 2.0), (OP, "TCC_HIT_sum", 300.0),
                                                   (OP, "TCC_MISS_sum", 100.0), (copy, "TCC_HIT_sum", 7.0)]
    multi(str(tmp_path / "f" / "pmc_counter_collection.csv"), f_entries)
    multi(str(tmp_path / "w" / "pmc_counter_collection.csv"), w_entries)
    out = str(tmp_path / "o" / "x")
    os.makedirs(os.path.dirname(out))
    assert rocprof_summary.main(["--workload", "fiit_stage1", "--dtype", "f16", "--fetch", str(tmp_path / "f"),
                                 "--write", str(tmp_path / "w"), "--command", "C", "--out", out]) == 0
    rec = json.load(open(out + "_hbm_counters.json"))
    assert rec["l2_hit"] == 0.75
    assert rec["valu_lane_ops_per_unit"] == 1000.0 and rec["lds_lane_ops_per_unit"] == 80.0
    assert rec["lds_bank_conflict_share"] == 0.25
    txt = open(out + "_hbm_counters.txt").read()
    assert "L2 (TCC) hit rate: 0.750" in txt and "1000 lane operations per (pixel, group) unit" in txt


def test_source_hash_is_stable_and_short():
    h = build.source_hash()
    assert h == build.source_hash() and len(h) == 16
    f = build.source_hash("forward")
    assert f == build.source_hash("forward") and len(f) == 16 and f != h


def test_committed_counter_records_match_the_forward_source():
    """Every measured configuration has a counter record in profiles/ taken on
    the current forward kernel source (bench.py reports the record's HBM
    traffic and L2 hit rate only when the source hashes agree)."""
    from deformable_convolution_vision_dcnv4_amd.workloads import CONFIGS
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")
    want = build.source_hash("forward")
    for name, dtype in CONFIGS:
        path = os.path.join(root, f"{name}_{dtype}_hbm_counters.json")
        assert os.path.exists(path), path
        with open(path) as fh:
            rec = json.load(fh)
        assert rec["kernel_source_hash"] == want, f"{path} was taken on another forward source"
        assert rec["hbm_bytes_per_launch"] > 0 and 0.0 < rec["l2_hit"] < 1.0
