"""Host-side checks of the rocprofv3 summarizer on small hand-made CSV files."""
import csv
import json
import os

from rate_allocated_weight_amd import profsum

CC_FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
             "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
             "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
             "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _cc(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, CC_FIELDS)
        w.writeheader()
        for i, (name, counter, value) in enumerate(rows):
            r = {k: 0 for k in CC_FIELDS}
            r.update(Dispatch_Id=i + 1, Kernel_Name=name, Counter_Name=counter, Counter_Value=value)
            w.writerow(r)


def test_short_names():
    s = profsum._short
    assert s("void wsic::(anonymous namespace)::k_sic_super<true, true>(wsic::SuperArgs)") == \
        "k_sic_super<true, true>"
    assert s("wsic::(anonymous namespace)::k_hist(int const*, long)") == "k_hist"
    assert s("__amd_rocclr_copyBuffer.kd") == "__amd_rocclr_copyBuffer"
    assert profsum.family_of("k_hist") == "hist"
    assert profsum.family_of("k_hist_cols") is None
    assert profsum.family_of("k_sic_super<false, true>") == "sic_leaf"


def test_traffic_record_scaling(tmp_path):
    mib = 4
    # the copy reads half of its bytes through the counted path, writes all of them
    _cc(str(tmp_path / "cf" / "x_counter_collection.csv"),
        [("__amd_rocclr_copyBuffer", "FETCH_SIZE", mib * 1024 / 2)])
    _cc(str(tmp_path / "cw" / "x_counter_collection.csv"),
        [("__amd_rocclr_copyBuffer", "WRITE_SIZE", mib * 1024)])
    k1 = "void wsic::(anonymous namespace)::k_hist(int const*)"
    k2 = "void wsic::(anonymous namespace)::k_sic_super<true, true>(wsic::SuperArgs)"
    k3 = "void wsic::(anonymous namespace)::k_sic_super<false, true>(wsic::SuperArgs)"
    _cc(str(tmp_path / "f" / "a" / "r_counter_collection.csv"),
        [(k1, "FETCH_SIZE", 100.0), (k1, "FETCH_SIZE", 300.0), (k2, "FETCH_SIZE", 10.0),
         (k3, "FETCH_SIZE", 30.0), (k2, "GRBM_COUNT", 5.0)])
    _cc(str(tmp_path / "w" / "r_counter_collection.csv"),
        [(k1, "WRITE_SIZE", 1.0), (k1, "WRITE_SIZE", 3.0), (k2, "WRITE_SIZE", 4.0),
         (k3, "WRITE_SIZE", 8.0)])
    out = tmp_path / "out"
    profsum.main(["--workload", "wl", "--name", "wl", "--fetch", str(tmp_path / "f"),
                  "--write", str(tmp_path / "w"), "--calib-fetch", str(tmp_path / "cf"),
                  "--calib-write", str(tmp_path / "cw"), "--calib-mib", str(mib),
                  "--cmd", "rocprofv3 --pmc FETCH_SIZE -- x", "--out", str(out)])
    rec = json.load(open(out / "traffic_wl.txt"))
    assert abs(rec["copy_scale_read"] - 2.0) < 1e-12 and abs(rec["copy_scale_write"] - 1.0) < 1e-12
    h = rec["families"]["hist"]
    assert h["launches_profiled"] == 2
    assert h["read_bytes_per_launch"] == 2.0 * 1024 * 200.0
    assert h["write_bytes_per_launch"] == 1024 * 2.0
    s = rec["families"]["sic_leaf"]
    assert s["launches_profiled"] == 2
    assert s["read_bytes_per_launch"] == 2.0 * 1024 * 20.0
    assert s["source"].endswith("k_sic.hip") and len(s["source_sha256"]) == 64
    assert "FETCH_SIZE" in (out / "wl_counters.md").read_text()
