"""Host logic of the HBM-traffic summaries (rocprofv3 counter CSVs -> bytes per launch)."""
import argparse
import csv

from hierarchical_tiling_amd import counters

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for i, (name, counter, value) in enumerate(rows):
            r = {k: 0 for k in FIELDS}
            r.update(Dispatch_Id=i + 1, Kernel_Name=name, Counter_Name=counter, Counter_Value=value)
            w.writerow(r)


def test_summary_scales_by_copy_calibration_and_tracks_source(tmp_path):
    kern = "void htk::gemm_dma<2, 256, 256>(htk::KParams)"
    # the copy counter reads half of the 1 GiB copied per call -> factor 2 for fetch, 1 for write
    write_csv(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0)] * 5)
    write_csv(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)] * 5)
    write_csv(tmp_path / "f.csv", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 7.0),
                                   (kern, "FETCH_SIZE", 1000.0), (kern, "FETCH_SIZE", 3000.0)])
    write_csv(tmp_path / "w.csv", [(kern, "WRITE_SIZE", 10.0), (kern, "WRITE_SIZE", 30.0)])
    a = argparse.Namespace(fetch=str(tmp_path / "f.csv"), write=str(tmp_path / "w.csv"),
                           copy_fetch=str(tmp_path / "cf.csv"), copy_write=str(tmp_path / "cw.csv"),
                           kernel="bf16_x", kernel_match="gemm_dma", workload="wl",
                           command="cmd", copy_bytes=1 << 30, copies=5)
    s = counters.summarize(a)
    assert s["fetch_factor"] == 2.0 and s["write_factor"] == 1.0
    assert s["dispatches"] == [2, 2]
    assert s["traffic_bytes"] == int(2000.0 * 1024 * 2 + 20.0 * 1024)
    prof = tmp_path / "profiles"
    prof.mkdir()
    counters.write_summary(str(prof / "bf16_x_wl_traffic.txt"), s)
    got, src = counters.traffic_for("bf16_x", "wl", str(prof))
    assert got == s["traffic_bytes"] and src.endswith("bf16_x_wl_traffic.txt")
    # another kernel, another workload, or changed sources: no figure
    assert counters.traffic_for("bf16_y", "wl", str(prof))[0] is None
    assert counters.traffic_for("bf16_x", "other", str(prof))[0] is None
    s["source_digest"] = "0" * 16
    counters.write_summary(str(prof / "bf16_x_wl_traffic.txt"), s)
    got, why = counters.traffic_for("bf16_x", "wl", str(prof))
    assert got is None and "changed" in why
