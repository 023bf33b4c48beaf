"""bench.py --record-traffic: the attention kernel's HBM bytes per launch from
rocprofv3 counter files (host logic only, synthetic CSVs).

FETCH_SIZE and WRITE_SIZE are KiB per dispatch summed over the counter's
instances; each is scaled by the ratio of the bytes a 1 GiB device copy
really moves to what the same counter reads for it."""
import csv
import os

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_run(d, counter, dispatches):
    """dispatches: list of (kernel name, [instance values])"""
    os.makedirs(os.path.join(d, "host"), exist_ok=True)
    with open(os.path.join(d, "host", "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, vals) in enumerate(dispatches):
            for v in vals:
                row = {k: "0" for k in FIELDS}
                row.update(Dispatch_Id=str(i + 1), Kernel_Name=name, Counter_Name=counter,
                           Counter_Value=str(v))
                w.writerow(row)


def test_record_traffic_scales_by_the_copy(tmp_path):
    att = "void " + bench.ATTEND_KERNEL + "(unsigned short const*, int)"
    other = "void abatt::k_scores<128, 8, true>(float const*)"
    gib_kib = (1 << 30) / 1024
    # the copy: FETCH reads half the bytes moved (scale 2), WRITE all of them (scale 1);
    # a small copy dispatch is ignored in favour of the 1 GiB one
    write_run(tmp_path / "copyf", "FETCH_SIZE",
              [("__amd_rocclr_copyBuffer", [gib_kib / 4, gib_kib / 4]), ("__amd_rocclr_copyBuffer", [3.0])])
    write_run(tmp_path / "copyw", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", [gib_kib])])
    # two attention dispatches (instances summed per dispatch, dispatches averaged)
    write_run(tmp_path / "fetch", "FETCH_SIZE",
              [(att, [100.0, 300.0]), (other, [7.0]), (att, [200.0, 400.0])])
    write_run(tmp_path / "write", "WRITE_SIZE", [(att, [10.0]), (att, [30.0]), (other, [1.0])])
    rec = bench.record_traffic(str(tmp_path))
    assert rec["kernel"] == bench.ATTEND_KERNEL
    assert rec["fetch_kib_per_launch"] == 500.0
    assert rec["write_kib_per_launch"] == 20.0
    assert abs(rec["copy_calibration"]["fetch_scale"] - 2.0) < 1e-12
    assert abs(rec["copy_calibration"]["write_scale"] - 1.0) < 1e-12
    assert rec["bytes_per_launch"] == (500.0 * 2 + 20.0) * 1024
    assert rec["other_kernels_kib_per_launch"]["abatt::k_scores<128, 8, true>"] == \
        {"fetch": 7.0, "write": 1.0}
    assert rec["attend_src_sha"] == bench.src_sha(os.path.join(
        bench.ROOT, "block_sparse_attention_09_amd", "csrc", "attend.hip"))
