"""The counter-summary tool: scaling by the copy calibration, and the source
hash that ties a stored figure to the kernel it was taken on."""
import json
import os

from bit_weight_only_w4a16_amd import traffic

HEADER = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id",'
          '"Grid_Size","Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size",'
          '"Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count","Counter_Name",'
          '"Counter_Value","Start_Timestamp","End_Timestamp"\n')


def _csv(path, counter, kernel_vals, copy_vals):
    os.makedirs(path, exist_ok=True)
    rows = [HEADER]
    i = 0
    for name, vals in (("w4::stream_kernel(w4::SweepOp const*, int, int const*)", kernel_vals),
                       ("w4::probe_copy_kernel(unsigned int __vector(4) const*, unsigned int "
                        "__vector(4)*, unsigned long)", copy_vals),
                       ("w4::pack_kernel(unsigned int const*)", [5.0])):
        for v in vals:
            i += 1
            rows.append('%d,%d,"Agent 1",1,1,1,256,1,"%s",256,0,0,8,0,32,"%s",%f,0,1\n'
                        % (i, i, name, counter, v))
    with open(os.path.join(path, "x_counter_collection.csv"), "w") as f:
        f.writelines(rows)


def test_traffic_scaling(tmp_path, monkeypatch):
    out = tmp_path / "t.json"
    monkeypatch.setattr(traffic, "OUT_FILE", str(out))
    # the copy reads 1 GiB; its FETCH_SIZE reads half of that, WRITE_SIZE all
    _csv(str(tmp_path / "f"), "FETCH_SIZE", [1000.0, 1002.0], [524288.0] * 3)
    _csv(str(tmp_path / "w"), "WRITE_SIZE", [10.0, 10.0], [1048576.0] * 3)
    traffic.main(["traffic", str(tmp_path / "f"), str(tmp_path / "w")])
    t = json.loads(out.read_text())
    assert t["copy_calibration"]["fetch_scale"] == 2.0
    assert t["copy_calibration"]["write_scale"] == 1.0
    assert t["hbm_bytes_per_launch"] == round(1001.0 * 1024 * 2 + 10.0 * 1024)
    assert t["algorithmic_weight_bytes_per_launch"] == 923_222_016
    assert t["kernel_source_hash"] == traffic.kernel_source_hash()
    assert t["dispatches"] == {"stream_kernel": 2, "probe_copy_kernel": 3}
