"""The counter-summary tool: scaling by the copy calibration, and the source
hash that ties a stored figure to the kernel it was taken on."""
import json
import os

import pytest

from bit_weight_only_w4a16_amd import traffic

HEADER = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id",'
          '"Grid_Size","Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size",'
          '"Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count","Counter_Name",'
          '"Counter_Value","Start_Timestamp","End_Timestamp"\n')


def _csv(path, counter, kernel_vals, copy_vals,
         kernel="w4::stream_kernel(w4::SweepOp const*, int, int const*)"):
    os.makedirs(path, exist_ok=True)
    rows = [HEADER]
    i = 0
    for name, vals in ((kernel, kernel_vals),
                       ("w4::probe_copy_kernel(unsigned int __vector(4) const*, unsigned int "
                        "__vector(4)*, unsigned long)", copy_vals),
                       ("w4::pack_kernel(unsigned int const*)", [5.0])):
        for v in vals:
            i += 1
            rows.append('%d,%d,"Agent 1",1,1,1,256,1,"%s",256,0,0,8,0,32,"%s",%f,0,1\n'
                        % (i, i, name, counter, v))
    with open(os.path.join(path, "x_counter_collection.csv"), "w") as f:
        f.writelines(rows)


@pytest.mark.parametrize("mode,kernel", [
    ("stream", "w4::stream_kernel(w4::SweepOp const*, int, int const*)"),
    ("persistent", "w4::ordered_kernel(w4::SweepOp const*, int, w4::SweepCtl*, int, int)")])
def test_traffic_scaling(tmp_path, monkeypatch, mode, kernel):
    out = tmp_path / "t.json"
    monkeypatch.setattr(traffic, "out_file", lambda m: str(out))
    # the copy reads 1 GiB; its FETCH_SIZE reads half of that, WRITE_SIZE all
    _csv(str(tmp_path / "f"), "FETCH_SIZE", [1000.0, 1002.0], [524288.0] * 3, kernel)
    _csv(str(tmp_path / "w"), "WRITE_SIZE", [10.0, 10.0], [1048576.0] * 3, kernel)
    traffic.main(["traffic", mode, str(tmp_path / "f"), str(tmp_path / "w")])
    t = json.loads(out.read_text())
    assert t["copy_calibration"]["fetch_scale"] == 2.0
    assert t["copy_calibration"]["write_scale"] == 1.0
    assert t["hbm_bytes_per_launch"] == round(1001.0 * 1024 * 2 + 10.0 * 1024)
    assert t["algorithmic_weight_bytes_per_launch"] == 923_222_016
    assert t["kernel_source_hash"] == traffic.kernel_source_hash(mode)
    assert t["dispatches"] == {kernel.split("(")[0].split("::")[1]: 2, "probe_copy_kernel": 3}


def test_traffic_hashes_differ_per_kernel():
    assert traffic.kernel_source_hash("stream") != traffic.kernel_source_hash("persistent")
    with pytest.raises(KeyError):
        traffic.out_file("graph")
