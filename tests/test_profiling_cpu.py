"""Host logic of the profile summaries: counter scaling by the calibration copy."""
import csv
import json

from mla_decode_03_amd import profiling


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_scales_by_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    dec = "void mla::mla_decode_bf16_kernel<1>(mla::DecodeArgs)"
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    # two counter instances per dispatch are summed; a small setup copy is ignored
    _write(f, [
        {"Dispatch_Id": 1, "Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 3},
        {"Dispatch_Id": 2, "Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 500},
        {"Dispatch_Id": 2, "Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 500},
        {"Dispatch_Id": 3, "Kernel_Name": dec, "Counter_Name": "FETCH_SIZE", "Counter_Value": 250},
        {"Dispatch_Id": 4, "Kernel_Name": dec, "Counter_Name": "FETCH_SIZE", "Counter_Value": 300},
        {"Dispatch_Id": 5, "Kernel_Name": dec, "Counter_Name": "FETCH_SIZE", "Counter_Value": 350},
    ])
    _write(w, [
        {"Dispatch_Id": 2, "Kernel_Name": copy, "Counter_Name": "WRITE_SIZE", "Counter_Value": 2000},
        {"Dispatch_Id": 3, "Kernel_Name": dec, "Counter_Name": "WRITE_SIZE", "Counter_Value": 100},
    ])
    out = tmp_path / "t.json"
    profiling.traffic(str(f), str(w), copy_bytes=1000 * 1024, out=str(out))
    rec = json.loads(out.read_text())
    assert rec["fetch"]["bytes_per_count"] == 1024.0          # 1000 KiB copied, counter read 1000
    assert rec["fetch"]["bytes_per_launch"] == 300 * 1024     # median of the decode launches
    assert rec["write"]["bytes_per_count"] == 512.0
    assert rec["hbm_bytes_per_launch"] == 300 * 1024 + 100 * 512
    assert rec["kernel_source_sha"] == profiling.kernel_source_hash()


def test_kernel_source_hash_is_stable():
    assert profiling.kernel_source_hash() == profiling.kernel_source_hash()
    assert len(profiling.kernel_source_hash()) == 16
