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


def test_trace_picks_the_timed_steps(tmp_path, capsys):
    """The timed steps are the decode launches W+1 .. W+K (W whole steps enqueued before
    them) with the launch just before (the planner) and just after (the combine) each, in
    start order whatever the file order."""
    path = tmp_path / "t_kernel_trace.csv"
    W, K = 2, 3
    rows, t = [], 0
    for step in range(W + K + 4):                # warm-up, timed, then settling steps
        timed = W <= step < W + K
        for name, d in (("void mla::mla_plan_kernel<true>(int)", 10 if timed else 1),
                        ("void mla::mla_decode_bf16_kernel<4, false>(mla::DecodeArgs)", 100 if timed else 7),
                        ("void mla::mla_combine_kernel(mla::CombineArgs)", 20 if timed else 3)):
            rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + 1000 * d})
            t += 1000 * d + 500
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in reversed(rows):
            w.writerow(r)
    res = profiling.trace(str(path), K, W)
    assert res["mla_decode_bf16_kernel<4, false>"]["timed"] == 100.0
    assert res["mla_plan_kernel<true>"]["timed"] == 10.0
    assert res["mla_combine_kernel"]["timed"] == 20.0
    assert "| mla_combine_kernel | 9 |" in capsys.readouterr().out
