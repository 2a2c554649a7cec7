"""Host logic of the rocprofv3 summary module: copy calibration and traffic per launch."""
import csv
import json
import os

import pytest

import profile_summary as ps

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_csv(d, counter, rows):
    os.makedirs(os.path.join(d, "host"), exist_ok=True)
    with open(os.path.join(d, "host", "pmc_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (k, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_uses_the_copy_calibration(tmp_path):
    gib = 1 << 30
    f, w = str(tmp_path / "f"), str(tmp_path / "w")
    # the counter reads half of a fetched copy and all of a written one; small copies are ignored
    write_csv(f, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", gib / 2048), ("__amd_rocclr_copyBuffer", 1.5),
                                ("void eff::(anonymous namespace)::k_gateup<0, 1>(args)", 100.0),
                                ("void eff::(anonymous namespace)::k_gateup<0, 1>(args)", 300.0),
                                ("void eff::(anonymous namespace)::k_down<0, 1>(args)", 7.0)])
    write_csv(w, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", gib / 1024),
                                ("void eff::(anonymous namespace)::k_gateup<0, 1>(args)", 10.0),
                                ("void eff::(anonymous namespace)::k_gateup<0, 1>(args)", 30.0)])
    out = str(tmp_path / "t.json")
    ps.main(["traffic", "--fetch", f, "--write", w, "--kernel", "k_gateup", "--copy-bytes", str(gib), "--out", out])
    d = json.load(open(out))
    assert d["fetch_factor"] == pytest.approx(2.0) and d["write_factor"] == pytest.approx(1.0)
    assert d["fetch_kib_per_dispatch"] == pytest.approx(200.0) and d["write_kib_per_dispatch"] == pytest.approx(20.0)
    assert d["hbm_bytes_per_launch"] == 200 * 1024 * 2 + 20 * 1024
    assert d["dispatches"] == [2, 2]


def test_source_hash_matches_the_bench():
    import bench
    assert ps.source_sha("k_decode.hip") == bench.src_hash("k_decode.hip")


def test_missing_counters_are_an_error(tmp_path):
    f = str(tmp_path / "f")
    write_csv(f, "FETCH_SIZE", [("void eff::k_gateup<0, 1>(args)", 1.0)])
    with pytest.raises(SystemExit):
        ps.main(["traffic", "--fetch", f, "--write", f, "--kernel", "k_gateup"])  # no copy to calibrate


def test_trace_window_averages(tmp_path, capsys):
    d = tmp_path / "t"
    os.makedirs(d / "host")
    with open(d / "host" / "x_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        # five dispatches of one kernel, out of order in the file; one of another kernel
        for start, dur in [(500, 9000), (100, 1000), (300, 3000), (400, 5000), (200, 2000)]:
            w.writerow({"Kernel_Name": "void eff::(anonymous namespace)::k_down<0, 1>(args)",
                        "Start_Timestamp": start, "End_Timestamp": start + dur})
        w.writerow({"Kernel_Name": "eff::(anonymous namespace)::k_control(args)", "Start_Timestamp": 50,
                    "End_Timestamp": 60})
    res = ps.main(["trace", str(d), "--kernel", "k_down", "--last", "2"]) or json.loads(capsys.readouterr().out)
    r = res["k_down<0, 1>"]
    assert r["dispatches"] == 5 and r["avg_us"] == pytest.approx(4.0)
    assert r["last"] == 2 and r["last_avg_us"] == pytest.approx(7.0)   # the two latest starts: 5000, 9000 ns
    res = ps.main(["trace", str(d), "--kernel", "k_down", "--skip", "2", "--last", "2"]) or json.loads(
        capsys.readouterr().out)
    r = res["k_down<0, 1>"]
    assert r["last"] == 2 and r["last_avg_us"] == pytest.approx(2.5)   # the two before those: 2000, 3000 ns


def test_traffic_last_window(tmp_path):
    f, w = str(tmp_path / "f"), str(tmp_path / "w")
    rows = [("__amd_rocclr_copyBuffer", 2048.0)] + [("void eff::k_gateup<0, 1>(a)", float(v)) for v in (1, 2, 3, 10, 20)]
    write_csv(f, "FETCH_SIZE", rows)
    write_csv(w, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 4096.0)] + [("void eff::k_gateup<0, 1>(a)", 1.0)] * 5)
    out = str(tmp_path / "t.json")
    ps.main(["traffic", "--fetch", f, "--write", w, "--kernel", "k_gateup", "--copy-bytes", str(1 << 22),
             "--last", "2", "--out", out])
    d = json.load(open(out))
    assert d["fetch_kib_per_dispatch"] == pytest.approx(15.0) and d["dispatches"] == [2, 2]   # the last two ids
