"""Host checks of the rocprofv3 summary tool on small hand-made CSV files."""
import csv
import json

from block_diffusion_drafter_fwd_amd import profiling


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        for r in rows:
            w.writerow(r)


def test_traffic_scales_by_the_copy_calibration(tmp_path):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    # the counter reads half of what a 1 GiB copy fetched, all of what it wrote
    _write(tmp_path / "f.csv", hdr, [["__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0],
                                     ["k_gemm_skinny_p<4, 1>", "FETCH_SIZE", 100.0],
                                     ["k_gemm_skinny_p<4, 1>", "FETCH_SIZE", 300.0],
                                     ["k_other", "FETCH_SIZE", 9e9]])
    _write(tmp_path / "w.csv", hdr, [["__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0],
                                     ["k_gemm_skinny_p<4, 1>", "WRITE_SIZE", 10.0],
                                     ["k_gemm_skinny_p<4, 1>", "WRITE_SIZE", 30.0]])
    d = profiling.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), r"k_gemm_skinny_p<4, 1>")
    assert d["dispatches"] == 2
    assert abs(d["fetch_scale"] - 2.0) < 1e-9 and abs(d["write_scale"] - 1.0) < 1e-9
    assert d["hbm_bytes_per_launch"] == (200 * 1024 * 2) + (20 * 1024)


def test_stats_table_orders_by_time_and_cli_writes_json(tmp_path, capsys):
    hdr = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"]
    _write(tmp_path / "s.csv", hdr, [["a", 2, 2000, 1000, 10, 900, 1100, 1],
                                     ["b", 1, 18000, 18000, 90, 18000, 18000, 0]])
    text = profiling.stats(str(tmp_path / "s.csv"))
    lines = text.splitlines()
    assert lines[1].startswith("b") and lines[2].startswith("a")
    assert "total GPU kernel time 0.020 ms over 3 launches" in text
    hdr2 = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(tmp_path / "f.csv", hdr2, [["__amd_rocclr_copyBuffer", "FETCH_SIZE", 1048576.0], ["k", "FETCH_SIZE", 1.0]])
    _write(tmp_path / "w.csv", hdr2, [["__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0], ["k", "WRITE_SIZE", 1.0]])
    out = tmp_path / "o.json"
    profiling.main(["traffic", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
                    "--kernel", "^k$", "--out", str(out), "--command", "x"])
    d = json.load(open(out))
    assert d["hbm_bytes_per_launch"] == 2048 and d["command"] == "x"
    capsys.readouterr()
