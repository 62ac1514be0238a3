"""bench.py's host logic on the CPU: the one-GPU refusal, and the arithmetic
that turns rocprofv3 counter values into HBM bytes (calibrated on a copy)."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert out.returncode == 2
    assert "one GPU" in out.stderr and not out.stdout


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, grid, ctr, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Grid_Size": grid, "Kernel_Name": name, "Counter_Name": ctr,
                        "Counter_Value": value})


def test_counter_summary_arithmetic(tmp_path):
    """A copy whose FETCH_SIZE reads half its bytes gives a fetch factor of
    2; kernels whose scaled counters equal their algorithmic bytes come out
    at traffic 1.0, one that reads 10% more at 1.1 of its reads; earlier
    dispatches of the same kernel and grid (set-up launches) are left out,
    and so are other grids of the same kernel."""
    copy = "__amd_rocclr_copyBuffer.kd"
    _counter_csv(str(tmp_path / "pmc_copy_fetch" / "c_counter_collection.csv"),
                 [(copy, 1 << 26, "FETCH_SIZE", (1 << 20) / 2)] * 8)
    _counter_csv(str(tmp_path / "pmc_copy_write" / "c_counter_collection.csv"),
                 [(copy, 1 << 26, "WRITE_SIZE", 1 << 20)] * 8)
    fetch, write, want = [], [], {}
    for key, what, name, grid, alg_r, alg_w in bench.counter_catalogue():
        scale = 1.1 if key == "ring_step" else 1.0
        last = 2 * bench.CHUNKS if key == "smallblock_reduce_chunk" else 4
        want[key] = (alg_r, alg_w, scale, last)
        full = f"void qar::{name}(args)"
        fetch += [(full, grid, "FETCH_SIZE", 1.0), (full, grid + 256, "FETCH_SIZE", 7.0)]       # set-up, other grid
        write += [(full, grid, "WRITE_SIZE", 1.0), (full, grid + 256, "WRITE_SIZE", 7.0)]
        fetch += [(full, grid, "FETCH_SIZE", alg_r * scale / 2 / 1024)] * last
        write += [(full, grid, "WRITE_SIZE", alg_w / 1024)] * last
    _counter_csv(str(tmp_path / "pmc_fetch" / "b_counter_collection.csv"), fetch)
    _counter_csv(str(tmp_path / "pmc_write" / "b_counter_collection.csv"), write)
    out = tmp_path / "profiles"
    out.mkdir()
    assert bench.summarize_counters(str(tmp_path), str(out)) == 0
    rec = json.loads((out / "hbm_traffic_all_kernels.json").read_text())
    assert rec["calibration"]["fetch_factor"] == 2.0 and rec["calibration"]["write_factor"] == 1.0
    for key, (alg_r, alg_w, scale, last) in want.items():
        r = rec["kernels"][key]
        assert r["dispatches"] == last
        assert abs(r["hbm_read_bytes"] - alg_r * scale) <= 2 and abs(r["hbm_write_bytes"] - alg_w) <= 2
        assert r["traffic_over_algorithmic"] == round((alg_r * scale + alg_w) / (alg_r + alg_w), 4)
    step = json.loads((out / "k_reduce_smallblock_counters.json").read_text())
    k5 = rec["kernels"]["smallblock_reduce_chunk"]
    assert step["hbm_bytes_per_step"] == bench.CHUNKS * (k5["hbm_read_bytes"] + k5["hbm_write_bytes"])
    assert step["kernel_source_sha256_16"] == bench.kernel_source_hash()
    top = json.loads((out / "k_quantize_reduce_outliers_counters.json").read_text())
    k2 = rec["kernels"]["outliers_step"]
    assert top["hbm_bytes_per_launch"] == k2["hbm_read_bytes"] + k2["hbm_write_bytes"]
