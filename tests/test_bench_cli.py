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
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, ctr, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": ctr, "Counter_Value": value})


def test_counter_summary_arithmetic(tmp_path):
    """A copy whose FETCH_SIZE reads half its bytes gives a fetch factor of
    2; kernels whose scaled counters equal their algorithmic bytes come out
    at traffic 1.0, and one that reads 10% more at 1.1 of its reads."""
    from block_wise_int8_amd import synth
    w = synth.WORKLOADS["outliers"]
    copy = "__amd_rocclr_copyBuffer.kd"
    _counter_csv(str(tmp_path / "pmc_copy_fetch" / "c_counter_collection.csv"),
                 [(copy, "FETCH_SIZE", (1 << 20) / 2)] * 8)
    _counter_csv(str(tmp_path / "pmc_copy_write" / "c_counter_collection.csv"),
                 [(copy, "WRITE_SIZE", 1 << 20)] * 8)
    fetch, write = [], []
    extra = {}
    for name, alg_r, alg_w in bench._counter_kernels(w.nranks, w.n, w.block):
        scale = 1.1 if name.startswith("k_quantize<") else 1.0
        extra[name.split("<")[0]] = (alg_r, alg_w, scale)
        fetch += [(f"void qar::{name}(args)", "FETCH_SIZE", alg_r * scale / 2 / 1024)] * 3
        write += [(f"void qar::{name}(args)", "WRITE_SIZE", alg_w / 1024)] * 3
    _counter_csv(str(tmp_path / "pmc_fetch" / "b_counter_collection.csv"), fetch)
    _counter_csv(str(tmp_path / "pmc_write" / "b_counter_collection.csv"), write)
    out = tmp_path / "summary.json"
    assert bench.summarize_counters(str(tmp_path), str(out)) == 0
    rec = json.loads(out.read_text())
    assert rec["calibration"]["fetch_factor"] == 2.0 and rec["calibration"]["write_factor"] == 1.0
    for k, (alg_r, alg_w, scale) in extra.items():
        r = rec["kernels"][k]
        assert r["dispatches"] == 3
        assert abs(r["hbm_read_bytes"] - alg_r * scale) <= 2 and abs(r["hbm_write_bytes"] - alg_w) <= 2
        assert r["traffic_over_algorithmic"] == round((alg_r * scale + alg_w) / (alg_r + alg_w), 4)
    top = rec["kernels"][bench.DOMINANT]
    assert rec["hbm_bytes_per_launch"] == top["hbm_read_bytes"] + top["hbm_write_bytes"]
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_hash()
