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
    top = json.loads((out / os.path.basename(bench.counters_path("outliers"))).read_text())
    k2 = rec["kernels"]["outliers_step"]
    assert top["hbm_bytes_per_launch"] == k2["hbm_read_bytes"] + k2["hbm_write_bytes"]


def test_kernel_trace_summary(tmp_path):
    """The all-kernels trace table: one row per libqar kernel and launch
    size with its dispatch count and durations; the launch size names the
    workload (16 elements per lane, 8 for the kernels whose name ends in 8;
    a ragged launch rounds up to whole tiles); other kernels are left out."""
    rows = [("void qar::k_reduce<64, -1, qar::FlatLanes<64>, qar::Int8Codes, 16>(x)", 524288, [(0, 25000), (0, 27000)]),
            ("void qar::k_reduce8<256, 0, qar::Int8Codes>(x)", 2097152, [(0, 30000)]),
            ("void qar::k_quantize_reduce<128, 0, unsigned short, qar::Int8Codes, false>(x)", 256, [(0, 3000)]),
            ("void qar::k_reduce_unquantized<unsigned short>(x)", 491520, [(0, 14000)]),
            ("void qar::k_ring_step<256, unsigned short, qar::FlatLanes<256>, qar::Int8Codes>(x)", 30720,
             [(0, 3000)]),
            ("__amd_rocclr_copyBuffer", 1 << 20, [(0, 9000)])]
    d = tmp_path / "prof"
    d.mkdir()
    with open(d / "bench_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"])
        w.writeheader()
        for name, grid, spans in rows:
            for t0, t1 in spans:
                w.writerow({"Kernel_Name": name, "Start_Timestamp": t0, "End_Timestamp": t1, "Grid_Size_X": grid})
    out = tmp_path / "profiles"
    out.mkdir()
    assert bench.summarize_kernel_trace(str(d), str(out)) == 0
    table = [ln for ln in (out / "kernel_trace_all_kernels.md").read_text().splitlines() if ln.startswith("| ")]
    body = {ln.split("|")[1].strip().strip("*`"): [c.strip() for c in ln.split("|")[2:-1]] for ln in table[1:]}
    assert len(body) == 5 and not any("copyBuffer" in k for k in body)
    head = body["k_reduce<64, -1, FlatLanes<64>, Int8Codes, 16>"]
    assert head[:5] == ["524,288", "8,388,608", f"small-block, {bench.CHUNKS} chunks (the headline)", "2", "26.00"]
    assert body["k_reduce8<256, 0, Int8Codes>"][1:3] == ["16,777,216", "outliers: N=8 x 16,777,216 bf16"]
    assert body["k_quantize_reduce<128, 0, unsigned short, Int8Codes, false>"][2] == "tiny: N=4 x 4,096 bf16"
    assert body["k_reduce_unquantized<unsigned short>"][2].startswith("ring: N=4")
    assert body["k_ring_step<256, unsigned short, FlatLanes<256>, Int8Codes>"][2] == \
        "simulated all-reduce of the ring workload, 16 chunks"


def test_kernel_hash_ignores_comments_only():
    """The counter summaries record a hash of the kernel code: editing a
    comment or a blank line keeps it, editing code (also inside a string
    literal, or a // inside one) changes it."""
    base = 'int f(int x) { // one\n  /* two\n three */ return x + 1; }\nconst char* s = "a // b";\n'
    same = ['int f(int x) { // other words\n  /* changed */ return x + 1; }\n\nconst char* s = "a // b";   \n',
            'int f(int x) {\n  return x + 1; }\nconst char* s = "a // b";\n']
    other = ['int f(int x) { // one\n  /* two */ return x + 2; }\nconst char* s = "a // b";\n',
             'int f(int x) { return x + 1; }\nconst char* s = "a // c";\n']
    h = bench.code_without_comments
    assert all(h(t) == h(base) for t in same)
    assert all(h(t) != h(base) for t in other)
