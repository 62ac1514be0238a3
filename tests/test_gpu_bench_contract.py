"""bench.py's output contract on the GPU: one JSON line with the required
keys and types, the roofline and CPU-baseline objects, and a step that
matches the oracle (short run: few steps, no extras, a short CPU sample)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    print("running bench.py --steps 5 --warmup 2 --no-extras --cpu-seconds 1", flush=True)
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "2",
                          "--no-extras", "--cpu-seconds", "1"], capture_output=True, text=True, timeout=300,
                         cwd=ROOT)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [ln for ln in out.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    r = json.loads(lines[0])
    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)]:
        assert isinstance(r[key], typ), (key, r.get(key))
    assert r["n_gpus"] == 1 and r["steps"] == 5 and r["warmup"] == 2 and r["vs_baseline"] is None
    assert r["value"] > 0 and r["unit"] == "GB/s" and r["higher_is_better"] is True
    assert "workload" in r["config"]
    roof = r["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > 0
    cpu = r["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s" and cpu["cores"] >= 1 and cpu["value"] > 0
    assert cpu["gpu_output_matches_oracle"] is True and cpu["threads_agree_with_single_thread"] is True
