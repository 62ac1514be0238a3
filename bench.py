"""Benchmark of one GPU's share of the dynamic block-wise int8 quantized
AllReduce (EQuARX) on the outlier workload: N=8 ranks x 16,777,216 bf16
elements ~ N(0,1) with 0.1% N(0,1)*50 outliers, blocks of 256.

One step = the whole per-GPU path over one batch:
  1. quantize this GPU's own bf16 buffer (absmax -> scale -> int8 codes);
  2. one fused kernel over the N quantized contributions (this rank's and
     the N-1 peers', resident in HBM): dequantize, fp32 sum in rank order,
     requantize, and dequantize the result back to bf16.
The peers' codes are produced by the same quantize kernel before timing.
Buffer sets rotate every step (footprint > 1 GiB) so the 256 MB Infinity
Cache cannot serve a step from the previous one's data: inputs are resident
in HBM, not in cache, when a step starts.

Prints ONE JSON line.  value = bf16 payload bytes (N * n * 2) per step /
step time.  roofline = the dominant kernel (the fused reduce) against the
MI355X HBM peak; cpu_baseline = the CPU oracle on the same inputs.
Extra keys report each kernel's own time, the reduce without the fused
dequantize (N*qbytes read + qbytes written) and a ring step.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--sets S]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
DOMINANT = "k_reduce"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "block_wise_int8_amd", "csrc", f)
                  for f in ("qar_kernels.hip", "qar_device.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_key: str):
    """HBM bytes per launch of the dominant kernel from the committed
    counter summary, if it was taken on the current kernel sources."""
    path = os.path.join(PROFILES, f"reduce_{workload_key}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--sets", type=int, default=8, help="buffer sets rotated across steps")
    p.add_argument("--workload", default="outliers")
    p.add_argument("--skew", type=int, default=4096,
                   help="bytes added to the stride between rank code buffers in one allocation "
                        "(multiple of 16); -1 = one allocation per rank")
    p.add_argument("--cpu-reps", type=int, default=4, help="oracle repetitions for the CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip the reduce-only and ring-step lines")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="only run 8 device-to-device copies of this many MiB (counter calibration) and exit")
    return p.parse_args()


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share of the path; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from block_wise_int8_amd import qar, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    qar.lib()
    dev = torch.device("cuda:0")
    if args.copy_probe_mib:
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE of these
        # dispatches calibrate the counters (bytes read = bytes written =
        # copy size)
        nbytes = args.copy_probe_mib << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": nbytes, "launches": 8}))
        return 0
    w = synth.WORKLOADS[args.workload]
    N, n, B = w.nranks, w.n, w.block
    nb = n // B
    qbytes = n + 4 * nb

    t0 = time.time()
    host = synth.ranks(w)
    gen_s = time.time() - t0

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    # quantized contributions of every rank (set 0), then clones per set
    base_codes, base_scales = [], []
    for r in range(N):
        c, s = qar.qar_quantize_blocks(to_dev(host[r]), B)
        base_codes.append(c)
        base_scales.append(s)
    x_own = to_dev(host[0])
    out_dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    # The N rank code buffers of a set live in one allocation, rank r at
    # r * (n + skew) bytes: a stride that is not a large power of two keeps
    # the N concurrent streams on different HBM channels.
    stride = n + args.skew

    def rank_codes():
        if args.skew < 0:
            return [c.clone() for c in base_codes]
        big = torch.empty(N * stride, dtype=torch.int8, device=dev)
        views = [big[r * stride:r * stride + n] for r in range(N)]
        for v, c in zip(views, base_codes):
            v.copy_(c)
        return views

    sets = []
    for _ in range(args.sets):
        sets.append({
            "x": x_own.clone(),
            "codes": rank_codes(),
            "scales": [s.clone() for s in base_scales],
            "codes_out": torch.empty(n, dtype=torch.int8, device=dev),
            "scales_out": torch.empty(nb, dtype=torch.float32, device=dev),
            "out": torch.empty(n, dtype=out_dtype, device=dev),
        })
    torch.cuda.synchronize()
    if args.skew >= 0 and args.skew % 16:
        raise SystemExit("--skew must be a multiple of 16")
    set_bytes = sum(t.numel() * t.element_size() for t in
                    [sets[0]["x"], *sets[0]["codes"], *sets[0]["scales"], sets[0]["codes_out"],
                     sets[0]["scales_out"], sets[0]["out"]])

    stream = torch.cuda.current_stream()

    def quantize_own(st):
        qar.qar_quantize_blocks(st["x"], B, st["codes"][0], st["scales"][0], stream=stream)

    def reduce_fused(st):
        qar.qar_reduce_quantized(st["codes"], st["scales"], B, st["codes_out"], st["scales_out"],
                                 out=st["out"], stream=stream)

    def step(i):
        st = sets[i % len(sets)]
        quantize_own(st)
        reduce_fused(st)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # the timed region: K whole steps back to back, no events inside
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # each kernel of the step on its own: R launches back to back over the
    # rotated sets, one event pair around them (events between kernels
    # would add their own overhead to every launch)
    def per_launch_us(fn, reps):
        for i in range(3):
            fn(sets[i % len(sets)])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(reps):
            fn(sets[i % len(sets)])
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3

    reps = max(args.steps, 50)
    q_us = per_launch_us(quantize_own, reps)
    r_us = per_launch_us(reduce_fused, reps)

    payload = N * n * 2
    value = payload / (ms_per_step * 1e-3) / 1e9
    out_bytes = n * (2 if out_dtype == torch.bfloat16 else 4)
    reduce_bytes = N * qbytes + qbytes + out_bytes          # algorithmic, per launch
    quant_bytes = n * (2 if w.dtype == "bf16" else 4) + qbytes
    achieved = reduce_bytes / (r_us * 1e-6) / 1e9

    result = {
        "metric": "GB/s of bf16 payload reduced per GPU and % of HBM peak, fused quantized reduce",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.key}: {w.description}",
            "nranks": N, "elements_per_rank": n, "block": B, "input_dtype": w.dtype,
            "step": "quantize own buffer + fused reduce/requantize/dequantize of N contributions",
            "buffer_sets": args.sets, "footprint_bytes": set_bytes * args.sets,
            "rank_stride_bytes": stride if args.skew >= 0 else None,
            "parallelism": "one GPU's share",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": DOMINANT,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.key),
            "algorithmic_bytes_per_launch": reduce_bytes,
            "avg_launch_us": round(r_us, 3),
            "timing": f"{reps} back-to-back launches over the rotated sets, one HIP event pair",
        },
        "kernels": {
            "k_quantize": {"avg_us": round(q_us, 3), "bytes": quant_bytes,
                           "GBps": round(quant_bytes / (q_us * 1e-6) / 1e9, 1)},
            "k_reduce (fused bf16 out)": {"avg_us": round(r_us, 3), "bytes": reduce_bytes,
                                          "GBps": round(achieved, 1)},
        },
        "input_generation_s": round(gen_s, 2),
    }

    if not args.no_extras:
        result["reduce_only"] = reduce_only(args, qar, torch, sets, B, N, n, qbytes)
        result["ring_step"] = ring_bench(qar, torch, np, synth, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, np, w, host, sets[0], torch)

    print(json.dumps(result), flush=True)
    return 0


def reduce_only(args, qar, torch, sets, B, N, n, qbytes):
    """The fused reduce without the optional dequantized output: reads
    N*qbytes, writes qbytes."""
    stream = torch.cuda.current_stream()
    reps = max(args.steps, 20)
    for i in range(5):
        st = sets[i % len(sets)]
        qar.qar_reduce_quantized(st["codes"], st["scales"], B, st["codes_out"], st["scales_out"], stream=stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(reps):
        st = sets[i % len(sets)]
        qar.qar_reduce_quantized(st["codes"], st["scales"], B, st["codes_out"], st["scales_out"], stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    nbytes = (N + 1) * qbytes
    return {"avg_us": round(us, 3), "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "payload_GBps": round(N * n * 2 / (us * 1e-6) / 1e9, 1),
            "note": "back-to-back launches over rotated buffer sets, out=NULL"}


def ring_bench(qar, torch, np, synth, dev):
    """One ring step on the ring workload (N=4 x [2048, 3840] bf16, block
    256): read codes+scales and the bf16 local buffer, write codes+scales."""
    w = synth.WORKLOADS["ring"]
    host = synth.ranks(w)
    B, n = w.block, w.n
    nb = n // B
    S = 32                                   # 32 sets x 31.7 MB > 1 GiB
    x0 = torch.from_numpy(host[0].view(np.int16)).to(dev).view(torch.bfloat16)
    c0, s0 = qar.qar_quantize_blocks(x0, B)
    loc = torch.from_numpy(host[1].view(np.int16)).to(dev).view(torch.bfloat16)
    sets = [(c0.clone(), s0.clone(), loc.clone(), torch.empty_like(c0), torch.empty_like(s0)) for _ in range(S)]
    stream = torch.cuda.current_stream()
    for i in range(5):
        c, s, l, co, so = sets[i % S]
        qar.qar_ring_step(c, s, l, B, co, so, stream=stream)
    reps = 200
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(reps):
        c, s, l, co, so = sets[i % S]
        qar.qar_ring_step(c, s, l, B, co, so, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    nbytes = 2 * (n + 4 * nb) + 2 * n
    return {"workload": w.description, "avg_us": round(us, 3), "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def cpu_baseline(args, np, w, host, set0, torch):
    """The CPU oracle (plain scalar C, one thread) running the same step on
    the same inputs: quantize rank 0, reduce the N quantized ranks, dequantize
    the result.  Also checks the GPU step's output against it."""
    import oracle
    o = oracle.load()
    B = w.block
    qs = [o.quantize(x, B) for x in host]          # peers' contributions (untimed)
    codes = [q[0] for q in qs]
    scales = [q[1] for q in qs]
    reps = max(1, args.cpu_reps)
    t0 = time.perf_counter()
    for _ in range(reps):
        c0, s0 = o.quantize(host[0], B)
        oc, os_ = o.reduce([c0] + codes[1:], [s0] + scales[1:], B)
        y = o.dequantize(oc, os_, B, "bf16" if w.dtype == "bf16" else "f32")
    dt = (time.perf_counter() - t0) / reps
    gpu_codes = set0["codes_out"].cpu().numpy()
    gpu_out = set0["out"].contiguous().view(torch.int16 if w.dtype == "bf16" else torch.int32).cpu().numpy()
    same = bool(np.array_equal(gpu_codes, oc)) and bool(np.array_equal(gpu_out.view(y.dtype), y))
    return {"value": round(w.nranks * w.n * 2 / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole workload, {reps} repetitions of the step (quantize own buffer, reduce "
                      f"{w.nranks} ranks, dequantize); {dt:.3f} s per step on one host thread",
            "gpu_output_matches_oracle": same}


if __name__ == "__main__":
    sys.exit(main())
