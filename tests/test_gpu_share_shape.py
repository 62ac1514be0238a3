"""One GPU's share of an 8-GPU one-shot AllReduce at its real shape: N = 8
slices of 2,097,152 elements (the outlier workload's 16,777,216 over 8 GPUs),
block 256.  At this size the reduce takes 8 elements per lane for int8 and
E4M3 codes and 16 for 4-bit codes, and the step 16 for every format.  For
all three code formats: the reduce with no, bf16 and fp32 output and the
one-kernel step (bf16 and fp32 input, own rank in the middle), each against
the CPU oracle on every element; then the reduce and the step as bench.py
times them, captured in one HIP graph and replayed on fresh inputs, against
the oracle again."""
import functools

import numpy as np
import pytest
import torch

from block_wise_int8_amd import qar, synth
from gpu_util import SUM_OUTLIER, assert_same_bits16, assert_same_codes, assert_same_f32, mixed_f32, say, to_dev, to_host

pytestmark = pytest.mark.gpu

N, n, B, OWN = 8, 2_097_152, 256, 3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qar.lib()


FORMATS = {
    "int8": dict(quant="quantize", red=qar.qar_reduce_quantized, step=qar.qar_quantize_reduce,
                 r=lambda o, c, s: o.reduce(c, s, B), d=lambda o, c, s, k: o.dequantize(c, s, B, k)),
    "e4m3": dict(quant="quantize_e4m3", red=qar.qar_reduce_quantized_e4m3, step=qar.qar_quantize_reduce_e4m3,
                 r=lambda o, c, s: o.reduce_e4m3(c, s, B), d=lambda o, c, s, k: o.dequantize_e4m3(c, s, B, k)),
    "int4": dict(quant="quantize_int4", red=qar.qar_reduce_quantized_int4, step=qar.qar_quantize_reduce_int4,
                 r=lambda o, c, s: o.reduce_int4(c, s, B, n), d=lambda o, c, s, k: o.dequantize_int4(c, s, B, n, k)),
}


@functools.lru_cache(maxsize=None)
def _slice_f32(seed: int, r: int) -> np.ndarray:
    return mixed_f32(seed + r, n, B, SUM_OUTLIER)


def _inputs(seed: int, dtype: str):
    xs = [_slice_f32(seed, r) for r in range(N)]
    return [synth.f32_to_bf16_bits(x) for x in xs] if dtype == "bf16" else xs


def _check_out(got, want, kind, what):
    if kind == "bf16":
        assert_same_bits16(got, want, what)
    else:
        assert_same_f32(got, want, what)


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_share_reduce_every_output(oracle_lib, fmt):
    f = FORMATS[fmt]
    xs = _inputs(5000, "bf16")
    qs = [getattr(oracle_lib, f["quant"])(x, B) for x in xs]
    codes, scales = [q[0] for q in qs], [q[1] for q in qs]
    wc, ws = f["r"](oracle_lib, codes, scales)
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    for out_kind in (None, "bf16", "f32"):
        say(f"share shape: {fmt} reduce N={N} x {n} out={out_kind}")
        out = None if out_kind is None else torch.empty(
            n, dtype=torch.bfloat16 if out_kind == "bf16" else torch.float32, device="cuda:0")
        oc, os_ = f["red"](dc, ds, B, out=out)
        torch.cuda.synchronize()
        assert_same_codes(to_host(oc).view(np.uint8), wc.view(np.uint8), f"{fmt} codes")
        assert_same_f32(to_host(os_), ws, f"{fmt} scales")
        if out_kind is not None:
            _check_out(to_host(out), f["d"](oracle_lib, wc, ws, out_kind), out_kind, f"{fmt} {out_kind} out")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", list(FORMATS))
def test_share_step(oracle_lib, fmt, dtype):
    f = FORMATS[fmt]
    xs = _inputs(6000, dtype)
    qs = [getattr(oracle_lib, f["quant"])(x, B) for x in xs]
    codes, scales = [q[0] for q in qs], [q[1] for q in qs]
    wc, ws = f["r"](oracle_lib, codes, scales)
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    dc[OWN].fill_(0x55)
    ds[OWN].fill_(-1.0)
    say(f"share shape: {fmt} step N={N} x {n} {dtype} own={OWN}")
    out = torch.empty(n, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda:0")
    oc, os_ = f["step"](to_dev(xs[OWN]), OWN, dc, ds, B, out=out)
    torch.cuda.synchronize()
    assert_same_codes(to_host(dc[OWN]).view(np.uint8), codes[OWN].view(np.uint8), f"{fmt} own codes")
    assert_same_f32(to_host(ds[OWN]), scales[OWN], f"{fmt} own scales")
    assert_same_codes(to_host(oc).view(np.uint8), wc.view(np.uint8), f"{fmt} codes")
    assert_same_f32(to_host(os_), ws, f"{fmt} scales")
    _check_out(to_host(out), f["d"](oracle_lib, wc, ws, dtype), dtype, f"{fmt} out")


def test_share_graph_replays(oracle_lib):
    """bench.py times this shape as HIP graph replays of the binding's calls:
    the int8 reduce (no output) and step (bf16 in and out) captured once,
    replayed on three fresh input sets copied in eagerly, each replay
    against the oracle."""
    dc = [torch.empty(n, dtype=torch.int8, device="cuda:0") for _ in range(N)]
    ds = [torch.empty(n // B, dtype=torch.float32, device="cuda:0") for _ in range(N)]
    x_own = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")
    rc = torch.empty(n, dtype=torch.int8, device="cuda:0")
    rs = torch.empty(n // B, dtype=torch.float32, device="cuda:0")
    fc, fs = torch.empty_like(rc), torch.empty_like(rs)
    own_c, own_s = torch.empty_like(rc), torch.empty_like(rs)
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")

    def calls():
        qar.qar_reduce_quantized(dc, ds, B, rc, rs)
        qar.qar_quantize_reduce(x_own, OWN, dc[:OWN] + [own_c] + dc[OWN + 1:], ds[:OWN] + [own_s] + ds[OWN + 1:],
                                B, fc, fs, out=out)

    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        xs = _inputs(7000 + 100 * rep, "bf16")
        qs = [oracle_lib.quantize(x, B) for x in xs]
        for r, (c, s) in enumerate(qs):
            dc[r].copy_(to_dev(c))
            ds[r].copy_(to_dev(s))
        x_own.copy_(to_dev(xs[OWN]))
        torch.cuda.synchronize()
        say(f"share shape: graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        wc, ws = oracle_lib.reduce([q[0] for q in qs], [q[1] for q in qs], B)
        assert_same_codes(to_host(rc), wc, f"replay {rep}: reduce codes")
        assert_same_f32(to_host(rs), ws, f"replay {rep}: reduce scales")
        assert_same_codes(to_host(own_c), qs[OWN][0], f"replay {rep}: own codes")
        assert_same_codes(to_host(fc), wc, f"replay {rep}: step codes")
        assert_same_f32(to_host(fs), ws, f"replay {rep}: step scales")
        assert_same_bits16(to_host(out), oracle_lib.dequantize(wc, ws, B, "bf16"), f"replay {rep}: step out")
    del g
