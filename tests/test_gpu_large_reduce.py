"""The reduce and the one-kernel step at sizes where the launcher deals
tiles to the XCDs in super-tiles of 64 (at least 8 ranks, at least 2^25
elements, a grid that is a multiple of 512 workgroups), against the CPU
oracle on every element.  Reduce: 8 ranks with 8 elements per lane (no
output and bf16 output), 16 ranks with load groups of 16 (no output), 9
ranks with load groups of 8 (fp32 output), and one size just past a
multiple of the super-tiles, where the launcher keeps the contiguous
ranges.  Step: int8 and E4M3 codes (8 elements per lane) and 4-bit codes
(16).  Every tile must be computed exactly once, so any flaw in the order
shows up as wrong or missing blocks."""
import numpy as np
import pytest
import torch

from block_wise_int8_amd import qar, synth
from gpu_util import assert_same_bits16, assert_same_codes, assert_same_f32, say, to_dev, to_host

pytestmark = pytest.mark.gpu

N25 = 1 << 25


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qar.lib()


def _ranks(seed: int, nranks: int, n: int, block: int) -> list:
    """bf16 data ~ N(0, 1) times a per-block log-normal magnitude (fast to
    draw at these sizes)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(nranks):
        x = rng.standard_normal(n, dtype=np.float32)
        x *= np.repeat(np.exp(rng.normal(0.0, 2.0, n // block)).astype(np.float32), block)
        out.append(synth.f32_to_bf16_bits(x))
    return out


CASES = [
    # nranks, n, block, out
    (8, N25, 256, None),
    (8, N25, 256, "bf16"),
    (16, N25, 64, None),
    (9, N25, 128, "f32"),
    (8, N25 + 5 * 256, 256, None),
]


@pytest.mark.parametrize("nranks,n,block,out_kind", CASES)
def test_large_reduce_parity(oracle_lib, nranks, n, block, out_kind):
    xs = _ranks(8000 + nranks, nranks, n, block)
    qs = [oracle_lib.quantize(x, block) for x in xs]
    del xs
    codes, scales = [q[0] for q in qs], [q[1] for q in qs]
    wc, ws = oracle_lib.reduce(codes, scales, block)
    say(f"large reduce N={nranks} n={n} B={block} out={out_kind}")
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    out = None
    if out_kind is not None:
        out = torch.empty(n, dtype=torch.bfloat16 if out_kind == "bf16" else torch.float32, device="cuda:0")
    oc, os_ = qar.qar_reduce_quantized(dc, ds, block, out=out)
    torch.cuda.synchronize()
    assert_same_codes(to_host(oc), wc, "codes")
    assert_same_f32(to_host(os_), ws, "scales")
    if out_kind == "bf16":
        assert_same_bits16(to_host(out), oracle_lib.dequantize(wc, ws, block, "bf16"), "bf16 out")
    elif out_kind == "f32":
        assert_same_f32(to_host(out), oracle_lib.dequantize(wc, ws, block, "f32"), "fp32 out")


STEP_CASES = [
    # fmt, nranks, own, block
    ("int8", 8, 3, 256),
    ("e4m3", 9, 8, 128),
    ("int4", 8, 0, 64),
]


@pytest.mark.parametrize("fmt,nranks,own,block", STEP_CASES)
def test_large_step_super_tiles(oracle_lib, fmt, nranks, own, block):
    n = N25
    quant, red, deq, step = {
        "int8": ("quantize", lambda c, s: oracle_lib.reduce(c, s, block),
                 lambda c, s: oracle_lib.dequantize(c, s, block, "bf16"), qar.qar_quantize_reduce),
        "e4m3": ("quantize_e4m3", lambda c, s: oracle_lib.reduce_e4m3(c, s, block),
                 lambda c, s: oracle_lib.dequantize_e4m3(c, s, block, "bf16"), qar.qar_quantize_reduce_e4m3),
        "int4": ("quantize_int4", lambda c, s: oracle_lib.reduce_int4(c, s, block, n),
                 lambda c, s: oracle_lib.dequantize_int4(c, s, block, n, "bf16"), qar.qar_quantize_reduce_int4),
    }[fmt]
    xs = _ranks(9000 + nranks, nranks, n, block)
    qs = [getattr(oracle_lib, quant)(x, block) for x in xs]
    codes, scales = [q[0] for q in qs], [q[1] for q in qs]
    wc, ws = red(codes, scales)
    say(f"large step {fmt} N={nranks} own={own} n={n} B={block}")
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    dc[own].fill_(0x55)
    ds[own].fill_(-1.0)
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")
    oc, os_ = step(to_dev(xs[own]), own, dc, ds, block, out=out)
    torch.cuda.synchronize()
    assert_same_codes(to_host(dc[own]).view(np.uint8), codes[own].view(np.uint8), "own codes")
    assert_same_f32(to_host(ds[own]), scales[own], "own scales")
    assert_same_codes(to_host(oc).view(np.uint8), wc.view(np.uint8), "codes")
    assert_same_f32(to_host(os_), ws, "scales")
    assert_same_bits16(to_host(out), deq(wc, ws), "bf16 out")
