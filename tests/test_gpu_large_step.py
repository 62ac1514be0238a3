"""The one-kernel step (quantize own + reduce) from 2^23 elements on, where
the library runs its 8-elements-per-lane kernel for int8 and E4M3 codes,
against the CPU oracle on every element: all three code formats (4-bit
codes keep the 16-per-lane kernel), bf16 and fp32 inputs, every output
kind, rank counts whose loads go dense (5, 8) and not (3, 9), the own rank
first, in the middle and last, and a ragged tail (n is a multiple of the
block but not of the 2048-element tile).  Below 2^23 the 16-per-lane kernel
runs for every format; the parity tests in test_gpu_parity.py,
test_gpu_e4m3.py and test_gpu_int4.py cover it."""
import functools

import numpy as np
import pytest
import torch

from block_wise_int8_amd import qar
from block_wise_int8_amd import synth
from gpu_util import SUM_OUTLIER, assert_same_bits16, assert_same_codes, assert_same_f32, mixed_f32, say, to_dev, to_host

pytestmark = pytest.mark.gpu

N_LARGE = (1 << 23) + 768        # 768: a multiple of every block size, not of 2048


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qar.lib()


FORMATS = {
    "int8": dict(step=qar.qar_quantize_reduce, q="quantize", r=lambda o, c, s, b, n: o.reduce(c, s, b),
                 d=lambda o, c, s, b, n, k: o.dequantize(c, s, b, k)),
    "e4m3": dict(step=qar.qar_quantize_reduce_e4m3, q="quantize_e4m3",
                 r=lambda o, c, s, b, n: o.reduce_e4m3(c, s, b),
                 d=lambda o, c, s, b, n, k: o.dequantize_e4m3(c, s, b, k)),
    "int4": dict(step=qar.qar_quantize_reduce_int4, q="quantize_int4",
                 r=lambda o, c, s, b, n: o.reduce_int4(c, s, b, n),
                 d=lambda o, c, s, b, n, k: o.dequantize_int4(c, s, b, n, k)),
}

CASES = [
    # fmt,  in,     N, own, block, out
    ("int8", "bf16", 8, 7, 256, "bf16"),
    ("int8", "f32", 3, 1, 64, "f32"),
    ("int8", "bf16", 9, 8, 128, None),
    ("int8", "f32", 5, 0, 256, "bf16"),
    ("e4m3", "bf16", 3, 2, 256, "f32"),
    ("e4m3", "f32", 8, 0, 64, "bf16"),
    ("e4m3", "bf16", 9, 4, 256, None),
    ("int4", "bf16", 5, 4, 256, "bf16"),
    ("int4", "f32", 9, 0, 128, "f32"),
    ("int4", "bf16", 3, 0, 64, None),
]


@functools.lru_cache(maxsize=None)
def _rank_f32(block: int, r: int) -> np.ndarray:
    # generating 2^23 elements takes about a second; the cases share them
    return mixed_f32(4100 + 97 * block + r, N_LARGE, block, SUM_OUTLIER)


def _rank(block: int, r: int, dtype: str) -> np.ndarray:
    x = _rank_f32(block, r)
    return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("fmt,dtype,nranks,own,block,out_kind", CASES)
def test_large_step_parity(oracle_lib, fmt, dtype, nranks, own, block, out_kind):
    f = FORMATS[fmt]
    n = N_LARGE
    xs = [_rank(block, r, dtype) for r in range(nranks)]
    qs = [getattr(oracle_lib, f["q"])(x, block) for x in xs]
    codes, scales = [q[0] for q in qs], [q[1] for q in qs]
    say(f"large step {fmt} {dtype} N={nranks} own={own} B={block} out={out_kind} n={n}")
    dc, ds = [to_dev(c) for c in codes], [to_dev(s) for s in scales]
    dc[own].fill_(0x55)                      # written by the call
    ds[own].fill_(-1.0)
    out = None
    if out_kind is not None:
        out = torch.empty(n, dtype=torch.bfloat16 if out_kind == "bf16" else torch.float32, device="cuda:0")
    oc, os_ = f["step"](to_dev(xs[own]), own, dc, ds, block, out=out)
    torch.cuda.synchronize()
    assert_same_codes(to_host(dc[own]).view(np.uint8), codes[own].view(np.uint8), "own codes")
    assert_same_f32(to_host(ds[own]), scales[own], "own scales")
    wc, ws = f["r"](oracle_lib, codes, scales, block, n)
    assert_same_codes(to_host(oc).view(np.uint8), wc.view(np.uint8), "codes")
    assert_same_f32(to_host(os_), ws, "scales")
    if out_kind is not None:
        want = f["d"](oracle_lib, wc, ws, block, n, out_kind)
        if out_kind == "bf16":
            assert_same_bits16(to_host(out), want, "out")
        else:
            assert_same_f32(to_host(out), want, "out")
