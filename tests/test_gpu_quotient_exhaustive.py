"""The fast quotient behind every quantize on the GPU path (reciprocal of
the block scale, one product, one FMA correction: qar::fast_quotient in
block_wise_int8_amd/csrc/qar_device.h) against the correctly rounded
binary32 quotient, on all 2^23 x 2^23 pairs of significands (x and s over
[1, 2)), run on the GPU by tests/quotient/quotient_sweep.hip with the
library's device code and compiler flags.  Each result is checked exactly
in binary64 (the residual x - y*s against half the spacing of y), with no
division, and so is the reciprocal 1/s of each of the 2^23 divisors.  The
checker itself must flag the uncorrected product x * (1/s) on some pairs.
The exponent range this extends to is checked on the CPU in
tests/test_quotient_exponents.py."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quotient", "libquotient_sweep.so")
SIG = 1 << 23
LAUNCHES = 64


def _sweep_lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    L.quotient_sweep.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p]
    L.quotient_sweep.restype = ctypes.c_int
    return L


def _buffers():
    dev = torch.device("cuda:0")
    bad = torch.zeros(SIG, dtype=torch.int32, device=dev)
    first = torch.full((SIG,), -1, dtype=torch.int32, device=dev)      # 0xFFFFFFFF: none yet
    recip = torch.zeros(SIG, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    return bad, first, recip


def _run(L, lo, count, mode, bufs):
    bad, first, recip = bufs
    assert L.quotient_sweep(lo, count, mode, bad.data_ptr(), first.data_ptr(), recip.data_ptr()) == 0


def test_checker_flags_the_uncorrected_product():
    L = _sweep_lib()
    bufs = _buffers()
    print("quotient checker: x * (1/s) over 4096 dividends x 2^23 divisors", flush=True)
    _run(L, 0, 4096, 1, bufs)
    torch.cuda.synchronize()
    bad, first, recip = bufs
    assert int(recip.sum()) == 0
    assert int(bad.sum()) > 0, "the checker found no fault in the uncorrected product"


def test_fast_quotient_is_correctly_rounded_on_every_significand_pair():
    L = _sweep_lib()
    bufs = _buffers()
    per = SIG // LAUNCHES
    for k in range(LAUNCHES):
        _run(L, k * per, per, 0, bufs)
        if k % 8 == 7:
            torch.cuda.synchronize()
            print(f"quotient sweep: {(k + 1) * per:,} of {SIG:,} dividend significands x {SIG:,} divisors done",
                  flush=True)
    torch.cuda.synchronize()
    bad, first, recip = bufs
    assert int(recip.sum()) == 0, "1/s is not correctly rounded for some divisor"
    nbad = int(bad.sum())
    if nbad:
        t = int(torch.nonzero(bad)[0])
        x = int(first[t]) & 0xFFFFFFFF
        pytest.fail(f"{nbad} mismatches; e.g. x = 1 + {x} * 2^-23, s = 1 + {t} * 2^-23")
