"""Randomized pins (hypothesis): the oracle against the exact-rational brute
force on arbitrary bit patterns, block lengths and rank counts.  No GPU."""
from fractions import Fraction

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import brute

FINITE_F32 = st.integers(0, 2 ** 32 - 1).filter(lambda u: ((u >> 23) & 0xFF) != 0xFF)
FINITE_BF16 = st.integers(0, 2 ** 16 - 1).filter(lambda u: ((u >> 7) & 0xFF) != 0xFF)
COMMON = settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def _f32(bits):
    return np.array(bits, np.uint32).view(np.float32)


@COMMON
@given(st.lists(FINITE_F32, min_size=1, max_size=24), st.integers(1, 9))
def test_quantize_fp32_any_bits(oracle_lib, bits, block):
    x = _f32(bits)
    codes, scales = oracle_lib.quantize(x, block)
    bc, bs = brute.quantize([Fraction(float(v)) for v in x], block)
    assert list(codes.astype(int)) == bc
    assert [Fraction(float(s)) for s in scales] == bs


@COMMON
@given(st.lists(FINITE_BF16, min_size=1, max_size=24), st.integers(1, 9))
def test_quantize_bf16_any_bits(oracle_lib, bits, block):
    x = np.array(bits, np.uint16)
    codes, scales = oracle_lib.quantize(x, block)
    bc, bs = brute.quantize([brute.bf16_bits_to_fraction(h) for h in x], block)
    assert list(codes.astype(int)) == bc
    assert [Fraction(float(s)) for s in scales] == bs


# scales of a real quantizer are at most FLT_MAX/127; keep every sum finite
SCALE = st.floats(min_value=2.0 ** -140, max_value=float(np.float32(1e30)), allow_nan=False,
                  allow_infinity=False, width=32)


@COMMON
@given(st.integers(1, 5), st.integers(1, 6), st.integers(1, 3), st.data())
def test_reduce_any_codes(oracle_lib, nranks, block, nblocks, data):
    n = block * nblocks - data.draw(st.integers(0, block - 1))
    codes = [np.array(data.draw(st.lists(st.integers(-128, 127), min_size=n, max_size=n)), np.int8)
             for _ in range(nranks)]
    scales = [np.array(data.draw(st.lists(SCALE, min_size=nblocks, max_size=nblocks)), np.float32)
              for _ in range(nranks)]
    oc, os_ = oracle_lib.reduce(codes, scales, block)
    bc, bs = brute.reduce([list(c.astype(int)) for c in codes],
                          [[Fraction(float(v)) for v in s] for s in scales], block)
    assert list(oc.astype(int)) == bc
    assert [Fraction(float(v)) for v in os_] == bs


@COMMON
@given(st.integers(1, 6), st.integers(1, 3), st.data())
def test_ring_step_any_input(oracle_lib, block, nblocks, data):
    n = block * nblocks
    codes = np.array(data.draw(st.lists(st.integers(-128, 127), min_size=n, max_size=n)), np.int8)
    scales = np.array(data.draw(st.lists(SCALE, min_size=nblocks, max_size=nblocks)), np.float32)
    local = np.array(data.draw(st.lists(st.floats(-float(np.float32(1e30)), float(np.float32(1e30)), width=32), min_size=n, max_size=n)), np.float32)
    oc, os_ = oracle_lib.ring_step(codes, scales, local, block)
    bc, bs = brute.ring_step(list(codes.astype(int)), [Fraction(float(v)) for v in scales],
                             [Fraction(float(v)) for v in local], block)
    assert list(oc.astype(int)) == bc
    assert [Fraction(float(v)) for v in os_] == bs


# ----------------------------------------------------------------------------
# FP8 E4M3 codes


def _neg_zero(x) -> list[bool]:
    return [bool(v == 0 and np.signbit(v)) for v in np.asarray(x, np.float32)]


@COMMON
@given(st.lists(FINITE_F32, min_size=1, max_size=24), st.integers(1, 9))
def test_quantize_e4m3_fp32_any_bits(oracle_lib, bits, block):
    x = _f32(bits)
    codes, scales = oracle_lib.quantize_e4m3(x, block)
    bc, bs = brute.quantize_e4m3([Fraction(float(v)) for v in x], block, _neg_zero(x))
    assert list(codes.astype(int)) == bc
    assert [Fraction(float(s)) for s in scales] == bs


@COMMON
@given(st.integers(1, 5), st.integers(1, 6), st.integers(1, 3), st.data())
def test_reduce_e4m3_any_codes(oracle_lib, nranks, block, nblocks, data):
    n = block * nblocks - data.draw(st.integers(0, block - 1))
    finite = st.integers(0, 255).filter(lambda c: c not in (0x7F, 0xFF))
    codes = [np.array(data.draw(st.lists(finite, min_size=n, max_size=n)), np.uint8) for _ in range(nranks)]
    scales = [np.array(data.draw(st.lists(SCALE, min_size=nblocks, max_size=nblocks)), np.float32)
              for _ in range(nranks)]
    oc, os_ = oracle_lib.reduce_e4m3(codes, scales, block)
    bc, bs = brute.reduce_e4m3([list(c.astype(int)) for c in codes],
                               [[Fraction(float(v)) for v in s] for s in scales], block)
    assert list(oc.astype(int)) == bc
    assert [Fraction(float(v)) for v in os_] == bs


# ----------------------------------------------------------------------------
# 4-bit codes


@COMMON
@given(st.lists(FINITE_F32, min_size=1, max_size=24), st.integers(1, 9))
def test_quantize_int4_fp32_any_bits(oracle_lib, bits, block):
    import pins_int4
    x = _f32(bits)
    packed, scales = oracle_lib.quantize_int4(x, block)
    bc, bs = brute.quantize4([Fraction(float(v)) for v in x], block)
    assert list(pins_int4.unpack(packed, x.size).astype(int)) == bc
    assert [Fraction(float(s)) for s in scales] == bs
