"""Exact-rational brute force for tiny inputs: an independent derivation of
every step the oracle takes, used to pin it.

Nothing here uses binary32 arithmetic.  Every value is a ``Fraction``; the
only rounding is ``rn32`` below, written from the definition of IEEE 754
binary32 round-to-nearest-even (24-bit significand, exponents -126..127,
gradual underflow with quantum 2**-149).  Codes are found by searching all
255 admissible codes for the one nearest to the rounded quotient, ties to the
even code, instead of calling a rounding function.

Method: "EQuARX: Efficient Quantized AllReduce in XLA for Distributed Machine
Learning Acceleration", section "technical framework" steps 1-4 and "key
design" item 1 (blocks, a per-block dynamic range, INT8 codes, sum over the
devices, dequantization).
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np

_TWO = Fraction(2)
_P = 24                      # binary32 significand bits
_EMIN = -126                 # smallest normal exponent
_FLT_MAX = (2 - _TWO ** (1 - _P)) * _TWO ** 127
CODES = range(-127, 128)     # the admissible int8 codes (-128 is never emitted)


def rn32(x: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value, ties to even."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while _TWO ** e > a:
        e -= 1
    while _TWO ** (e + 1) <= a:
        e += 1
    e = max(e, _EMIN)                     # below 2**-126 the spacing stays 2**-149
    quantum = _TWO ** (e - (_P - 1))
    m = a / quantum
    whole = m.numerator // m.denominator
    frac = m - whole
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    r = whole * quantum
    if r > _FLT_MAX:
        raise OverflowError("rounds to infinity")
    return sign * r


def rn_bf16(x: Fraction) -> Fraction:
    """Round an exact rational to the nearest bfloat16 value (8-bit
    significand, binary32 exponent range), ties to even."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while _TWO ** e > a:
        e -= 1
    while _TWO ** (e + 1) <= a:
        e += 1
    e = max(e, _EMIN)
    quantum = _TWO ** (e - 7)
    m = a / quantum
    whole = m.numerator // m.denominator
    frac = m - whole
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    return sign * whole * quantum


def reduce_unquantized(ranks: list[list[Fraction]], to_bf16: bool) -> list[Fraction]:
    """Rank-order binary32 sum of exact values, then bf16 rounding if asked."""
    acc = list(ranks[0])
    for r in ranks[1:]:
        acc = [rn32(a + b) for a, b in zip(acc, r)]
    return [rn_bf16(a) for a in acc] if to_bf16 else acc


def to_fraction(v) -> Fraction:
    """Exact value of a Python/numpy float (binary32 or binary64)."""
    return Fraction(float(v))


def bf16_bits_to_fraction(h: int) -> Fraction:
    (f,) = struct.unpack("<f", struct.pack("<I", (int(h) & 0xFFFF) << 16))
    return Fraction(f)


def fraction_to_f32(x: Fraction) -> np.float32:
    """A rational that is already a binary32 value, as np.float32 (checked)."""
    f = np.float32(float(x))
    if Fraction(float(f)) != x:
        raise ValueError("not a binary32 value")
    return f


def nearest_code(t: Fraction) -> int:
    """The code in -127..127 nearest to t; on a tie the even code wins."""
    best = None
    for q in CODES:
        d = abs(t - q)
        if best is None or d < best[0] or (d == best[0] and q % 2 == 0):
            best = (d, q)
    return best[1]


def quantize_block(values: list[Fraction]) -> tuple[list[int], Fraction]:
    """One block of exact values -> (codes, scale)."""
    absmax = max((abs(v) for v in values), default=Fraction(0))
    s = rn32(absmax / 127)
    if s == 0:
        return [0] * len(values), s
    return [nearest_code(rn32(v / s)) for v in values], s


def quantize(values: list[Fraction], block: int) -> tuple[list[int], list[Fraction]]:
    codes, scales = [], []
    for start in range(0, len(values), block):
        c, s = quantize_block(values[start:start + block])
        codes += c
        scales.append(s)
    return codes, scales


def dequantize(codes: list[int], scales: list[Fraction], block: int) -> list[Fraction]:
    return [rn32(q * scales[i // block]) for i, q in enumerate(codes)]


def reduce(rank_codes: list[list[int]], rank_scales: list[list[Fraction]], block: int):
    """Dequantize every rank, add in rank order with one rounding per add,
    quantize the sum."""
    acc = dequantize(rank_codes[0], rank_scales[0], block)
    for c, s in zip(rank_codes[1:], rank_scales[1:]):
        y = dequantize(c, s, block)
        acc = [rn32(a + b) for a, b in zip(acc, y)]
    return quantize(acc, block)


def ring_step(codes: list[int], scales: list[Fraction], local: list[Fraction], block: int):
    y = dequantize(codes, scales, block)
    return quantize([rn32(a + b) for a, b in zip(y, local)], block)
