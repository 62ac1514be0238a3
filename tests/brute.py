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


# ---------------------------------------------------------------------------
# FP8 E4M3 codes (the TACO page, sections 2.A "Waarom FP8?" and 2.B item 2
# "Dual-Scale (DS) Quantization"; format from the OCP 8-bit floating point
# specification).
# Every finite E4M3 value is listed from the format's fields; the nearest one
# is found by scanning the whole list, ties to the code with an even
# mantissa.

E4M3_QMAX = Fraction(448)


def e4m3_exact(code: int) -> Fraction | None:
    """Exact value of an E4M3 byte; None for the two NaN codes."""
    code = int(code)
    sign = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        return sign * Fraction(m, 8) * _TWO ** -6
    return sign * (1 + Fraction(m, 8)) * _TWO ** (e - 7)


E4M3_FINITE = [(c, e4m3_exact(c)) for c in range(256) if e4m3_exact(c) is not None]


def e4m3_nearest_code(t: Fraction, negative: bool) -> int:
    """The E4M3 code nearest to t (|t| <= 448); ties to the even mantissa.
    A result of zero takes the sign of the quotient (`negative`), which t
    alone cannot carry once it has rounded to 0."""
    best = None
    for c, v in E4M3_FINITE:
        d = abs(t - v)
        key = (d, c & 1)                              # smaller distance, then even mantissa
        if best is None or key < best[0]:
            best = (key, c)
    c = best[1]
    if e4m3_exact(c) == 0:
        c = 0x80 if negative else 0x00
    return c


def quantize_block_e4m3(values: list[Fraction], signs: list[bool] | None = None):
    """One block of exact values -> (E4M3 codes, scale).  signs[i] marks an
    input that is a negative zero."""
    absmax = max((abs(v) for v in values), default=Fraction(0))
    s = rn32(absmax / E4M3_QMAX)
    if s == 0:
        return [0x00] * len(values), s
    out = []
    for i, v in enumerate(values):
        t = rn32(v / s)
        t = max(-E4M3_QMAX, min(E4M3_QMAX, t))
        out.append(e4m3_nearest_code(t, v < 0 or (v == 0 and bool(signs and signs[i]))))
    return out, s


def quantize_e4m3(values: list[Fraction], block: int, signs: list[bool] | None = None):
    codes, scales = [], []
    for start in range(0, len(values), block):
        c, s = quantize_block_e4m3(values[start:start + block], signs[start:start + block] if signs else None)
        codes += c
        scales.append(s)
    return codes, scales


def dequantize_e4m3(codes: list[int], scales: list[Fraction], block: int) -> list[Fraction]:
    return [rn32(e4m3_exact(c) * scales[i // block]) for i, c in enumerate(codes)]


def _neg_zero_flags(codes: list[int], scales: list[Fraction], block: int) -> list[bool]:
    """Which dequantized values are -0 in binary32: a -0 code times a
    positive scale (a zero scale only comes with +0 codes)."""
    return [c == 0x80 and scales[i // block] > 0 for i, c in enumerate(codes)]


def reduce_e4m3(rank_codes: list[list[int]], rank_scales: list[list[Fraction]], block: int):
    """Dequantize every rank, add in rank order (one rounding per add),
    quantize the sum.  A binary32 sum is -0 only when both addends are -0."""
    acc = dequantize_e4m3(rank_codes[0], rank_scales[0], block)
    neg = _neg_zero_flags(rank_codes[0], rank_scales[0], block)
    for c, s in zip(rank_codes[1:], rank_scales[1:]):
        y = dequantize_e4m3(c, s, block)
        ny = _neg_zero_flags(c, s, block)
        new = [rn32(a + b) for a, b in zip(acc, y)]
        neg = [n == 0 and a == 0 and b == 0 and na and nb
               for n, a, b, na, nb in zip(new, acc, y, neg, ny)]
        acc = new
    return quantize_e4m3(acc, block, neg)


def ring_step_e4m3(codes: list[int], scales: list[Fraction], local: list[Fraction],
                   local_neg_zero: list[bool], block: int):
    y = dequantize_e4m3(codes, scales, block)
    ny = _neg_zero_flags(codes, scales, block)
    acc = [rn32(a + b) for a, b in zip(y, local)]
    neg = [v == 0 and a == 0 and b == 0 and na and nb
           for v, a, b, na, nb in zip(acc, y, local, ny, local_neg_zero)]
    return quantize_e4m3(acc, block, neg)


# ---------------------------------------------------------------------------
# 4-bit integer codes: the int8 rules with 7 in place of 127 (codes -7..7).

CODES4 = range(-7, 8)


def nearest_code4(t: Fraction) -> int:
    best = None
    for q in CODES4:
        d = abs(t - q)
        if best is None or d < best[0] or (d == best[0] and q % 2 == 0):
            best = (d, q)
    return best[1]


def quantize4(values: list[Fraction], block: int) -> tuple[list[int], list[Fraction]]:
    """-> (codes -7..7 per element, scales); packing is the caller's."""
    codes, scales = [], []
    for start in range(0, len(values), block):
        blk = values[start:start + block]
        absmax = max((abs(v) for v in blk), default=Fraction(0))
        s = rn32(absmax / 7)
        codes += [0] * len(blk) if s == 0 else [nearest_code4(rn32(v / s)) for v in blk]
        scales.append(s)
    return codes, scales


def reduce4(rank_codes: list[list[int]], rank_scales: list[list[Fraction]], block: int):
    acc = [rn32(q * rank_scales[0][i // block]) for i, q in enumerate(rank_codes[0])]
    for c, s in zip(rank_codes[1:], rank_scales[1:]):
        acc = [rn32(a + rn32(q * s[i // block])) for i, (a, q) in enumerate(zip(acc, c))]
    return quantize4(acc, block)


def ring_step4(codes: list[int], scales: list[Fraction], local: list[Fraction], block: int):
    acc = [rn32(rn32(q * scales[i // block]) + x) for i, (q, x) in enumerate(zip(codes, local))]
    return quantize4(acc, block)
