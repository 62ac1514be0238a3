"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` takes an oracle object (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with:
  - exact-rational brute force (``tests/brute.py``) on tiny inputs,
  - closed forms (power-of-two scales, integer-valued ranks),
  - an independent binary64 route whose double rounding is innocuous
    (S. A. Figueroa, "When is double rounding innocuous?", SIGNUM Newsletter
    30(3), 1995: for +, -, *, / and sqrt of binary32 operands, rounding the
    binary64 result to binary32 equals rounding the exact result, because
    53 >= 2*24 + 2),
  - a library conversion (torch's float32 -> bfloat16, round-to-nearest-even),
  - invariants and error bounds of the method.
``tests/test_oracle_pins.py`` runs them on the oracle;
``tests/test_oracle_mutants.py`` runs them on copies of the oracle with a
planted mistake and checks that some pin fails for every mistake.

Method: "EQuARX: Efficient Quantized AllReduce in XLA for Distributed Machine
Learning Acceleration", section "technical framework" steps 1-4 and "key
design" item 1.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import brute
from block_wise_int8_amd import synth
from oracle import bounds

# ----------------------------------------------------------------------------
# helpers (independent of the oracle's arithmetic)


def all_finite_bf16() -> np.ndarray:
    """Every finite bf16 bit pattern (both signs, zeros, subnormals)."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (h >> 7) & 0xFF
    return h[exp != 0xFF]


def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, np.float32).view(np.uint32)


def expect_codes_via_f64(x64: np.ndarray, s32: np.float32) -> np.ndarray:
    """Codes from the binary64 route: fl32(x/s) as RN32(RN64(x/s))
    (innocuous double rounding), numpy's rint (ties to even), clip."""
    if s32 == 0:
        return np.zeros(x64.size, np.int8)
    t = (x64 / np.float64(s32)).astype(np.float32)
    return np.clip(np.rint(t), -127, 127).astype(np.int8)


def scale_via_f64(absmax64: float) -> np.float32:
    return np.float32(np.float64(absmax64) / 127.0)


def brute_check_quantize(o, x: np.ndarray, block: int, what: str) -> None:
    """Compare oracle.quantize with the exact-rational brute force."""
    codes, scales = o.quantize(x, block)
    if x.dtype == np.uint16:
        vals = [brute.bf16_bits_to_fraction(h) for h in x]
    else:
        vals = [brute.to_fraction(v) for v in x]
    bc, bs = brute.quantize(vals, block)
    assert list(codes.astype(int)) == bc, f"{what}: codes differ from brute force"
    assert [Fraction(float(s)) for s in scales] == bs, f"{what}: scales differ from brute force"


# ----------------------------------------------------------------------------
# scale (per-block absmax -> absmax / 127)


def pin_scale_exact_rational(o) -> None:
    """Every positive finite bf16 absmax: scale == RN32(absmax / 127) by
    exact rationals; a one-element block's code is 127."""
    h = all_finite_bf16()
    h = h[(h > 0) & (h < 0x8000)]
    codes, scales = o.quantize(h, 1)
    for hv, s in zip(h, scales):
        want = brute.rn32(brute.bf16_bits_to_fraction(hv) / 127)
        assert Fraction(float(s)) == want, f"scale of bf16 {hv:#06x}"
    assert np.all(codes == 127), "a lone positive element must get code 127"
    # fp32 absmax across the whole range, subnormal included
    a = np.abs(synth.wide_range_f32(11, 400, 1, log2_span=140)).astype(np.float32)
    a = np.concatenate([a, np.float32([2.0 ** -149, 2.0 ** -140, 1.5e-36, 3.0e38])])
    a = a[np.isfinite(a) & (a > 0)]
    _, scales = o.quantize(a, 1)
    for av, s in zip(a, scales):
        assert Fraction(float(s)) == brute.rn32(Fraction(float(av)) / 127), f"scale of {av!r}"


def pin_scale_closed_form(o) -> None:
    """absmax = 127 * 2**k -> scale = 2**k exactly; then x = j * 2**k has
    code j, and x = (j + 1/2) * 2**k (an exact tie) has the even neighbour."""
    j = np.arange(-127, 128, dtype=np.float64)
    for k in (-126, -100, -60, -20, -7, -1, 0, 1, 5, 20, 60, 100, 120):
        p = 2.0 ** k
        block = np.concatenate([[127.0 * p], j * p, (j[:-1] + 0.5) * p]).astype(np.float32)
        codes, scales = o.quantize(block, block.size)
        assert scales[0] == np.float32(p), f"scale for 127*2**{k}"
        assert list(codes[1:256]) == list(range(-127, 128)), f"integer quotients at 2**{k}"
        ties = j[:-1] + 0.5
        even = np.where(np.floor(ties) % 2 == 0, np.floor(ties), np.ceil(ties))
        assert np.array_equal(codes[256:].astype(np.float64), even), f"ties at 2**{k} not to even"


# ----------------------------------------------------------------------------
# codes


def pin_codes_brute_tiny(o) -> None:
    """Tiny random blocks, every block length 1..16 and a partial last block,
    bf16 and fp32: codes and scales equal the exact-rational brute force."""
    rng = np.random.default_rng(5)
    for block in (1, 2, 3, 5, 8, 16):
        n = 3 * block + (block // 2)
        x = rng.normal(0, 1, n) * np.exp(rng.normal(0, 3, n))
        brute_check_quantize(o, x.astype(np.float32), block, f"fp32 block {block}")
        brute_check_quantize(o, synth.f32_to_bf16_bits(x.astype(np.float32)), block, f"bf16 block {block}")
    # near-tie quotients: x = (j + 1/2) * s nudged by a few ulps
    s_abs = np.float32(3.3)                      # absmax 3.3 gives an inexact scale
    s = np.float32(s_abs / np.float32(127.0))
    base = (np.arange(-20, 20) + 0.5) * np.float64(s)
    near = np.concatenate([np.nextafter(base.astype(np.float32), np.float32(np.inf)),
                           base.astype(np.float32),
                           np.nextafter(base.astype(np.float32), np.float32(-np.inf))])
    brute_check_quantize(o, np.concatenate([[s_abs], near]).astype(np.float32), 121, "near ties")
    # clamp: tiny fp32 absmax whose scale is a rounded subnormal (quotient 128)
    tiny = np.float32([-2.0 ** -140, 2.0 ** -141, 2.0 ** -142, 0.0])
    brute_check_quantize(o, tiny, 4, "subnormal scale clamp")


def pin_codes_exhaustive_bf16(o) -> None:
    """For 48 absmax values spread over the bf16 range: one block holding the
    absmax and every finite bf16 x with |x| <= absmax; codes equal the
    binary64 route."""
    h = all_finite_bf16()
    v = bf16_to_f64(h)
    rng = np.random.default_rng(3)
    pos = h[(h > 0) & (h < 0x7F80)]
    picks = np.concatenate([rng.choice(pos, 40, replace=False),
                            np.uint16([0x0001, 0x0080, 0x3F80, 0x42FE, 0x7F7F, 0x3C01, 0x4300, 0x0400])])
    for a_bits in picks:
        a = bf16_to_f64(np.uint16([a_bits]))[0]
        sel = h[np.abs(v) <= a]
        block = np.concatenate([np.uint16([a_bits]), sel])
        codes, scales = o.quantize(block, block.size)
        s = scale_via_f64(a)
        assert f32_bits(scales[0]) == f32_bits(s), f"scale for absmax {a!r}"
        want = expect_codes_via_f64(bf16_to_f64(block), s)
        bad = np.nonzero(codes != want)[0]
        assert bad.size == 0, f"absmax {a!r}: {bad.size} codes differ, first x={bf16_to_f64(block[bad[:1]])}"


def pin_codes_random_f32(o) -> None:
    """Wide-range fp32 blocks (scales from 2**-60 to 2**60): scales and codes
    equal the binary64 route."""
    for block in (64, 256):
        x = synth.wide_range_f32(21 + block, 1 << 15, block, log2_span=60)
        codes, scales = o.quantize(x, block)
        x64 = x.astype(np.float64).reshape(-1, block)
        amax = np.abs(x64).max(axis=1)
        s = (amax / 127.0).astype(np.float32)
        assert np.array_equal(f32_bits(scales), f32_bits(s)), "scales differ from the binary64 route"
        t = (x64 / s.astype(np.float64)[:, None]).astype(np.float32)
        want = np.clip(np.rint(t), -127, 127).astype(np.int8).reshape(-1)
        assert np.array_equal(codes, want), f"block {block}: codes differ from the binary64 route"


# ----------------------------------------------------------------------------
# dequantize


def pin_dequant_exact(o) -> None:
    """fl32(q * s): q*s is exact in binary64 (<= 8 + 24 bits), so one
    rounding to binary32 is the definition.  bf16 output equals torch's
    round-to-nearest-even conversion of that fp32 value."""
    rng = np.random.default_rng(7)
    block = 32
    nb = 4096
    codes = rng.integers(-128, 128, nb * block).astype(np.int8)
    scales = np.abs(synth.wide_range_f32(8, nb, 1, log2_span=110)).astype(np.float32)
    scales[:8] = np.float32([0.0, 2.0 ** -149, 2.0 ** -130, 1.0, 1 / 127, 2.0 ** 110, 1.0e36, 2.6e36])
    out = o.dequantize(codes, scales, block, "f32")
    want = (codes.astype(np.float64) * np.repeat(scales.astype(np.float64), block)).astype(np.float32)
    assert np.array_equal(f32_bits(out), f32_bits(want)), "fp32 dequantize is not RN32(q*s)"
    out16 = o.dequantize(codes, scales, block, "bf16")
    assert np.array_equal(out16, synth.f32_to_bf16_bits(want)), "bf16 dequantize != RNE(fp32 value)"


def pin_bf16_rounding(o) -> None:
    """The fp32 -> bf16 rounding agrees with torch on ties, carries into the
    exponent, subnormals and values that round past the largest bf16."""
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32)
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]
    hi = rng.integers(0, 1 << 16, 4000, dtype=np.uint64).astype(np.uint32) << 16
    ties = hi | 0x8000
    ties = ties[((ties >> 23) & 0xFF) != 0xFF]
    special = np.uint32([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x3F80FFFF, 0x00008000, 0x00018000,
                         0x80008000, 0x3FFF8000, 0x3FFE8000])
    f = np.concatenate([bits, ties, special]).view(np.float32)
    assert np.array_equal(o.f32_to_bf16(f), synth.f32_to_bf16_bits(f)), "bf16 rounding differs from torch"


# ----------------------------------------------------------------------------
# quantize invariants


def pin_roundtrip_bound(o) -> None:
    """|x - dequantize(quantize(x))| <= s/2 + 2**-22 |x| for every element."""
    for x, block in ((synth.wide_range_f32(31, 1 << 16, 64, 100), 64),
                     (synth.uniform_f32(32, 1, 1 << 16)[0], 256),
                     (synth.uniform_bf16(33, 1, 1 << 16, 20.0)[0], 128)):
        codes, scales = o.quantize(x, block)
        y = o.dequantize(codes, scales, block, "f32").astype(np.float64)
        x64 = bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
        b = bounds.requant_bound(np.abs(x64), bounds.per_element(scales, block, x64.size))
        assert np.all(np.abs(x64 - y) <= b), "round trip exceeds s/2 + 2**-22 |x|"


def pin_constant_block(o) -> None:
    """A block of equal bf16 values +-c gets codes +-127 and dequantizes to
    exactly c in bf16, for every positive finite bf16 c."""
    h = all_finite_bf16()
    h = h[(h > 0) & (h < 0x8000)]
    x = np.repeat(h, 4).copy()
    x[1::4] |= 0x8000                      # one negative copy per block
    codes, scales = o.quantize(x, 4)
    want = np.tile(np.int8([127, -127, 127, 127]), h.size)
    assert np.array_equal(codes, want), "constant block codes must be +-127"
    back = o.dequantize(codes, scales, 4, "bf16")
    assert np.array_equal(back, x), "constant bf16 block does not round-trip"


def pin_zero_and_signed_zero(o) -> None:
    """All-zero block: scale +0.0 and codes 0; -0.0 inside a non-zero block
    is code 0 and dequantizes to +0.0; an fp32 block whose scale underflows
    to 0 (absmax 2**-149) gets all-zero codes."""
    x = np.float32([0.0, -0.0, 0.0, 0.0, -0.0, 1.0, 0.0, -3.0, 2.0 ** -149, -2.0 ** -149, 0.0, 0.0])
    codes, scales = o.quantize(x, 4)
    assert f32_bits(scales[0]) == 0, "all-zero block scale must be +0.0"
    assert np.all(codes[:4] == 0)
    assert codes[4] == 0 and codes[6] == 0
    assert f32_bits(scales[2]) == 0 and np.all(codes[8:] == 0), "underflowed scale must give zero codes"
    y = o.dequantize(codes, scales, 4, "f32")
    assert f32_bits(y[4]) == 0, "-0.0 must dequantize to +0.0"
    hb = np.uint16([0x8000, 0x8000, 0x0000, 0x8000])
    codes, scales = o.quantize(hb, 4)
    assert np.all(codes == 0) and f32_bits(scales[0]) == 0


def pin_permutation(o) -> None:
    """absmax is order-independent: permuting a block keeps its scale bit for
    bit and permutes its codes the same way."""
    rng = np.random.default_rng(13)
    block = 64
    x = synth.wide_range_f32(14, 64 * block, block, 30)
    perm = np.concatenate([rng.permutation(block) + b * block for b in range(64)])
    c1, s1 = o.quantize(x, block)
    c2, s2 = o.quantize(x[perm], block)
    assert np.array_equal(f32_bits(s1), f32_bits(s2)), "scale depends on element order"
    assert np.array_equal(c1[perm], c2), "codes do not follow the permutation"


def pin_block_layout(o) -> None:
    """Block b covers elements [b*B, (b+1)*B): quantizing the whole buffer
    equals quantizing each block alone (blocks of very different
    magnitudes), and a partial last block is quantized on its own elements."""
    block = 16
    x = synth.wide_range_f32(15, 10 * block + 5, block, 40)
    codes, scales = o.quantize(x, block)
    assert scales.size == 11
    for b in range(11):
        part = x[b * block:(b + 1) * block]
        c, s = o.quantize(part, part.size)
        assert f32_bits(s[0]) == f32_bits(scales[b]), f"scale of block {b}"
        assert np.array_equal(c, codes[b * block:(b + 1) * block]), f"codes of block {b}"


def pin_idempotence(o) -> None:
    """quantize(dequantize(quantize(x))) == quantize(x) (observed property;
    not proven)."""
    for x, block in ((synth.uniform_bf16(41, 1, 1 << 16)[0], 256),
                     (synth.wide_range_f32(42, 1 << 16, 64, 40), 64)):
        c, s = o.quantize(x, block)
        c2, s2 = o.quantize(o.dequantize(c, s, block, "f32"), block)
        assert np.array_equal(c, c2) and np.array_equal(f32_bits(s), f32_bits(s2)), "not idempotent"


def pin_nonfinite_rejected(o) -> None:
    """Non-finite input, and a reduce or ring step whose binary32 sum
    overflows (two values of 3e38), are refused."""
    for bad in (np.inf, -np.inf, np.nan):
        x = np.float32([1.0, bad, 2.0, 3.0])
        try:
            o.quantize(x, 4)
        except ValueError:
            continue
        raise AssertionError("non-finite input accepted")
    c, s = o.quantize(np.float32([3.0e38, 1.0]), 2)
    for call in (lambda: o.reduce([c, c], [s, s], 2),
                 lambda: o.ring_step(c, s, np.float32([3.0e38, 0.0]), 2)):
        try:
            call()
        except ValueError:
            continue
        raise AssertionError("overflowing sum accepted")


# ----------------------------------------------------------------------------
# reduce


def _quantized_ranks(o, xs, block):
    qs = [o.quantize(x, block) for x in xs]
    return [q[0] for q in qs], [q[1] for q in qs]


def pin_reduce_brute_tiny(o) -> None:
    """Tiny reduces (N = 1, 2, 3, 5; several block lengths; a partial last
    block) equal the exact-rational brute force."""
    rng = np.random.default_rng(17)
    for nr, block, n in ((1, 4, 10), (2, 8, 20), (3, 5, 17), (5, 8, 24), (4, 1, 6)):
        codes = [rng.integers(-128, 128, n).astype(np.int8) for _ in range(nr)]
        nb = -(-n // block)
        scales = [np.abs(rng.normal(0, 1, nb) * np.exp(rng.normal(0, 4, nb))).astype(np.float32)
                  for _ in range(nr)]
        oc, os_ = o.reduce(codes, scales, block)
        bc, bs = brute.reduce([list(c.astype(int)) for c in codes],
                              [[Fraction(float(v)) for v in s] for s in scales], block)
        assert list(oc.astype(int)) == bc, f"reduce codes differ from brute force (N={nr}, B={block})"
        assert [Fraction(float(v)) for v in os_] == bs, f"reduce scales differ (N={nr}, B={block})"


def pin_reduce_rank_order(o) -> None:
    """fp32 addition is not associative.  Ranks 0 and 1 hold 1 (scale 1),
    rank 2 holds 127*2**18 (scale 2**18).  In rank order (1 + 1) + 127*2**18
    is exact; any order that adds the big term first loses both ones to ties
    to even.  The brute force, which adds in rank order, decides."""
    big = 127.0 * 2.0 ** 18
    xs = [np.float32([1.0, 127.0]), np.float32([1.0, 127.0]), np.float32([big, 0.0])]
    codes, scales = _quantized_ranks(o, xs, 2)
    oc, os_ = o.reduce(codes, scales, 2)
    bc, bs = brute.reduce([list(c.astype(int)) for c in codes],
                          [[Fraction(float(v)) for v in s] for s in scales], 2)
    assert list(oc.astype(int)) == bc and [Fraction(float(v)) for v in os_] == bs, "rank order"
    want = np.float32(np.float64(big + 2.0) / 127.0)      # Figueroa: innocuous double rounding
    assert os_[0] == want, "sum must be (1 + 1) + 127*2**18"


def pin_reduce_integer_textbook(o) -> None:
    """Integer-valued ranks with per-block absmax 127 have scale 1 and codes
    equal to their values; if the integer sum has absmax exactly 127 the
    reduce returns scale 1 and codes equal to the exact integer sum."""
    rng = np.random.default_rng(19)
    for nr, block in ((2, 8), (4, 16), (8, 64), (16, 32)):
        nb = 6
        k = 126 // nr
        vals = rng.integers(-k, k + 1, (nr, nb, block))
        for b in range(nb):
            for r in range(nr):
                vals[r, b, 0] = 127 if r % 2 == 0 else -127
            vals[1:, b, 1] = np.abs(vals[1:, b, 1])
            vals[0, b, 1] = 127 - vals[1:, b, 1].sum()
        total = vals.sum(axis=0)
        assert np.abs(total).max() <= 127
        xs = [vals[r].reshape(-1).astype(np.float32) for r in range(nr)]
        codes, scales = _quantized_ranks(o, xs, block)
        for r in range(nr):
            assert np.all(scales[r] == 1.0) and np.array_equal(codes[r], xs[r].astype(np.int8))
        oc, os_ = o.reduce(codes, scales, block)
        assert np.all(os_ == 1.0), f"N={nr}: output scale must be 1"
        assert np.array_equal(oc.astype(np.int64), total.reshape(-1)), f"N={nr}: codes != integer sum"


def pin_reduce_composition(o) -> None:
    """reduce == quantize(((y_0 + y_1) + ...) + y_{N-1}) with y_r the
    oracle's fp32 dequantization and the adds done by numpy in binary32."""
    for nr, block in ((4, 128), (8, 256), (16, 64)):
        xs = synth.uniform_bf16(50 + nr, nr, 8 * block + block, 3.0)
        codes, scales = _quantized_ranks(o, xs, block)
        acc = o.dequantize(codes[0], scales[0], block, "f32")
        for c, s in zip(codes[1:], scales[1:]):
            acc = (acc + o.dequantize(c, s, block, "f32")).astype(np.float32)
        wc, ws = o.quantize(acc, block)
        oc, os_ = o.reduce(codes, scales, block)
        assert np.array_equal(oc, wc) and np.array_equal(f32_bits(os_), f32_bits(ws)), f"composition N={nr}"


def pin_reduce_single_rank(o) -> None:
    """N = 1: the reduce requantizes its input, which gives it back."""
    x = synth.uniform_bf16(61, 1, 4096)[0]
    c, s = o.quantize(x, 128)
    oc, os_ = o.reduce([c], [s], 128)
    assert np.array_equal(oc, c) and np.array_equal(f32_bits(os_), f32_bits(s))


def pin_reduce_bound(o) -> None:
    """The dequantized reduce is within bound (3) of the exact sum on the
    outlier recipe (small instance), and within N*max_scale/2 +
    1e-6*|sum| there."""
    w = synth.WORKLOADS["outliers"].resized(n=1 << 17)
    xs = synth.ranks(w)
    codes, scales = _quantized_ranks(o, xs, w.block)
    oc, os_ = o.reduce(codes, scales, w.block)
    out = o.dequantize(oc, os_, w.block, "f32").astype(np.float64)
    x64 = [bf16_to_f64(x) for x in xs]
    exact = np.sum(x64, axis=0)
    ys = [o.dequantize(c, s, w.block, "f32") for c, s in zip(codes, scales)]
    err = np.abs(out - exact)
    assert np.all(err <= bounds.oneshot_bound(x64, scales, ys, os_, w.block)), "bound (3) violated"
    assert np.all(err <= bounds.oneshot_bound_simple(scales, os_, exact, w.block)), "simple bound violated"


# ----------------------------------------------------------------------------
# ring step


def pin_ring_brute_tiny(o) -> None:
    rng = np.random.default_rng(23)
    for block, n, kind in ((4, 10, "f32"), (8, 24, "bf16"), (3, 7, "f32")):
        nb = -(-n // block)
        codes = rng.integers(-128, 128, n).astype(np.int8)
        scales = np.abs(rng.normal(0, 1, nb) * np.exp(rng.normal(0, 3, nb))).astype(np.float32)
        local32 = (rng.normal(0, 1, n) * np.exp(rng.normal(0, 3, n))).astype(np.float32)
        local = synth.f32_to_bf16_bits(local32) if kind == "bf16" else local32
        oc, os_ = o.ring_step(codes, scales, local, block)
        lv = ([brute.bf16_bits_to_fraction(h) for h in local] if kind == "bf16"
              else [Fraction(float(v)) for v in local])
        bc, bs = brute.ring_step(list(codes.astype(int)), [Fraction(float(v)) for v in scales], lv, block)
        assert list(oc.astype(int)) == bc, f"ring codes differ from brute force ({kind}, B={block})"
        assert [Fraction(float(v)) for v in os_] == bs, f"ring scales differ ({kind}, B={block})"


def pin_ring_bound(o) -> None:
    """Ring reduction on the ring recipe (small instance): after every step
    the dequantized partial result is within bound (4) of the exact partial
    sum, and within sum_j s_j/2 + 1e-6*|sum|."""
    w = synth.WORKLOADS["ring"].resized(rows=32)
    xs = synth.ranks(w)
    x64 = [bf16_to_f64(x) for x in xs]
    c, s = o.quantize(xs[0], w.block)
    step_scales, step_values = [s], [x64[0]]
    exact = x64[0].copy()
    for k in range(1, w.nranks):
        p = (o.dequantize(c, s, w.block, "f32") + bf16_to_f64(xs[k]).astype(np.float32)).astype(np.float32)
        c, s = o.ring_step(c, s, xs[k], w.block)
        step_scales.append(s)
        step_values.append(p)
        exact = exact + x64[k]
        out = o.dequantize(c, s, w.block, "f32").astype(np.float64)
        err = np.abs(out - exact)
        assert np.all(err <= bounds.ring_bound(step_scales, step_values, w.block)), f"bound (4) step {k}"
        assert np.all(err <= bounds.ring_bound_simple(step_scales, exact, w.block)), f"simple ring bound step {k}"


# ----------------------------------------------------------------------------
# unquantized comparator


def pin_reduce_unquantized(o) -> None:
    """The unquantized reduce equals the exact-rational brute force (rank
    order, one binary32 rounding per add, bf16 rounding of the sum), keeps
    rank order ((1 + 1) + 2**25 vs 2**25 + 1 + 1), and sums integers
    exactly."""
    rng = np.random.default_rng(29)
    for nr, kind in ((1, "bf16"), (2, "f32"), (3, "bf16"), (5, "f32"), (8, "bf16")):
        v = (rng.normal(0, 1, (nr, 40)) * np.exp(rng.normal(0, 4, (nr, 40)))).astype(np.float32)
        xs = [synth.f32_to_bf16_bits(r) if kind == "bf16" else r for r in v]
        got = o.reduce_unquantized(xs)
        fr = [[brute.bf16_bits_to_fraction(h) for h in x] if kind == "bf16" else [Fraction(float(t)) for t in x]
              for x in xs]
        want = brute.reduce_unquantized(fr, kind == "bf16")
        got_fr = [brute.bf16_bits_to_fraction(h) for h in got] if kind == "bf16" else [Fraction(float(t)) for t in got]
        assert got_fr == want, f"unquantized reduce differs from brute force (N={nr}, {kind})"
    big = np.float32([1.0, 1.0, 2.0 ** 25])
    xs = [np.float32([b]) for b in big]
    assert o.reduce_unquantized(xs)[0] == np.float32(2.0 ** 25 + 2.0), "rank order"
    ints = [np.arange(-50, 50, dtype=np.float32) * (r + 1) for r in range(6)]
    assert np.array_equal(o.reduce_unquantized(ints), np.arange(-50, 50, dtype=np.float32) * 21)


ALL_PINS = [
    pin_scale_closed_form,
    pin_zero_and_signed_zero,
    pin_codes_brute_tiny,
    pin_reduce_integer_textbook,
    pin_reduce_brute_tiny,
    pin_reduce_rank_order,
    pin_ring_brute_tiny,
    pin_reduce_unquantized,
    pin_dequant_exact,
    pin_bf16_rounding,
    pin_block_layout,
    pin_permutation,
    pin_constant_block,
    pin_codes_random_f32,
    pin_codes_exhaustive_bf16,
    pin_scale_exact_rational,
    pin_roundtrip_bound,
    pin_idempotence,
    pin_nonfinite_rejected,
    pin_reduce_composition,
    pin_reduce_single_rank,
    pin_reduce_bound,
    pin_ring_bound,
]
