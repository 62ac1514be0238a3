"""Pins of the CPU oracle's FP8 E4M3 variant to things other than itself.

Each ``pin_*`` takes an oracle object and raises AssertionError when the
oracle disagrees with:
  - torch's float8_e4m3fn conversions (a library implementation of the OCP
    E4M3 format: decode of all 256 codes, round-to-nearest-even encode),
  - the exact-rational brute force of ``tests/brute.py`` on tiny inputs,
  - closed forms and invariants (the block's absmax maps to 448, sign
    symmetry, power-of-two scaling, zero blocks),
  - the error bounds (1e) of ``oracle/bounds.py``.

Method: "TACO: Efficient Communication Compression of Intermediate Tensors
for Scalable Tensor-Parallel LLM Training" (page summary, in Dutch), sections
2.A "Waarom FP8?" (why FP8: E4M3 codes) and 2.B item 2 "Dual-Scale (DS)
Quantization" (a per-block scale that brings the block into FP8's range
Q_max), applied to
the block-wise quantized reduce of "EQuARX: Efficient Quantized AllReduce in
XLA ...", section "technical framework" steps 1-4.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

import brute
from block_wise_int8_amd import synth
from oracle import bounds

_NAN_CODES = (0x7F, 0xFF)


def torch_decode(c: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(c, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def torch_encode(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bits(a) -> np.ndarray:
    return np.asarray(a, np.float32).view(np.uint32)


def _frac_list(x: np.ndarray) -> tuple[list[Fraction], list[bool]]:
    """Exact values of bf16 patterns or float32 values, and their -0 flags."""
    if x.dtype == np.uint16:
        f = (x.astype(np.uint32) << 16).view(np.float32)
    else:
        f = x.astype(np.float32)
    return [Fraction(float(v)) for v in f], [bool(v == 0 and np.signbit(v)) for v in f]


def brute_check_quantize(o, x: np.ndarray, block: int, what: str) -> None:
    codes, scales = o.quantize_e4m3(x, block)
    vals, neg = _frac_list(x)
    bc, bs = brute.quantize_e4m3(vals, block, neg)
    assert list(codes.astype(int)) == bc, f"{what}: E4M3 codes differ from brute force"
    assert [Fraction(float(s)) for s in scales] == bs, f"{what}: scales differ from brute force"


# ----------------------------------------------------------------------------
# the format


def pin_e4m3_decode(o) -> None:
    """All 256 codes decode as torch's float8_e4m3fn does (bit for bit; the
    two NaN codes to NaN), and a few values read off the format's fields."""
    c = np.arange(256, dtype=np.uint8)
    got, want = o.e4m3_decode(c), torch_decode(c)
    fin = ~np.isin(c, _NAN_CODES)
    assert np.all(np.isnan(got[~fin])), "codes 0x7f/0xff must decode to NaN"
    assert np.array_equal(_bits(got[fin]), _bits(want[fin])), "E4M3 decode differs from torch"
    for code, v in ((0x7E, 448.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
                    (0x38, 1.0), (0x3F, 1.875), (0xFE, -448.0)):
        assert got[code] == np.float32(v), f"E4M3 code {code:#04x}"
    assert _bits(got[0x80]) == 0x80000000, "0x80 is -0"
    assert np.all(np.diff(got[:127].astype(np.float64)) > 0), "codes 0..126 must increase"


def pin_e4m3_encode_torch(o) -> None:
    """Every finite bf16 value within [-448, 448], every midpoint between
    neighbouring E4M3 values and the float32 values next to it, and random
    float32 across the range: the oracle's code equals torch's
    round-to-nearest-even conversion."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (h.astype(np.uint32) << 16).view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) <= 448.0)]
    v = torch_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)              # exact in binary32
    near = np.concatenate([mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))])
    near = near[np.abs(near) <= 448.0]
    rng = np.random.default_rng(41)
    r = (rng.uniform(-1, 1, 200000) * np.exp2(rng.uniform(-30, 8.8, 200000))).astype(np.float32)
    r = r[np.abs(r) <= 448.0]
    x = np.concatenate([f, near, -near, r, np.float32([0.0, -0.0, 2.0 ** -149, -2.0 ** -149])])
    assert np.array_equal(o.e4m3_encode(x), torch_encode(x)), "E4M3 encode differs from torch"


def pin_e4m3_encode_brute(o) -> None:
    """A sample of values: the oracle's code equals the nearest of all 254
    finite E4M3 values, found by exact rationals, ties to the even mantissa."""
    rng = np.random.default_rng(43)
    x = (rng.uniform(-1, 1, 400) * np.exp2(rng.uniform(-12, 8.8, 400))).astype(np.float32)
    x = np.concatenate([x[np.abs(x) <= 448.0], np.float32([2.0 ** -10, -2.0 ** -10, 3 * 2.0 ** -11, 448.0,
                                                           -0.0, 0.0, 240.0, 232.0, 248.0])])
    got = o.e4m3_encode(x)
    for v, c in zip(x, got):
        want = brute.e4m3_nearest_code(Fraction(float(v)), bool(np.signbit(v)))
        assert int(c) == want, f"E4M3 code of {v!r}: {int(c):#04x}, want {want:#04x}"


# ----------------------------------------------------------------------------
# quantize


def pin_e4m3_quantize_brute_tiny(o) -> None:
    """Tiny random blocks of every length 1..16 with a partial last block,
    bf16 and fp32, signed zeros, and blocks whose scale is a rounded
    subnormal (the clamp to 448 binds): codes and scales equal the brute
    force."""
    rng = np.random.default_rng(47)
    for block in (1, 2, 3, 5, 8, 16):
        n = 3 * block + (block // 2)
        x = rng.normal(0, 1, n) * np.exp(rng.normal(0, 3, n))
        x[::7] = -0.0
        brute_check_quantize(o, x.astype(np.float32), block, f"fp32 block {block}")
        brute_check_quantize(o, synth.f32_to_bf16_bits(x.astype(np.float32)), block, f"bf16 block {block}")
    tiny = np.float32([-2.0 ** -140, 2.0 ** -141, 3 * 2.0 ** -143, -0.0, 2.0 ** -149, -2.0 ** -148])
    brute_check_quantize(o, tiny, 6, "subnormal scale")
    brute_check_quantize(o, np.float32([1e-30, -1e-36, 1e-38, 3e-39]), 4, "small scale")


def pin_e4m3_absmax_code(o) -> None:
    """With a normal scale the block's largest magnitude maps to +-448
    (code 0x7e / 0xfe): fl32(a / fl32(a/448)) lies within a few ulps of 448,
    and the neighbours of 448 are 416 and none."""
    rng = np.random.default_rng(53)
    x = (rng.normal(0, 1, 64 * 300) * np.repeat(np.exp2(rng.uniform(-100, 100, 300)), 64)).astype(np.float32)
    codes, _ = o.quantize_e4m3(x, 64)
    for b in range(300):
        blk = x[64 * b:64 * b + 64]
        i = int(np.argmax(np.abs(blk)))
        assert codes[64 * b + i] == (0xFE if blk[i] < 0 else 0x7E), f"block {b}: absmax code"


def pin_e4m3_sign_and_scaling(o) -> None:
    """quantize(-x) flips every code's sign bit and keeps the scales;
    quantize(2^k x) keeps the codes and multiplies the scales by 2^k while
    the scales stay normal."""
    rng = np.random.default_rng(59)
    x = (rng.normal(0, 1, 4096) * np.exp(rng.normal(0, 2, 4096))).astype(np.float32)
    c, s = o.quantize_e4m3(x, 128)
    cn, sn = o.quantize_e4m3(-x, 128)
    assert np.array_equal(cn, c ^ np.uint8(0x80)) and np.array_equal(sn, s), "sign symmetry"
    for k in (-60, -9, 1, 7, 50):
        ck, sk = o.quantize_e4m3((x * np.float32(2.0 ** k)).astype(np.float32), 128)
        assert np.array_equal(ck, c), f"codes change under scaling by 2**{k}"
        assert np.array_equal(sk, (s * np.float32(2.0 ** k)).astype(np.float32)), f"scales under 2**{k}"


def pin_e4m3_zero_blocks(o) -> None:
    """A block of zeros (either sign) gets scale 0 and codes 0x00; its
    values dequantize to +0."""
    x = np.float32([0.0, -0.0, -0.0, 0.0, 1.0, -0.0, 2.0, 0.0])
    c, s = o.quantize_e4m3(x, 4)
    assert s[0] == 0 and not np.signbit(s[0]) and list(c[:4]) == [0, 0, 0, 0], "zero block"
    assert list(c[4:]) == [0x76, 0x80, 0x7E, 0x00], "1, -0, 2, 0 with scale 2/448 (1 -> 224 = 1.75 * 2^7)"
    y = o.dequantize_e4m3(c, s, 4)
    assert np.array_equal(_bits(y), _bits(np.float32([0, 0, 0, 0, 1.0, -0.0, 2.0, 0]))), "dequantized"


def pin_e4m3_dequant(o) -> None:
    """dequantize = float32 product of torch's decoded code and the scale
    (numpy's float32 multiply), then bf16 by torch's conversion."""
    rng = np.random.default_rng(61)
    codes = rng.integers(0, 256, 4096).astype(np.uint8)
    codes[np.isin(codes, _NAN_CODES)] = 0x11
    scales = (np.exp2(rng.uniform(-140, 120, 32))).astype(np.float32)
    want = (torch_decode(codes) * np.repeat(scales, 128)).astype(np.float32)
    got = o.dequantize_e4m3(codes, scales, 128, "f32")
    assert np.array_equal(_bits(got), _bits(want)), "E4M3 dequantize f32"
    gb = o.dequantize_e4m3(codes, scales, 128, "bf16")
    wb = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    fin = np.isfinite(want)
    assert np.array_equal(gb[fin], wb[fin]), "E4M3 dequantize bf16"


def pin_e4m3_roundtrip_bound(o) -> None:
    """|x - dequantize(quantize(x))| <= (1e) on wide-range data."""
    x = synth.wide_range_f32(67, 64 * 512, 64, log2_span=100)
    c, s = o.quantize_e4m3(x, 64)
    y = o.dequantize_e4m3(c, s, 64).astype(np.float64)
    err = np.abs(y - x.astype(np.float64))
    bnd = bounds.requant_bound_e4m3(np.abs(x.astype(np.float64)), bounds.per_element(s, 64, x.size))
    assert np.all(err <= bnd), f"round trip exceeds (1e): worst {np.max(err / bnd)}"


def pin_e4m3_nonfinite_rejected(o) -> None:
    for bad in (np.inf, -np.inf, np.nan):
        x = np.float32([1.0, bad, 2.0, 3.0])
        try:
            o.quantize_e4m3(x, 4)
        except ValueError:
            continue
        raise AssertionError(f"quantize_e4m3 accepted {bad}")


# ----------------------------------------------------------------------------
# reduce and ring


def _ranks(o, xs, block):
    qs = [o.quantize_e4m3(x, block) for x in xs]
    return [q[0] for q in qs], [q[1] for q in qs]


def pin_e4m3_reduce_brute_tiny(o) -> None:
    """N = 1..5 tiny ranks with cancellations and signed zeros: the reduce
    equals the brute force (rank-order binary32 sum of the exact dequantized
    values, then quantize)."""
    rng = np.random.default_rng(71)
    for nranks, block, n in ((1, 4, 8), (2, 3, 10), (3, 8, 24), (5, 5, 23)):
        xs = [(rng.normal(0, 1, n) * np.exp(rng.normal(0, 3, n))).astype(np.float32) for _ in range(nranks)]
        if nranks > 1:
            xs[1][:3] = -xs[0][:3]                   # exact cancellations
            xs[0][3] = xs[1][3] = -0.0
        codes, scales = _ranks(o, xs, block)
        oc, os_ = o.reduce_e4m3(codes, scales, block)
        bc, bs = brute.reduce_e4m3([list(c.astype(int)) for c in codes],
                                   [[Fraction(float(v)) for v in s] for s in scales], block)
        assert list(oc.astype(int)) == bc, f"N={nranks}: reduce codes differ from brute force"
        assert [Fraction(float(v)) for v in os_] == bs, f"N={nranks}: reduce scales differ"


def pin_e4m3_reduce_order_and_single(o) -> None:
    """N = 1 is quantize(dequantize(.)) of the one rank; for N = 5 the
    oracle's result equals the brute force taken in rank order, which
    differs from the reversed order on these inputs."""
    rng = np.random.default_rng(73)
    x = (rng.normal(0, 1, 256) * np.exp(rng.normal(0, 4, 256))).astype(np.float32)
    c, s = o.quantize_e4m3(x, 32)
    rc, rs = o.reduce_e4m3([c], [s], 32)
    c2, s2 = o.quantize_e4m3(o.dequantize_e4m3(c, s, 32), 32)
    assert np.array_equal(rc, c2) and np.array_equal(rs, s2), "N=1 reduce"
    # rank 0 adds L = 448 * 2^20 (dequantized exactly) and rank 3 takes it
    # away: in rank order ranks 1-2 are rounded at L's spacing (32) and rank
    # 4 is added exactly; in reverse order rank 4 is the one rounded
    big = np.full(64, 448.0 * 2.0 ** 20, np.float32)
    mid = [(rng.normal(0, 100, 64)).astype(np.float32) for _ in range(3)]
    xs = [big, mid[0], mid[1], -big, mid[2]]
    codes, scales = _ranks(o, xs, 16)
    oc, _ = o.reduce_e4m3(codes, scales, 16)
    fc = [list(cc.astype(int)) for cc in codes]
    fs = [[Fraction(float(v)) for v in ss] for ss in scales]
    fwd, _ = brute.reduce_e4m3(fc, fs, 16)
    rev, _ = brute.reduce_e4m3(fc[::-1], fs[::-1], 16)
    assert fwd != rev, "inputs do not separate the two orders"
    assert list(oc.astype(int)) == fwd, "reduce is not in rank order"


def pin_e4m3_reduce_bound(o) -> None:
    """The one-shot result stays within (3) with (1e) of the exact sum."""
    rng = np.random.default_rng(79)
    xs = [(rng.normal(0, 1, 8192) * np.exp(rng.normal(0, 2, 8192))).astype(np.float32) for _ in range(8)]
    codes, scales = _ranks(o, xs, 256)
    oc, os_ = o.reduce_e4m3(codes, scales, 256)
    ys = [o.dequantize_e4m3(c, s, 256) for c, s in zip(codes, scales)]
    out = o.dequantize_e4m3(oc, os_, 256).astype(np.float64)
    exact = np.sum([x.astype(np.float64) for x in xs], axis=0)
    bnd = bounds.oneshot_bound_e4m3(xs, scales, ys, os_, 256)
    assert np.all(np.abs(out - exact) <= bnd), "E4M3 one-shot bound"


def pin_e4m3_ring_brute_tiny(o) -> None:
    """Ring steps with bf16 and fp32 local data, signed zeros included:
    equal to the brute force."""
    rng = np.random.default_rng(83)
    for block, n, kind in ((4, 12, "f32"), (5, 13, "bf16"), (16, 40, "f32")):
        x0 = (rng.normal(0, 1, n) * np.exp(rng.normal(0, 3, n))).astype(np.float32)
        x1 = (rng.normal(0, 1, n) * np.exp(rng.normal(0, 3, n))).astype(np.float32)
        x1[0] = -0.0
        local = synth.f32_to_bf16_bits(x1) if kind == "bf16" else x1
        c, s = o.quantize_e4m3(x0, block)
        oc, os_ = o.ring_step_e4m3(c, s, local, block)
        lv, ln = _frac_list(local)
        bc, bs = brute.ring_step_e4m3(list(c.astype(int)), [Fraction(float(v)) for v in s], lv, ln, block)
        assert list(oc.astype(int)) == bc, f"ring {kind} block {block}: codes differ from brute force"
        assert [Fraction(float(v)) for v in os_] == bs, f"ring {kind} block {block}: scales differ"


def pin_e4m3_ring_bound(o) -> None:
    rng = np.random.default_rng(89)
    xs = [(rng.laplace(0, 0.5, 4096)).astype(np.float32) for _ in range(4)]
    c, s = o.quantize_e4m3(xs[0], 256)
    step_scales, step_values = [s], [xs[0]]
    exact = xs[0].astype(np.float64)
    for k in range(1, 4):
        p = (o.dequantize_e4m3(c, s, 256) + xs[k]).astype(np.float32)
        c, s = o.ring_step_e4m3(c, s, xs[k], 256)
        exact = exact + xs[k]
        step_scales.append(s)
        step_values.append(p)
        err = np.abs(o.dequantize_e4m3(c, s, 256).astype(np.float64) - exact)
        assert np.all(err <= bounds.ring_bound_e4m3(step_scales, step_values, 256)), f"ring step {k} bound"


ALL_PINS = [
    pin_e4m3_decode,
    pin_e4m3_encode_torch,
    pin_e4m3_encode_brute,
    pin_e4m3_quantize_brute_tiny,
    pin_e4m3_absmax_code,
    pin_e4m3_sign_and_scaling,
    pin_e4m3_zero_blocks,
    pin_e4m3_dequant,
    pin_e4m3_roundtrip_bound,
    pin_e4m3_nonfinite_rejected,
    pin_e4m3_reduce_brute_tiny,
    pin_e4m3_reduce_order_and_single,
    pin_e4m3_reduce_bound,
    pin_e4m3_ring_brute_tiny,
    pin_e4m3_ring_bound,
]
