"""Pins of the error bounds in ``oracle/bounds.py``: inputs built by hand so
that the roundings line up, whose errors (the oracle's dequantized result
against the exact sum) come within a few percent of bounds (1), (3), (4)
and (1e).  A bound loosened in its main terms (a scale term doubled, E4M3's
relative or absolute term doubled) then falls far short of these errors and
a pin fails; ``tests/test_bounds_pins.py`` plants each such change in a copy
of ``bounds.py`` and checks that.  One more pin shows that bound (1) needs
its second term: a quotient that binary32 rounds onto a tie, which then goes
to the far integer, misses by more than s/2.

Not pinned by data: the gamma term of (3) and the 2^-21|p| term of (4).
Each is below a few 1e-5 of the scale terms beside it, so no input can tell
them from twice or half their size; they follow from the standard binary32
error model (one rounding per operation, |delta| <= 2^-24).

Each ``pin_*`` takes the bounds module and the oracle.

Method: "EQuARX: Efficient Quantized AllReduce in XLA for Distributed Machine
Learning Acceleration": the abstract and the "problem definition" section
name the error that summing quantized data builds up; the pages give no
bound.
"""
from __future__ import annotations

import numpy as np


def _f32(vals, n=64):
    x = np.zeros(n, np.float32)
    for i, v in vals.items():
        x[i] = v
    return x


def pin_requant_bound_reached(bounds, o):
    """x = 2.5 in a block whose absmax is 127: s = 1, the quotient 2.5 is a
    tie that goes to the even code 2, so the error is exactly s/2."""
    x = _f32({0: 127.0, 5: 2.5, 6: -2.5, 7: 6.5})
    c, s = o.quantize(x, 64)
    y = o.dequantize(c, s, 64, "f32").astype(np.float64)
    err = np.abs(y - x.astype(np.float64))
    bnd = bounds.requant_bound(np.abs(x.astype(np.float64)), bounds.per_element(s, 64, x.size))
    assert np.all(err <= bnd), "bound (1) violated"
    assert err[5] / bnd[5] >= 0.999 and err[7] / bnd[7] >= 0.999, ("bound (1) far above a reachable error",
                                                                    err[5] / bnd[5])


def pin_requant_second_term_needed(bounds, o):
    """A quotient x/s just below a tie k + 1/2 that binary32 rounds onto the
    tie, which then goes to the even k + 1: the error exceeds s/2, so bound
    (1) cannot be s/2 alone; it stays within s/2 + 2^-22 |x|."""
    rng = np.random.default_rng(5)
    worst = 0.0
    for _ in range(400):
        absmax = np.float32(rng.uniform(64.0, 127.0) * 2.0 ** int(rng.integers(-20, 20)))
        s = np.float32(absmax / np.float32(127.0))
        k = int(rng.integers(60, 125)) | 1                  # k odd: the tie k + 1/2 goes up to k + 1
        x0 = np.float32((k + 0.5) * float(s))
        for step in range(1, 40):
            x = np.nextafter(x0, np.float32(0.0), dtype=np.float32)
            x0 = x
            if np.float32(x / s) != np.float32(k + 0.5):
                break
            if float(x) / float(s) >= k + 0.5:              # not below the tie: skip
                continue
            blk = _f32({0: absmax, 3: x})
            c, sc = o.quantize(blk, 64)
            if sc[0] != s:
                continue
            y = float(o.dequantize(c, sc, 64, "f32")[3])
            err = abs(y - float(x))
            bnd = float(bounds.requant_bound(np.array([abs(float(x))]), np.array([float(s)]))[0])
            assert err <= bnd, "bound (1) violated"
            worst = max(worst, err / float(s))
    assert worst > 0.5, f"no error above s/2 found (worst {worst} s): the second term of (1) would be idle"


def pin_oneshot_bound_reached(bounds, o):
    """Four ranks, each block with its own 127 (so every input scale is 1),
    2.5 at element 4 (code 2 in every rank: errors add up to 2) and codes
    56, 56, 57, 57 at element 5, whose sum 226 sets the output scale
    s_out = 226/127: element 4's sum 8 is 4.4955 s_out and goes down to
    4 s_out, an output error of nearly s_out/2 on top."""
    xs = []
    for r, v in enumerate((56.0, 56.0, 57.0, 57.0)):
        xs.append(_f32({r: 127.0, 4: 2.5, 5: v}))
    qs = [o.quantize(x, 64) for x in xs]
    oc, os_ = o.reduce([q[0] for q in qs], [q[1] for q in qs], 64)
    y = o.dequantize(oc, os_, 64, "f32").astype(np.float64)
    exact = sum(x.astype(np.float64) for x in xs)
    ys = [o.dequantize(c, s, 64, "f32") for c, s in qs]
    bnd = bounds.oneshot_bound(xs, [q[1] for q in qs], ys, os_, 64)
    err = np.abs(y - exact)
    assert np.all(err <= bnd), "bound (3) violated"
    assert err[4] / bnd[4] >= 0.99, ("bound (3) far above a reachable error", err[4] / bnd[4])


def pin_ring_bound_reached(bounds, o):
    """Ring of three steps with scale 1 throughout (rank 0 holds the 127) and
    2.5 added at element 4 in every rank: 2.5 -> 2, 4.5 -> 4, 6.5 -> 6, each
    a tie to the even code, so the error after step k is exactly (k+1)/2,
    the sum of the step scales' halves."""
    xs = [_f32({0: 127.0, 4: 2.5})] + [_f32({4: 2.5}) for _ in range(2)]
    c, s = o.quantize(xs[0], 64)
    step_scales, step_values = [s], [xs[0]]
    exact = xs[0].astype(np.float64)
    for k in range(1, 3):
        p = (o.dequantize(c, s, 64, "f32") + xs[k]).astype(np.float32)
        c, s = o.ring_step(c, s, xs[k], 64)
        step_scales.append(s)
        step_values.append(p)
        exact = exact + xs[k]
        err = np.abs(o.dequantize(c, s, 64, "f32").astype(np.float64) - exact)
        bnd = bounds.ring_bound(step_scales, step_values, 64)
        assert np.all(err <= bnd), f"bound (4) violated at step {k}"
        assert err[4] / bnd[4] >= 0.999, ("bound (4) far above a reachable error", k, err[4] / bnd[4])


def pin_e4m3_bound_reached(bounds, o):
    """E4M3 codes with s = 1 (absmax 448): 1.0625 lies halfway between the
    E4M3 values 1 and 1.125 and goes to 1 (even mantissa): a relative error
    of 1/17, near the 2^-4 |x| term; 2^-10 lies halfway between 0 and the
    smallest subnormal 2^-9 and goes to 0: an error of 2^-10 s, the
    absolute term."""
    x = _f32({0: 448.0, 3: 1.0625, 4: 2.0 ** -10, 5: -17.0})
    c, s = o.quantize_e4m3(x, 64)
    y = o.dequantize_e4m3(c, s, 64, "f32").astype(np.float64)
    err = np.abs(y - x.astype(np.float64))
    bnd = bounds.requant_bound_e4m3(np.abs(x.astype(np.float64)), bounds.per_element(s, 64, x.size))
    assert np.all(err <= bnd), "bound (1e) violated"
    for i in (3, 4, 5):
        assert err[i] / bnd[i] >= 0.9, ("bound (1e) far above a reachable error", i, err[i] / bnd[i])


PINS = [pin_requant_bound_reached, pin_requant_second_term_needed, pin_oneshot_bound_reached,
        pin_ring_bound_reached, pin_e4m3_bound_reached]
