"""Error bounds of quantized reduction against the exact (fp64) sum.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``).

EQuARX's pages warn that summing quantized data across devices can build up
error ("EQuARX: Efficient Quantized AllReduce in XLA ...": abstract, and the
page summary's "problem definition"); they give no bound.  The bounds below
are derived from the binary32 model (unit roundoff u = 2**-24, one rounding
per operation, gradual underflow adds at most 2**-150 absolute per rounding):

  requantization of a finite value x in a block with scale s:
      |x - fl32(q*s)| <= s/2 + 2**-22 * |x|                          (1)
  (the quotient rounding contributes u*|x|, the product rounding u*|q*s|;
  the clamp never binds for a normal scale);

  recursive fp32 summation of N terms y_0..y_{N-1} in a fixed order:
      |acc - sum y_r| <= gamma_{N-1} * sum |y_r|,
      gamma_k = k*u / (1 - k*u)                                      (2)

  one-shot reduce (quantize each rank, sum, requantize), per element:
      |out - sum x_r| <= sum_r (s_r/2 + 2**-22 |x_r|)
                         + gamma_{N-1} sum_r |y_r|
                         + s_out/2 + 2**-22 (1 + gamma_{N-1}) sum_r |y_r|   (3)

  ring reduction, after step k (p_0 = x_0, p_j = fl32(y_{j-1} + x_j)):
      |out_k - sum_{j<=k} x_j| <= sum_{j<=k} (s_j/2 + 2**-21 |p_j|)        (4)
  (each step adds one fp32 add, u*|p_j|, and one requantization, (1)).

The simpler forms used as a second, data-dependent check are
N*max_scale/2 + 1e-6*|sum| (one-shot; max_scale over every scale applied to
the element: the N input scales and the output scale) and
sum_j s_j/2 + 1e-6*|sum| (ring).  Adversarial inputs can exceed them; (3) and
(4) cannot be exceeded.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24
TINY = 2.0 ** -149      # slack per rounding for results in the subnormal range


def gamma(k: int) -> float:
    return k * U / (1.0 - k * U)


def per_element(scales: np.ndarray, block: int, n: int) -> np.ndarray:
    """Broadcast per-block scales to elements, as float64."""
    return np.repeat(np.asarray(scales, np.float64), block)[:n]


def requant_bound(x_abs: np.ndarray, s_elem: np.ndarray) -> np.ndarray:
    """(1): bound on |x - dequantize(quantize(x))|."""
    return s_elem / 2.0 + 2.0 ** -22 * x_abs + 2 * TINY


def oneshot_bound(xs, scales_in, ys, scale_out, block: int) -> np.ndarray:
    """(3) per element.  xs: the N original rank values (any float dtype);
    scales_in: the N per-block scale arrays; ys: the N dequantized fp32
    arrays; scale_out: per-block scales of the requantized sum."""
    n = np.asarray(xs[0]).size
    nr = len(xs)
    sum_abs_y = np.zeros(n)
    bound = np.zeros(n)
    for x, s, y in zip(xs, scales_in, ys):
        bound += requant_bound(np.abs(np.asarray(x, np.float64).reshape(-1)), per_element(s, block, n))
        sum_abs_y += np.abs(np.asarray(y, np.float64).reshape(-1))
    g = gamma(nr - 1)
    bound += g * sum_abs_y + nr * TINY
    bound += per_element(scale_out, block, n) / 2.0 + 2.0 ** -22 * (1.0 + g) * sum_abs_y + 2 * TINY
    return bound


def oneshot_bound_simple(scales_in, scale_out, exact_sum: np.ndarray, block: int) -> np.ndarray:
    """N * max_scale / 2 + 1e-6 * |sum| per element."""
    n = exact_sum.size
    m = per_element(scale_out, block, n)
    for s in scales_in:
        m = np.maximum(m, per_element(s, block, n))
    return len(scales_in) * m / 2.0 + 1e-6 * np.abs(exact_sum)


def ring_bound(step_scales, step_values, block: int) -> np.ndarray:
    """(4) after the last listed step.  step_scales[j]: per-block scales
    produced at step j; step_values[j]: the fp32 values quantized at step j."""
    n = np.asarray(step_values[0]).size
    b = np.zeros(n)
    for s, p in zip(step_scales, step_values):
        b += per_element(s, block, n) / 2.0 + 2.0 ** -21 * np.abs(np.asarray(p, np.float64).reshape(-1)) + 3 * TINY
    return b


def ring_bound_simple(step_scales, exact_sum: np.ndarray, block: int) -> np.ndarray:
    n = exact_sum.size
    b = np.zeros(n)
    for s in step_scales:
        b += per_element(s, block, n) / 2.0
    return b + 1e-6 * np.abs(exact_sum)


# ---------------------------------------------------------------------------
# FP8 E4M3 codes.  An E4M3 value has 3 mantissa bits: on [2^e, 2^(e+1)),
# e >= -6, neighbours are 2^(e-3) apart, so rounding a quotient t moves it by
# at most 2^-4 |t|; below 2^-6 the spacing is the subnormal step 2^-9, so at
# most 2^-10.  With the quotient and product roundings (u each):
#
#   |x - fl32(e4m3(t) * s)| <= (2^-4 + 4u) |x| + (2^-10 + u) s      (1e)
#
# (u|y| <= 2u|x| + u s because |y| <= (1 + 2^-3)|x| + 2^-9 s).  The one-shot
# and ring bounds are (3) and (4) above with (1e) in place of (1).

E4M3_REL = 2.0 ** -4 + 4 * U
E4M3_ABS = 2.0 ** -10 + U


def requant_bound_e4m3(x_abs: np.ndarray, s_elem: np.ndarray) -> np.ndarray:
    """(1e): bound on |x - dequantize(quantize(x))| for E4M3 codes."""
    return E4M3_REL * x_abs + E4M3_ABS * s_elem + 2 * TINY


def oneshot_bound_e4m3(xs, scales_in, ys, scale_out, block: int) -> np.ndarray:
    n = np.asarray(xs[0]).size
    nr = len(xs)
    sum_abs_y = np.zeros(n)
    bound = np.zeros(n)
    for x, s, y in zip(xs, scales_in, ys):
        bound += requant_bound_e4m3(np.abs(np.asarray(x, np.float64).reshape(-1)), per_element(s, block, n))
        sum_abs_y += np.abs(np.asarray(y, np.float64).reshape(-1))
    g = gamma(nr - 1)
    bound += g * sum_abs_y + nr * TINY
    bound += requant_bound_e4m3((1.0 + g) * sum_abs_y, per_element(scale_out, block, n))
    return bound


def ring_bound_e4m3(step_scales, step_values, block: int) -> np.ndarray:
    n = np.asarray(step_values[0]).size
    b = np.zeros(n)
    for s, p in zip(step_scales, step_values):
        pa = np.abs(np.asarray(p, np.float64).reshape(-1))
        b += requant_bound_e4m3(pa, per_element(s, block, n)) + U * pa + TINY
    return b
