"""The kernels' fast quotient path (normal block scales) skips the clamp of
the rounded quotient to [-Q, Q]: with s = fl(m/Q) normal and |x| <= m (the
block's absmax), fl(x/s) <= Q + 2^-16, so its nearest integer is at most Q.
Checked here in IEEE binary32 (numpy) for every significand of m at several
exponents, Q = 127 (int8) and Q = 7 (4-bit), at x = m, the largest quotient
of the block.  Also checks that a subnormal scale does need the clamp."""
import numpy as np
import pytest


@pytest.mark.parametrize("q", [127.0, 7.0])
@pytest.mark.parametrize("exp", [-93, -60, -1, 0, 1, 37, 100, 127])
def test_quotient_of_the_absmax_never_exceeds_q(q, exp):
    mant = np.arange(1 << 23, dtype=np.uint32)
    m = ((np.uint32(exp + 127) << np.uint32(23)) | mant).view(np.float32)
    s = m / np.float32(q)
    assert s.dtype == np.float32
    normal = s >= np.float32(2.0 ** -100)
    assert normal.all()
    quot = m / s                                       # correctly rounded binary32
    assert quot.dtype == np.float32
    assert float(quot.max()) <= q + 2.0 ** -16
    assert float(np.rint(quot).max()) <= q


def test_subnormal_scale_needs_the_clamp():
    m = np.float32(190 * 2.0 ** -149)
    s = m / np.float32(127.0)
    assert s == np.float32(2.0 ** -149)
    assert m / s == np.float32(190.0)
