// quotient_sweep.hip -- test support, not part of libqar: runs libqar's
// fast quotient (qar::fast_quotient, with the reciprocal computed as the
// kernels compute it) on binary32 significand pairs and checks every result
// exactly, without any floating-point division.
//
// x and s run over [1, 2), i.e. over every pair of significands.  A normal
// binary32 value y is the correctly rounded x / s exactly when the residual
// d = x - y*s satisfies 2|d| < s*u, or 2|d| == s*u with an even significand,
// where u is the spacing of binary32 values at y; when y is a power of two
// and x / s lies below it the spacing there is u/2, so 2|d| <= s*u/2 (the
// tie then goes to y, whose significand is even).  In binary64, y*s is
// exact (two 24-bit significands), x - y*s is exact whenever y is within a
// few spacings of x / s (a multiple of u*2^-23 below 2^-21 in magnitude),
// and s*u is exact (a power of two times s); a y further off yields a large
// |d| and fails either way.  The reciprocal r = 1/s is checked the same way
// with x = 1.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qar_device.h"

namespace {

__device__ __forceinline__ float f_of(uint32_t b) { return __builtin_bit_cast(float, b); }

// y (normal) is the correctly rounded num / den; num, den binary32 values
__device__ __forceinline__ bool rounds_exactly(float y, double num, double den) {
    const uint32_t b = __builtin_bit_cast(uint32_t, y);
    const double d = __builtin_fma(-(double)y, den, num);
    double lim = den * (double)f_of((b & 0x7F800000u) - (23u << 23));   // s * u
    if (d < 0.0 && (b & 0x7FFFFFu) == 0u) lim *= 0.5;
    const double a2 = 2.0 * __builtin_fabs(d);
    return a2 < lim || (a2 == lim && (b & 1u) == 0u);
}

} // namespace

// Thread t takes the divisor significand S = 2^23 + t (t < 2^23) and the
// dividend significands X = 2^23 + x_lo .. 2^23 + x_lo + x_count - 1.
// bad[t] += mismatches of the quotient; first[t] = the first mismatching
// dividend (if none before); bad_recip[t] = 1 when 1/s is not the correctly
// rounded reciprocal.  mode 0 checks libqar's fast_quotient; mode 1 checks
// the uncorrected product x * r instead, which the checker must catch on
// some pairs (a check of the checker).
__global__ __launch_bounds__(256) void k_quotient_sweep(uint32_t x_lo, uint32_t x_count, int mode, uint32_t* bad,
                                                        uint32_t* first, uint32_t* bad_recip) {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    const float s = f_of(0x3F800000u | t);
    const float r = 1.0f / s;
    const double sd = (double)s;
    if (x_lo == 0) bad_recip[t] = rounds_exactly(r, 1.0, sd) ? 0u : 1u;
    uint32_t nbad = 0, fx = first[t];
    for (uint32_t i = 0; i < x_count; ++i) {
        const uint32_t xm = x_lo + i;
        const float x = f_of(0x3F800000u | xm);
        const float y = mode == 0 ? qar::fast_quotient(x, s, r) : x * r;
        if (!rounds_exactly(y, (double)x, sd)) {
            ++nbad;
            if (fx == 0xFFFFFFFFu) fx = xm;
        }
    }
    bad[t] += nbad;
    first[t] = fx;
}

// Host entry for the test: one launch over x_lo .. x_lo + x_count - 1 for
// all 2^23 divisors, on the default stream; buffers of 2^23 uint32 each.
extern "C" int quotient_sweep(uint32_t x_lo, uint32_t x_count, int mode, uint32_t* bad, uint32_t* first,
                              uint32_t* bad_recip) {
    if ((uint64_t)x_lo + x_count > (1u << 23) || !bad || !first || !bad_recip) return -1;
    void* args[] = {&x_lo, &x_count, &mode, &bad, &first, &bad_recip};
    return (int)hipLaunchKernel(reinterpret_cast<const void*>(k_quotient_sweep), dim3((1u << 23) / 256u), dim3(256),
                                args, 0, nullptr);
}
