// rans_coding.hpp -- device arithmetic shared by the coding kernels.
#pragma once

#include "rans_internal.hpp"

namespace rans {

// Reciprocal of f in fp64 for the quotient estimate: the hardware estimate
// refined by two Newton-Raphson steps r <- r + r(1 - f r), which square the
// relative error each time (from about 2^-23 to far below the 2^-52 of the
// final rounding).
__device__ inline double reciprocal(uint32_t f)
{
    const double fd = (double)f;
    double r = __builtin_amdgcn_rcp(fd);
    double e = __builtin_fma(-fd, r, 1.0);
    r = __builtin_fma(r, e, r);
    e = __builtin_fma(-fd, r, 1.0);
    return __builtin_fma(r, e, r);
}

// x <- floor(x/f)*2^16 + (x mod f) + start, for x < f * 2^47.
// q = round(x * (1/f)) is read from the mantissa of fma(x, 1/f, 2^52); with
// x/f < 2^47 and a relative error below 2^-50 the estimate is floor(x/f) or
// one more, so one exact correction on the low 32 bits of x - q*f (which lie
// in [-f, f)) gives the true quotient and remainder.
__device__ inline uint64_t reg_step(uint64_t x, uint32_t start, uint32_t f, double rcp)
{
    const double xd = __builtin_fma((double)(uint32_t)(x >> 32), 4294967296.0,
                                    (double)(uint32_t)x);
    const double t = __builtin_fma(xd, rcp, 4503599627370496.0);   // 2^52
    uint64_t q = (uint64_t)__double_as_longlong(t) & ((1ull << 52) - 1);
    int32_t r = (int32_t)((uint32_t)x - (uint32_t)q * f);
    if (r < 0) {
        q -= 1;
        r += (int32_t)f;
    }
    return (q << kPrecision) + (uint32_t)r + start;
}

}  // namespace rans
