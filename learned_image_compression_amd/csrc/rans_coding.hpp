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

// x <- floor(x/f)*2^16 + (x mod f) + start, for x < f * 2^47 and
// 1 <= f <= 2^16.  q = round(x * (1/f)) is read from the mantissa of
// fma(x, 1/f, 2^52); with x/f < 2^47 and a relative error below 2^-50 the
// estimate is floor(x/f) or one more, and r = x - q*f (whose low 32 bits
// hold it exactly, as |r| < 2^16) says which.  The result is then
//   q*2^16 + r + start                  when r >= 0,
//   (q-1)*2^16 + (r + f) + start        when r < 0,
// i.e. q*2^16 + s with the 32-bit s = r + start + (r < 0 ? f - 2^16 : 0),
// s in [-2^16, 2^17).  Shifting the double's bit pattern left by 16 keeps
// exactly q*2^16 (q < 2^47 sits in its low 47 bits; the exponent bits move
// out), and s is added sign-extended.
__device__ inline uint64_t reg_step(uint64_t x, uint32_t start, uint32_t f, double rcp)
{
    // (the halves taken as a two-word vector: written as x >> 32, the high
    // half's conversion becomes a 64-bit one with an extra fp64 add)
    typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
    const u32x2 h = __builtin_bit_cast(u32x2, x);
    const uint32_t lo = h.x, hi = h.y;
    const double xd = __builtin_fma((double)hi, 4294967296.0, (double)lo);
    const double t = __builtin_fma(xd, rcp, 4503599627370496.0);   // 2^52
    const uint64_t tb = (uint64_t)__double_as_longlong(t);
    const int32_t r = (int32_t)(lo - (uint32_t)tb * f);
    // s < 0 exactly when r < 0 (then s < start + f - 2^16 <= 0), so r's sign
    // word m serves as s's high word (no sign extension of s itself)
    const uint32_t m = (uint32_t)(r >> 31);
    const uint32_t s = (uint32_t)r + start + (m & (f - kTotal));
    const u32x2 sm = {s, m};
    return (tb << kPrecision) + __builtin_bit_cast(uint64_t, sm);
}

}  // namespace rans
