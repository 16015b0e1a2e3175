// Device helpers shared by the gfx950 kernels: rounding to bfloat16 and the
// fp64 sine and cosine of RoPE angles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ct {

// bf16 bits (in the low 16 bits) of an fp32 value, rounded to nearest even.
// A NaN stays a NaN (quieted, sign kept) instead of carrying into Inf.
__device__ inline uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// bf16 bits of a double with one rounding to nearest even.  When the rounded
// value is a normal bf16 the rounding is done on the fp64 bits: add half an
// ulp of 8 significant bits (less one, plus the kept lowest bit for ties) and
// cut; a carry moves into the exponent field, which is then re-biased.
// Otherwise (zero, subnormal, overflow, Inf, NaN) the value is truncated to
// binary32 with a sticky bit (round to odd) and rounded again, which cannot
// double-round.  NaN stays NaN.
__device__ inline uint16_t bf16_from_f64(double d) {
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  const uint64_t mag = u & 0x7fffffffffffffffull;
  const uint64_t r = mag + 0x00000fffffffffffull + ((mag >> 45) & 1ull);
  const int e = (int)(r >> 52) - 1023 + 127;
  if (e >= 1 && e <= 254)
    return (uint16_t)(((uint32_t)(u >> 48) & 0x8000u) | ((uint32_t)e << 7) | ((uint32_t)(r >> 45) & 0x7fu));
  const float f = __double2float_rz(d);
  uint32_t b = __float_as_uint(f);
  if ((double)f != d && !__builtin_isnan(d)) b |= 1u;
  return (uint16_t)bf16_bits_rne(__uint_as_float(b));
}

// sin and cos of an angle in fp64 without branches: Cody-Waite reduction by
// quarter turns (pi/2 split into two doubles), then Taylor polynomials on
// |r| <= pi/4 (sin to degree 13, cos to degree 14: truncation below 1e-14).
// Accurate to a few ulp for the RoPE angles of positions below 2^24.
__device__ inline void rope_sincos(double ang, double* s, double* c) {
  const double q = rint(ang * 0.6366197723675814);
  double r = fma(-q, 1.5707963267948966, ang);
  r = fma(-q, 6.123233995736766e-17, r);
  const double r2 = r * r;
  double ps = 1.6059043836821613e-10;              // 1/13!
  ps = fma(ps, r2, -2.505210838544172e-08);        // -1/11!
  ps = fma(ps, r2, 2.7557319223985893e-06);        // 1/9!
  ps = fma(ps, r2, -1.984126984126984e-04);        // -1/7!
  ps = fma(ps, r2, 8.333333333333333e-03);         // 1/5!
  ps = fma(ps, r2, -1.6666666666666666e-01);       // -1/3!
  const double sr = fma(ps * r2, r, r);
  double pc = -1.1470745597729725e-11;             // -1/14!
  pc = fma(pc, r2, 2.08767569878681e-09);          // 1/12!
  pc = fma(pc, r2, -2.755731922398589e-07);        // -1/10!
  pc = fma(pc, r2, 2.48015873015873e-05);          // 1/8!
  pc = fma(pc, r2, -1.388888888888889e-03);        // -1/6!
  pc = fma(pc, r2, 4.1666666666666664e-02);        // 1/4!
  pc = fma(pc, r2, -0.5);
  const double cr = fma(pc, r2, 1.0);
  const int quad = (int)((long long)q & 3);
  const double sv = (quad & 1) ? cr : sr, cv = (quad & 1) ? sr : cr;
  *s = (quad & 2) ? -sv : sv;
  *c = (quad == 1 || quad == 2) ? -cv : cv;
}

}  // namespace ct
