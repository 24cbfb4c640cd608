// Rotary position embedding for the HIP kernels.  The angle of pair i at
// position p is formed and reduced modulo 2 pi in double precision (positions
// reach 2^31, where a float angle would be off by whole radians), and its
// cosine and sine are taken in double.  Keys, which the cache stores, are
// rotated in double and rounded once to the cache dtype, so the stored value
// (and an FP8 code quantized from it) is the correctly rounded rotation;
// queries, which are only attended, are rotated in float.
#pragma once

#include <math.h>

#include "duo_internal.h"

namespace duo {

__device__ __forceinline__ void rope_cs(const Rope& r, int d, int64_t p, int i, double& c, double& s) {
  const double f = exp2(-(2.0 * i / d) * r.log2_theta);  // theta^(-2i/d)
  const double a = (double)p * f;
  const double red = a - rint(a * 0.15915494309189535) * 6.283185307179586;  // a - 2 pi k, |red| <= pi
  sincos(red, &s, &c);
}

// bf16 bits of the double x rounded to nearest, ties to even (x finite and in
// float range): one rounding, straight from double.
__device__ __forceinline__ uint32_t bf16_bits_from_double(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint64_t lsb = (u >> 45) & 1ull;  // bf16 keeps 7 of double's 52 mantissa bits
  u += (1ull << 44) - 1ull + lsb;
  u &= ~((1ull << 45) - 1ull);
  return __float_as_uint((float)__longlong_as_double((long long)u)) >> 16;  // exact conversion
}

}  // namespace duo
