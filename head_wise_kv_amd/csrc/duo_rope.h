// Rotary position embedding for the HIP kernels.  The pages name no
// positional encoding, only that a cached token keeps its logical position
// ("Attention Variants and Memory Efficiency", "Sliding-Window and Mixed
// Attention"); the reading taken is the rotary embedding of Su et al.
// (RoFormer, 2021): pair i of a row at position p turns by the angle
// p * theta^(-2i/d).
//
// The angle is formed so that it stays exact to double rounding at every
// position up to 2^31: the powers theta^(-2 * 2^k / d) come from the host as
// double-doubles (about 104 bits), the frequency theta^(-2i/d) is the product
// of those of i's set bits, taken in double-double,
// the product with p is kept as a double-double (an FMA gives the low part),
// and the reduction modulo 2 pi subtracts k * 2 pi in three parts (Cody and
// Waite), the first two short enough that k times them is exact for
// |k| < 2^29.  Cosine and sine of the reduced angle are then taken in double.
// Keys, which the cache stores, are rotated in double and rounded once to the
// cache dtype, so the stored value (and an FP8 code quantized from it) is the
// correctly rounded rotation; queries, which are only attended, are rotated
// in float.
#pragma once

#include <math.h>

#include "duo_internal.h"

namespace duo {

// (h, l) <- (h, l) * (bh, bl), double-double.  Contraction stays off: fusing
// h = p + e into fma(h, bh, e) would add the product's rounding error, which e
// already holds, a second time.
__device__ __forceinline__ void dd_mul(double& h, double& l, double bh, double bl) {
#pragma clang fp contract(off)
  const double p = h * bh;
  double e = fma(h, bh, -p);
  e = fma(h, bl, fma(l, bh, e));
  h = p + e;
  l = e - (h - p);
}

// 2 pi = kTwoPi1 + kTwoPi2 + kTwoPi3 to about 101 bits; the first two have at
// most 24 significant bits.
constexpr double kTwoPi1 = 0x1.921fb6p+2;
constexpr double kTwoPi2 = -0x1.777a5cp-23;
constexpr double kTwoPi3 = -0x1.ee59d9cceba4p-48;
constexpr double kInvTwoPi = 0x1.45f306dc9c883p-3;

// cos and sin of the angle of pair i at position p (0 <= p < 2^31).
__device__ __forceinline__ void rope_cs(const Rope& r, int64_t p, int i, double& c, double& s) {
#pragma clang fp contract(off)
  double fh = 1.0, fl = 0.0;  // f = theta^(-2i/d): the product over i's set bits
#pragma unroll
  for (int k = 0; k < kRopeBits; ++k)
    if ((i >> k) & 1) dd_mul(fh, fl, r.hi[k], r.lo[k]);
  const double pd = (double)p;  // exact
  const double ah = pd * fh;
  const double al = fma(pd, fh, -ah) + pd * fl;  // p * f = ah + al
  const double k = rint(ah * kInvTwoPi);
  double red = fma(-k, kTwoPi1, ah);  // exact
  red = fma(-k, kTwoPi2, red);
  red = fma(-k, kTwoPi3, red);
  sincos(red + al, &s, &c);
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
