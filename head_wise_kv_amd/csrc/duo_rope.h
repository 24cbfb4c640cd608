// Rotary position embedding for the HIP kernels: the angle of pair i at
// position p is formed and reduced modulo 2 pi in double precision (positions
// reach 2^31, where a float angle would be off by whole radians), and the
// reduced angle's cosine and sine are taken in float.
#pragma once

#include <math.h>

#include "duo_internal.h"

namespace duo {

__device__ __forceinline__ void rope_cs(const Rope& r, int d, int64_t p, int i, float& c, float& s) {
  const double f = exp2(-(2.0 * i / d) * r.log2_theta);  // theta^(-2i/d)
  const double a = (double)p * f;
  const double red = a - rint(a * 0.15915494309189535) * 6.283185307179586;  // a - 2 pi k, |red| <= pi
  sincosf((float)red, &s, &c);
}

}  // namespace duo
