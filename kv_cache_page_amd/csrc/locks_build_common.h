// Helpers shared by the LOCKS page-summary build kernels (gfx950).
#pragma once

#include "locks_device.h"

namespace locks {

__device__ __forceinline__ uint16_t fp16_scale_bits(double absmax, float qmax) {
  // scale = fp16(RNE(fp32(absmax) / qmax)); an infinite result saturates at 65504
  _Float16 h = (_Float16)((float)absmax / qmax);
  uint16_t b = __builtin_bit_cast(uint16_t, h);
  if ((b & 0x7fffu) == 0x7c00u) b = 0x7bffu;
  return b;
}

__device__ __forceinline__ int quant_code(double x, float scale, int qmax) {
  if (scale == 0.f) return 0;
  float r = rintf((float)x / scale);
  r = fminf(fmaxf(r, (float)-qmax), (float)qmax);
  return (int)r;
}

// Jacobi rotation for [[app, apq], [apq, aqq]] (Golub & Van Loan's symmetric
// Schur 2x2, |angle| <= pi/4). tau = (aqq - app) / (2 apq) comes from the
// hardware fp64 reciprocal estimate and is then rounded to fp32, so
// t = sgn(tau) / (|tau| + sqrt(1 + tau^2)) (a sum of positive terms) is good
// to a few fp32 ulps; tau = +-inf (a_pq below the resolution of the gap)
// gives t = 0, and so does a_pq = 0. c = 1/sqrt(1 + t^2) then comes from the
// fp32 estimate y with one third-order correction y (1 + e/2 + 3e^2/8),
// e = 1 - x y^2, which is exact to fp64 rounding, so c^2 + s^2 = 1 to fp64
// rounding.
__device__ __forceinline__ void rotation_fast(double app, double aqq, double apq, double& c,
                                              double& s) {
  const double num = aqq - app, den = 2.0 * apq;
  const float tau = (num == 0.0) ? 0.f : (float)(num * __builtin_amdgcn_rcp(den));
  float t = copysignf(1.f, tau) *
            __builtin_amdgcn_rcpf(fabsf(tau) + __builtin_amdgcn_sqrtf(fmaf(tau, tau, 1.f)));
  if (den == 0.0) t = 0.f;
  const double td = (double)t;
  const double x = fma(td, td, 1.0);
  const double y = (double)__builtin_amdgcn_rsqf((float)x);
  const double er = fma(-(x * y), y, 1.0);
  c = fma(y * er, fma(0.375, er, 0.5), y);
  s = td * c;
}

}  // namespace locks
