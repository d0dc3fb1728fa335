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

}  // namespace locks
