// Device helpers shared by the LOCKS page-selection kernels (gfx950, wave64).
#pragma once

#include "locks_device.h"

namespace locks {

// Selection bins: 1/32 nat wide below the best key, the last bin collecting
// everything further down (and -inf keys).
constexpr int kBins = 512;
constexpr float kBinsPerNat = 32.f;

// ---- block-wide helpers (up to 16 waves)
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}
// Exclusive prefix sum of one int per thread over the workgroup (<= 16 waves).
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh_waves, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh_waves[wave] = x;
  __syncthreads();
  int base = 0, all = 0;
  const int nw = blockDim.x >> 6;
  for (int w = 0; w < nw; ++w) {
    const int t = sh_waves[w];
    if (w < wave) base += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return base + x - v;
}


// Inclusive prefix sum over one wave with DPP row shifts and row broadcasts
// (no LDS): rows of 16 first, then lane 15 of each row into the next row and
// lane 31 into the upper half.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  int x = v + __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);         // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, v, 0x113, 0xF, 0xF, true);         // row_shr:3
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xE, false);        // row_shr:4, lanes 4..15
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xC, false);        // row_shr:8, lanes 8..15
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);        // row_bcast:15, rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);        // row_bcast:31, rows 2, 3
  return x;
}

template <int G>
__device__ __forceinline__ void load_scores(const float* p, float (&v)[G]) {
  if constexpr (G == 4) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else if constexpr (G == 2) {
    const float2 x = *reinterpret_cast<const float2*>(p);
    v[0] = x.x; v[1] = x.y;
  } else {
    v[0] = p[0];
  }
}

// Block-wide max / sum of G values per thread at once (one barrier pair).
template <int G>
__device__ __forceinline__ void block_max_g(float (&v)[G], float (*red)[4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    v[g] = wave_max(v[g]);
    if (lane == 0) red[wave][g] = v[g];
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = red[0][g];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, red[w][g]);
    v[g] = m;
  }
  __syncthreads();
}
template <int G>
__device__ __forceinline__ void block_sum_g(float (&v)[G], float (*red)[4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    v[g] = wave_sum(v[g]);
    if (lane == 0) red[wave][g] = v[g];
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float t = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w][g];
    v[g] = t;
  }
  __syncthreads();
}

template <int G>
__device__ __forceinline__ float group_key(const float (&v)[G], const float (&logZ)[G], float logG) {
  float d[G], m = -__builtin_inff();
#pragma unroll
  for (int g = 0; g < G; ++g) { d[g] = v[g] - logZ[g]; m = fmaxf(m, d[g]); }
  float t = 0.f;
#pragma unroll
  for (int g = 0; g < G; ++g) t += __expf(d[g] - m);
  const float key = m + __logf(t) - logG;
  return (key == key && m != -__builtin_inff()) ? key : -__builtin_inff();
}

// Merge rules (natural log): 0 = share average (group_key), 1 = group-max
// log max_g exp(s_g - logZ_g), 2 = group-mass log sum_g exp(s_g) - logZtot
// with logZtot = log sum_g Z_g.
constexpr int kMergeShare = 0;
constexpr int kMergeMax = 1;
constexpr int kMergeMass = 2;
template <int G>
__device__ __forceinline__ float group_key_rule(const float (&v)[G], const float (&logZ)[G],
                                                float logG, int rule, float logZtot) {
  if (rule == kMergeShare) return group_key<G>(v, logZ, logG);
  float m = -__builtin_inff();
  if (rule == kMergeMax) {
#pragma unroll
    for (int g = 0; g < G; ++g) m = fmaxf(m, v[g] - logZ[g]);
    return (m == m) ? m : -__builtin_inff();
  }
#pragma unroll
  for (int g = 0; g < G; ++g) m = fmaxf(m, v[g]);
  float t = 0.f;
#pragma unroll
  for (int g = 0; g < G; ++g) t += __expf(v[g] - m);
  const float key = m + __logf(t) - logZtot;
  return (key == key && m != -__builtin_inff()) ? key : -__builtin_inff();
}

}  // namespace locks
