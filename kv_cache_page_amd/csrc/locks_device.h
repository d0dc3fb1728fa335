// Internal device helpers of the LOCKS HIP library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace locks {

constexpr int kHeadDim = 128;
constexpr int kPage = 16;
// Pages one score workgroup covers (one Z partial per tile of this many).
constexpr int kScorePagesPerWg = 128;
// Flag bits of the score kernels: fill the entries of pages that are not
// scored with NaN; score only the pages full before the current token (the
// deferred build: F = (len - 1) / page_size).
constexpr int kScoreFillNan = 1;
constexpr int kScoreDeferred = 2;
// Bits 8..15 of the score flags: a head divisor (0 reads as 1). Head h of H
// then reads the slots of, and appends the new K/V row to, head h / div of
// H / div in the pools, while its query, outputs and workspace rows stay its
// own: with div = G every query head of a group is a head of its own.
constexpr int kScoreHeadDivShift = 8;
__host__ __device__ inline int score_head_div(int flags) {
  const int v = (flags >> kScoreHeadDivShift) & 0xFF;
  return v ? v : 1;
}

// Full pages that are summarised (scored) at length len: floor(len / B), or,
// when the build of a page completed by the current token is deferred,
// floor((len - 1) / B).
__device__ __forceinline__ int scored_pages(int len, int lag) {
  return (len - lag > 0 ? len - lag : 0) / kPage;
}
// Exchange counters of the fused decode step, per (sequence, KV head): 4
// counters, one 128-byte line each, at the start of its mailbox.
constexpr int kCoopCounters = 4;
constexpr int kCoopCtrWords = 32;

// Where the score kernel of a fused decode step zeroes the decode kernel's
// mailboxes: `words` words at base + sh * stride for every (sequence, KV
// head) sh, shared out over the tile rows of that head.
struct CoopZero {
  uint32_t* base;
  int64_t stride;
  int words;
};

// Called by every workgroup of the score grid (tile row blockIdx.y of
// gridDim.y); coherent agent-scope stores; no-op for a null base.
// Stores that reach memory coherently for every XCD (agent-scope relaxed
// atomics), for data read by other workgroups of the same launch.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint4* p, uint4 v) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  __hip_atomic_store(q, (uint64_t)v.x | ((uint64_t)v.y << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, (uint64_t)v.z | ((uint64_t)v.w << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup `part` of `nparts` zeroes its share of mailbox `sh`.
__device__ __forceinline__ void zero_coop_mailbox(const CoopZero& z, int64_t sh, int part, int nparts) {
  if (!z.base) return;
  uint32_t* p = z.base + sh * z.stride;
  for (int w = part * blockDim.x + threadIdx.x; w < z.words; w += nparts * blockDim.x)
    __hip_atomic_store(p + w, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Summary slot byte layout: [Vq r*d*bits/8][Cq B*r][muq d][fp16 scales r+B+1][pad]
// (bits = 4 for the int4 basis; 8 and 2 for the precision ablation). The
// stride is a whole number of 128-byte lines, so every slot starts on a line
// and no two slots (read by the workgroups of different heads, on different
// XCDs) share one.
struct SlotLayout {
  int v, c, mu, sv, sc, smu, payload, stride;
};

__host__ __device__ constexpr SlotLayout slot_layout(int r, int bits = 4) {
  return SlotLayout{0,
                    r * kHeadDim * bits / 8,
                    r * kHeadDim * bits / 8 + kPage * r,
                    r * kHeadDim * bits / 8 + kPage * r + kHeadDim,
                    r * kHeadDim * bits / 8 + kPage * r + kHeadDim + 2 * r,
                    r * kHeadDim * bits / 8 + kPage * r + kHeadDim + 2 * (r + kPage),
                    r * kHeadDim * bits / 8 + kPage * r + kHeadDim + 2 * (r + kPage + 1),
                    (r * kHeadDim * bits / 8 + kPage * r + kHeadDim + 2 * (r + kPage + 1) + 127) / 128 * 128};
}

// Largest code of the symmetric b-bit basis quantiser: 2^(b-1) - 1.
__host__ __device__ constexpr int basis_qmax(int bits) { return (1 << (bits - 1)) - 1; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Lane exchanges. DPP quad permutations move data inside groups of 4 lanes;
// ds_swizzle in bit-mask mode xors the lane id inside groups of 32 lanes.
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
// Sum over the 4 lanes of a quad. (a+b)+(c+d) is bit-identical on every lane.
__device__ __forceinline__ float quad_sum(float v) {
  v += quad_xor1(v);
  return v + quad_xor2(v);
}
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, quad_xor1(v));
  return fmaxf(v, quad_xor2(v));
}

template <int M>
__device__ __forceinline__ int swz_xor(int v) {
  static_assert(M > 0 && M < 32, "xor mask");
  return __builtin_amdgcn_ds_swizzle(v, 0x1F | (M << 10));
}
template <int M>
__device__ __forceinline__ float swz_xor(float v) {
  return __int_as_float(swz_xor<M>(__float_as_int(v)));
}
template <int M>
__device__ __forceinline__ double swz_xor(double v) {
  uint64_t u = __builtin_bit_cast(uint64_t, v);
  int lo = swz_xor<M>((int)(uint32_t)u);
  int hi = swz_xor<M>((int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Full-wave reductions: DPP inside rows of 16 (quad xor 1, quad xor 2, half-
// row mirror, row mirror), then a swizzle across rows of a half-wave and one
// lane permute across the halves. Every lane ends with the result.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_allmax(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  v = fmaxf(v, dppf<0x140>(v));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
// Sum in a fixed order: lanes holding the same inputs get the same bits.
__device__ __forceinline__ float wave_allsum(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x141>(v);
  v += dppf<0x140>(v);
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  return v + __shfl_xor(v, 32, 64);
}

// Max / sum over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 (same column of the
// four 16-lane rows); the result is bit-identical in all four.
__device__ __forceinline__ float xrow_max(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t y = __float_as_uint(m);
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xrow_sum(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t y = __float_as_uint(m);
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Order-preserving map of a float onto uint32 (larger float -> larger uint).
__device__ __forceinline__ uint32_t float_to_ordered(float f) {
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Online log-sum-exp state (max m, sum s of exp(x - m)): absorb (m2, s2).
// Branch-free (an empty state has m = -inf, s = 0).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  const bool empty = (M == -__builtin_inff());
  const float a = empty ? 0.f : __expf(m - M), b = empty ? 0.f : __expf(m2 - M);
  s = s * a + s2 * b;
  m = M;
}

// Same in base 2 (s is a sum of 2^(x - m)).
__device__ __forceinline__ void lse2_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  const bool empty = (M == -__builtin_inff());
  const float a = empty ? 0.f : __builtin_amdgcn_exp2f(m - M);
  const float b = empty ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
  s = s * a + s2 * b;
  m = M;
}

}  // namespace locks
