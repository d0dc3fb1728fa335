// Wave-level flash-decoding core over 16 x 128 bf16 KV pages on the matrix
// cores (gfx950).
//
// Per page, with lane l = 16 b + c (b = l / 16, c = l % 16):
//   QK: S^T = K q^T on four v_mfma_f32_16x16x32_bf16 (M = the 16 tokens,
//       N = the G queries padded to 16 with zeros, 32 dims each): lane l
//       feeds dims 32 kk + 8 b .. +7 of key row c (16 contiguous bytes per
//       load, so each load covers 64 contiguous bytes of every row) and the
//       same dims of query c, and receives the logits of query c for tokens
//       4 b .. 4 b + 3.
//   softmax: the 4 lanes of column c hold the 16 tokens of query c; the
//       page max and sum combine them with lane permutes across the four
//       16-lane rows. The running (m, l) of query c live in those lanes.
//   PV: O^T = V^T P^T on eight v_mfma_f32_16x16x16_bf16 (M = 16 dims,
//       N = queries, K = the 16 tokens). P^T, rounded to bf16, is the QK
//       result in place. Row m of dim tile T stands for dim 8 m + T, so lane
//       l reads dims 8 c .. 8 c + 7 of value rows 4 b .. 4 b + 3 (16
//       contiguous bytes each, one whole row per 16 lanes) and takes element
//       T of each row for tile T. Lane l accumulates dims 32 b .. 32 b + 31
//       of query c (dim 32 b + 8 i + T in acc[T][i]), so a wave's partial
//       needs no cross-lane reduction.
// A wave streams its pages with an online softmax (base-2 logits); the K/V of
// the next page load while the current page is computed.
#pragma once

#include "locks_device.h"

namespace locks {

// A workgroup partial holds, per query, acc[128] then (max, sum) and 2 pad
// floats, so every query row starts 16-byte aligned.
constexpr int kPartStride = kHeadDim + 4;

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

struct AttnAcc {
  float m, l;        // running max (base 2) and sum of query lane % 16
  float4v acc[8];    // acc[T][i]: dim 32 (lane / 16) + 8 i + T of that query
};

// Query fragment: dims 32 kk + 8 (lane / 16) .. +7 of query lane % 16 (zero
// for the padding queries).
struct AttnQ {
  uint4 w[4];
};

struct PageRegs {
  uint4 k[4], v[4];
};

__device__ __forceinline__ void attn_init(AttnAcc& a) {
  a.m = -__builtin_inff();
  a.l = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) a.acc[t] = float4v{0.f, 0.f, 0.f, 0.f};
}

// Query fragment from G x 128 bf16 queries, row-major at qg.
template <int G>
__device__ __forceinline__ void attn_load_q(AttnQ& q, const uint16_t* qg, int lane) {
  const int c = lane & 15, b = lane >> 4;
  const uint4* qp = reinterpret_cast<const uint4*>(qg + (c < G ? c : 0) * kHeadDim + 8 * b);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const uint4 w = qp[4 * kk];  // dims 32 kk + 8 b ..
    q.w[kk] = (c < G) ? w : make_uint4(0u, 0u, 0u, 0u);
  }
}

// K/V of the page at element offset `off` of the pools (16 x 128 bf16 each).
__device__ __forceinline__ void attn_load_page(PageRegs& p, const uint16_t* __restrict__ kpool,
                                               const uint16_t* __restrict__ vpool, int64_t off,
                                               int lane) {
  const int c = lane & 15, b = lane >> 4;
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(kpool + off);
  const uint8_t* vb = reinterpret_cast<const uint8_t*>(vpool + off);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) p.k[kk] = *reinterpret_cast<const uint4*>(kb + c * 256 + 64 * kk + 16 * b);
#pragma unroll
  for (int i = 0; i < 4; ++i) p.v[i] = *reinterpret_cast<const uint4*>(vb + (4 * b + i) * 256 + 16 * c);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}

// Online-softmax update with one page whose first `nvalid` tokens are live
// (token 0 always is).
__device__ __forceinline__ void attn_page(AttnAcc& a, const PageRegs& p, const AttnQ& q, int nvalid,
                                          int lane) {
  const int b = lane >> 4;
  constexpr float kScale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(d)
  float4v s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, p.k[kk]),
                                                 __builtin_bit_cast(bf16x8v, q.w[kk]), s, 0, 0, 0);
  float lg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lg[i] = (4 * b + i < nvalid) ? s[i] * kScale : -__builtin_inff();
  const float pm = xrow_max(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])));
  const float mn = fmaxf(a.m, pm);  // finite
  const float alpha = __builtin_amdgcn_exp2f(a.m - mn);
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(lg[i] - mn);
  // the sum in fp32; P^T goes to the matrix cores in bf16 (nearest)
  const float ps = xrow_sum((pr[0] + pr[1]) + (pr[2] + pr[3]));
  const bf16x2v p01 = {(__bf16)pr[0], (__bf16)pr[1]}, p23 = {(__bf16)pr[2], (__bf16)pr[3]};
  const uint32_t w01 = __builtin_bit_cast(uint32_t, p01), w23 = __builtin_bit_cast(uint32_t, p23);
  a.l = a.l * alpha + ps;
  a.m = mn;
  const short4v pb = __builtin_bit_cast(short4v, make_uint2(w01, w23));
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    // element t of value rows 4 b .. 4 b + 3 (dim 8 c + t), as bf16 pairs
    const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t a01 = __builtin_amdgcn_perm(word_of(p.v[1], t >> 1), word_of(p.v[0], t >> 1), sel);
    const uint32_t a23 = __builtin_amdgcn_perm(word_of(p.v[3], t >> 1), word_of(p.v[2], t >> 1), sel);
    a.acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, make_uint2(a01, a23)), pb,
                                                         a.acc[t] * alpha, 0, 0, 0);
  }
}

// Streams up to kMax pages. page_at(i, off, nvalid) gives the pool element
// offset of the wave's i-th page (or off < 0 to skip it) and its live tokens.
template <int kMax, typename PageAt>
__device__ __forceinline__ void attn_wave_pages(AttnAcc& a, const AttnQ& qw,
                                                const uint16_t* __restrict__ kpool,
                                                const uint16_t* __restrict__ vpool, int cnt,
                                                PageAt page_at, int lane) {
  int64_t off[kMax];
  int nv[kMax];
#pragma unroll
  for (int i = 0; i < kMax; ++i) {
    off[i] = -1;
    nv[i] = 0;
    if (i < cnt) page_at(i, off[i], nv[i]);
  }
  PageRegs cur, nxt;
  if (cnt > 0 && off[0] >= 0) attn_load_page(cur, kpool, vpool, off[0], lane);
#pragma unroll
  for (int i = 0; i < kMax; ++i) {
    if (i >= cnt) break;
    if (i + 1 < kMax && i + 1 < cnt && off[i + 1 < kMax ? i + 1 : i] >= 0)
      attn_load_page(nxt, kpool, vpool, off[i + 1 < kMax ? i + 1 : i], lane);
    if (off[i] >= 0) attn_page(a, cur, qw, nv[i], lane);
    cur = nxt;
  }
}

// Leaves the wave's partial in LDS: acc[G][128] and (m, l) per query.
template <int G>
__device__ __forceinline__ void attn_wave_to_lds(const AttnAcc& a, float (*sh_acc)[kHeadDim],
                                                 float (*sh_ml)[2], int lane) {
  const int c = lane & 15, b = lane >> 4;
  if (c < G) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* d = &sh_acc[c][32 * b + 8 * i];
      *reinterpret_cast<float4*>(d) = make_float4(a.acc[0][i], a.acc[1][i], a.acc[2][i], a.acc[3][i]);
      *reinterpret_cast<float4*>(d + 4) = make_float4(a.acc[4][i], a.acc[5][i], a.acc[6][i], a.acc[7][i]);
    }
    if (b == 0) {
      sh_ml[c][0] = a.m;
      sh_ml[c][1] = a.l;
    }
  }
}

// Combines the partials of nw waves held in LDS into one workgroup partial
// at dst ([G][kPartStride]). Called by one whole wave: lane = 16 g + c
// handles dims 8c..8c+7 of query g.
template <int G>
__device__ __forceinline__ void wg_partial_store(const float (*sh_acc)[G][kHeadDim],
                                                 const float (*sh_ml)[G][2], int nw, float* dst,
                                                 int lane) {
  if (lane >= G * 16) return;
  const int g = lane >> 4, d0 = 8 * (lane & 15);
  float M = -__builtin_inff();
  for (int w = 0; w < nw; ++w) M = fmaxf(M, sh_ml[w][g][0]);
  float a[8], L = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = 0.f;
  for (int w = 0; w < nw; ++w) {
    const float f = (M == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(sh_ml[w][g][0] - M);
    L += f * sh_ml[w][g][1];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] += f * sh_acc[w][g][d0 + e];
  }
  float* p = dst + g * kPartStride;
  *reinterpret_cast<float4*>(p + d0) = make_float4(a[0], a[1], a[2], a[3]);
  *reinterpret_cast<float4*>(p + d0 + 4) = make_float4(a[4], a[5], a[6], a[7]);
  if ((lane & 15) == 0) *reinterpret_cast<float2*>(p + kHeadDim) = make_float2(M, L);
}

// Base-2 online merge of (m, l) states: returns the factor for the old
// state and sets f2 for the incoming one (both 0 when everything is empty).
// Branch-free, so loads feeding a chain of merges can all be in flight.
__device__ __forceinline__ float merge_factors(float& m, float m2, float& f2) {
  const float M = fmaxf(m, m2);
  const bool empty = (M == -__builtin_inff());
  const float f1 = empty ? 0.f : __builtin_amdgcn_exp2f(m - M);
  f2 = empty ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
  m = M;
  return f1;
}

}  // namespace locks
