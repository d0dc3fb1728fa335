// Wave-level flash-decoding core over 16 x 128 bf16 KV pages (gfx950).
//
// Lane roles inside a wave for one page:
//   QK: lane = 4 t + c reads 64 contiguous bytes of key row t (dims 32c..),
//       so the wave reads the 4 KB key page in one coalesced sweep, and forms
//       q_g . k_t with v_dot2c_f32_bf16 plus one quad butterfly.
//   PV: lane = 16 ts + dg holds dims 8 dg.. of value rows ts, ts+4, ts+8,
//       ts+12 (also one coalesced 4 KB sweep) and accumulates p_t v_t.
// A wave streams its pages with an online softmax (base-2 logits); the block
// ids of all its pages are read up front and the K/V of the next page load
// while the current page is computed.
#pragma once

#include "locks_device.h"

namespace locks {

// A workgroup partial holds, per query, acc[128] then (max, sum) and 2 pad
// floats, so every query row starts 16-byte aligned.
constexpr int kPartStride = kHeadDim + 4;

template <int G>
struct AttnAcc {
  float m[G], l[G], acc[G][8];
};

struct PageRegs {
  uint4 k[4], v[4];
};

template <int G>
__device__ __forceinline__ void attn_init(AttnAcc<G>& a) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    a.m[g] = -__builtin_inff();
    a.l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a.acc[g][e] = 0.f;
  }
}

// Query registers for the QK role: dims [32c, 32c+32) of each of the G
// queries (row-major G x 128 bf16 at qg) as bf16 pairs.
template <int G>
__device__ __forceinline__ void attn_load_q(uint32_t (&qw)[G][16], const uint16_t* qg, int lane) {
  const int c = lane & 3;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4* qp = reinterpret_cast<const uint4*>(qg + g * kHeadDim + 32 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint4 w = qp[e];
      qw[g][4 * e + 0] = w.x;
      qw[g][4 * e + 1] = w.y;
      qw[g][4 * e + 2] = w.z;
      qw[g][4 * e + 3] = w.w;
    }
  }
}

// K/V of the page at element offset `off` of the pools (16 x 128 bf16 each).
__device__ __forceinline__ void attn_load_page(PageRegs& p, const uint16_t* __restrict__ kpool,
                                               const uint16_t* __restrict__ vpool, int64_t off,
                                               int lane) {
  const int t = lane >> 2, c = lane & 3, ts = lane >> 4, dg = lane & 15;
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(kpool + off);
  const uint8_t* vb = reinterpret_cast<const uint8_t*>(vpool + off);
#pragma unroll
  for (int e = 0; e < 4; ++e) p.k[e] = *reinterpret_cast<const uint4*>(kb + t * 256 + 64 * c + 16 * e);
#pragma unroll
  for (int e = 0; e < 4; ++e) p.v[e] = *reinterpret_cast<const uint4*>(vb + (ts + 4 * e) * 256 + 16 * dg);
}

// Online-softmax update with one page whose first `nvalid` tokens are live.
template <int G>
__device__ __forceinline__ void attn_page(AttnAcc<G>& a, const PageRegs& p,
                                          const uint32_t (&qw)[G][16], int nvalid, int lane) {
  const int t_qk = lane >> 2, ts = lane >> 4;
  const float qk_scale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(d)
  float lg[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t kk[4] = {p.k[e].x, p.k[e].y, p.k[e].z, p.k[e].w};
#pragma unroll
      for (int f = 0; f < 4; ++f)
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, kk[f]),
                                            __builtin_bit_cast(bf16x2v, qw[g][4 * e + f]), s, false);
    }
    lg[g] = quad_sum(s) * qk_scale;
    if (t_qk >= nvalid) lg[g] = -__builtin_inff();
  }
  float pv[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float pm = lg[g];
    pm = fmaxf(pm, shfl_xor(pm, 4));
    pm = fmaxf(pm, shfl_xor(pm, 8));
    pm = fmaxf(pm, shfl_xor(pm, 16));
    pm = fmaxf(pm, shfl_xor(pm, 32));
    const float mn = fmaxf(a.m[g], pm);  // finite: token 0 of a page is always live
    const float alpha = __builtin_amdgcn_exp2f(a.m[g] - mn);
    const float pt = __builtin_amdgcn_exp2f(lg[g] - mn);
    float ps = pt;
    ps += shfl_xor(ps, 4);
    ps += shfl_xor(ps, 8);
    ps += shfl_xor(ps, 16);
    ps += shfl_xor(ps, 32);
    a.l[g] = a.l[g] * alpha + ps;
    a.m[g] = mn;
#pragma unroll
    for (int e = 0; e < 8; ++e) a.acc[g][e] *= alpha;
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[g][e] = __shfl(pt, 4 * (ts + 4 * e), 64);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t vv[4] = {p.v[e].x, p.v[e].y, p.v[e].z, p.v[e].w};
    float v8[8];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      v8[2 * f] = bf16_lo(vv[f]);
      v8[2 * f + 1] = bf16_hi(vv[f]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int f = 0; f < 8; ++f) a.acc[g][f] = fmaf(pv[g][e], v8[f], a.acc[g][f]);
  }
}

// Streams up to kMax pages. page_at(i, off, nvalid) gives the pool element
// offset of the wave's i-th page (or off < 0 to skip it) and its live tokens.
template <int G, int kMax, typename PageAt>
__device__ __forceinline__ void attn_wave_pages(AttnAcc<G>& a, const uint32_t (&qw)[G][16],
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
    if (off[i] >= 0) attn_page<G>(a, cur, qw, nv[i], lane);
    cur = nxt;
  }
}

// Sums the 4 value-row groups of the wave and leaves the wave's partial in
// LDS: acc[G][128] and (m, l) per query.
template <int G>
__device__ __forceinline__ void attn_wave_to_lds(AttnAcc<G>& a, float (*sh_acc)[kHeadDim],
                                                 float (*sh_ml)[2], int lane) {
  const int ts = lane >> 4, dg = lane & 15;
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      float v = a.acc[g][f];
      v += shfl_xor(v, 16);
      v += shfl_xor(v, 32);
      a.acc[g][f] = v;
    }
  if (ts == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      *reinterpret_cast<float4*>(&sh_acc[g][8 * dg]) =
          make_float4(a.acc[g][0], a.acc[g][1], a.acc[g][2], a.acc[g][3]);
      *reinterpret_cast<float4*>(&sh_acc[g][8 * dg + 4]) =
          make_float4(a.acc[g][4], a.acc[g][5], a.acc[g][6], a.acc[g][7]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sh_ml[g][0] = a.m[g];
      sh_ml[g][1] = a.l[g];
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
