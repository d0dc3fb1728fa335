// LOCKS sparse decode attention over the selected pages only (gfx950).
//
// [N] = LOCKS reading notes (zhongzhuzhou.org 2026-07-29), §4.4 Algorithm 2
// (last steps) and §3.1 eq. 1: every query head of a GQA group attends, with
// ordinary softmax renormalised over S, to the full K/V of the pages in S.
//
// Split-K flash decoding. A workgroup of 4 waves takes 4 * PPW consecutive
// entries of the (sequence, KV head) selection list; each wave streams PPW
// pages with an online softmax, the 4 waves merge in LDS, and the workgroup
// writes one partial (max, sum, accumulator[G][d]) to the workspace. A second
// kernel merges the partials of each (sequence, KV head) in split order, so
// the result does not depend on scheduling. (Merging inside the first kernel
// would need agent-scope release/acquire fences, which on the multi-XCD
// MI355X write back and invalidate a whole L2 per workgroup.)
//
// Lane roles inside a wave for one 16 x 128 page:
//   QK: lane = 4 t + c reads 64 contiguous bytes of key row t (dims 32c..),
//       so the wave reads the 4 KB key page in one coalesced sweep, and forms
//       q_g . k_t with v_dot2c_f32_bf16 plus one quad butterfly.
//   PV: lane = 16 ts + dg holds dims 8 dg.. of value rows ts, ts+4, ts+8,
//       ts+12 (also one coalesced 4 KB sweep) and accumulates p_t v_t.
#include "locks_device.h"

namespace locks {

constexpr int kAttnWaves = 4;
constexpr int kAttnMaxSplits = 128;  // host raises pages per wave to stay within this

template <int G>
__global__ __launch_bounds__(256) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kpool,
    const uint16_t* __restrict__ vpool, const int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, float* __restrict__ part, int64_t num_blocks, int H,
    int MP, int max_budget, int nsplit, int ppw) {
  constexpr int kPart = G * (kHeadDim + 2);
  __shared__ float sh_acc[kAttnWaves][G][kHeadDim];
  __shared__ float sh_ml[kAttnWaves][G][2];

  const int s = blockIdx.z, h = blockIdx.y, x = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t sh_idx = (int64_t)s * H + h;
  const int len = clampi(seq_lens[s], 0, MP * kPage);
  const int P = (len + kPage - 1) / kPage;
  const int n = clampi(cnt[sh_idx], 0, max_budget);
  const int per_wg = kAttnWaves * ppw;
  const int nact = (n + per_wg - 1) / per_wg;
  if (x >= nact) return;

  // ---- query registers for the QK role: dims [32c, 32c+32) as bf16 pairs
  const int t_qk = lane >> 2, c_qk = lane & 3;
  const int ts = lane >> 4, dg = lane & 15;
  uint32_t qw[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4* qp = reinterpret_cast<const uint4*>(
        q + ((sh_idx * G + g) * kHeadDim) + 32 * c_qk);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint4 w = qp[e];
      qw[g][4 * e + 0] = w.x; qw[g][4 * e + 1] = w.y; qw[g][4 * e + 2] = w.z; qw[g][4 * e + 3] = w.w;
    }
  }
  const float qk_scale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(d)

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -__builtin_inff();
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  const int32_t* sel_row = sel + sh_idx * max_budget;
  for (int pi = 0; pi < ppw; ++pi) {
    const int idx = x * per_wg + wave * ppw + pi;
    if (idx >= n) break;
    const int j = sel_row[idx];
    if (j < 0 || j >= P) continue;
    const int blk = table[(int64_t)s * MP + j];
    if (blk < 0 || blk >= num_blocks) continue;
    const int nvalid = (j == P - 1) ? len - kPage * (P - 1) : kPage;
    const int64_t page_off = ((int64_t)blk * H + h) * (kPage * kHeadDim);
    const uint8_t* kb = reinterpret_cast<const uint8_t*>(kpool + page_off);
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(vpool + page_off);

    uint4 kw[4], vw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      kw[e] = *reinterpret_cast<const uint4*>(kb + t_qk * 256 + 64 * c_qk + 16 * e);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      vw[e] = *reinterpret_cast<const uint4*>(vb + (ts + 4 * e) * 256 + 16 * dg);

    // ---- logits (log2 units) of token t_qk for every query of the group
    float lg[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kk[4] = {kw[e].x, kw[e].y, kw[e].z, kw[e].w};
#pragma unroll
        for (int f = 0; f < 4; ++f)
          a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, kk[f]),
                                              __builtin_bit_cast(bf16x2v, qw[g][4 * e + f]), a,
                                              false);
      }
      lg[g] = quad_sum(a) * qk_scale;
      if (t_qk >= nvalid) lg[g] = -__builtin_inff();
    }
    // ---- online softmax over the page's tokens
    float pv[G][4];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float pm = lg[g];
      pm = fmaxf(pm, shfl_xor(pm, 4));
      pm = fmaxf(pm, shfl_xor(pm, 8));
      pm = fmaxf(pm, shfl_xor(pm, 16));
      pm = fmaxf(pm, shfl_xor(pm, 32));
      const float mn = fmaxf(m[g], pm);
      const float alpha = __builtin_amdgcn_exp2f(m[g] - mn);
      const float pt = __builtin_amdgcn_exp2f(lg[g] - mn);
      float ps = pt;
      ps += shfl_xor(ps, 4);
      ps += shfl_xor(ps, 8);
      ps += shfl_xor(ps, 16);
      ps += shfl_xor(ps, 32);
      l[g] = l[g] * alpha + ps;
      m[g] = mn;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[g][e] = __shfl(pt, 4 * (ts + 4 * e), 64);
    }
    // ---- p . V for the lane's 4 value rows and 8 dims
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t vv[4] = {vw[e].x, vw[e].y, vw[e].z, vw[e].w};
      float v8[8];
#pragma unroll
      for (int f = 0; f < 4; ++f) { v8[2 * f] = bf16_lo(vv[f]); v8[2 * f + 1] = bf16_hi(vv[f]); }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int f = 0; f < 8; ++f) acc[g][f] = fmaf(pv[g][e], v8[f], acc[g][f]);
    }
  }

  // ---- wave partial: sum the 4 row groups, then merge the 4 waves in LDS
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      float v = acc[g][f];
      v += shfl_xor(v, 16);
      v += shfl_xor(v, 32);
      acc[g][f] = v;
    }
  if (ts == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int f = 0; f < 8; ++f) sh_acc[wave][g][8 * dg + f] = acc[g][f];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) { sh_ml[wave][g][0] = m[g]; sh_ml[wave][g][1] = l[g]; }
  }
  __syncthreads();

  float* my_part = part + (sh_idx * nsplit + x) * kPart;
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) {
    const int g = i / kHeadDim, d = i % kHeadDim;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sh_ml[w][g][0]);
    float a = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float f = (M == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(sh_ml[w][g][0] - M);
      a += f * sh_acc[w][g][d];
      L += f * sh_ml[w][g][1];
    }
    my_part[g * (kHeadDim + 2) + d] = a;
    if (d == 0) {
      my_part[g * (kHeadDim + 2) + kHeadDim] = M;
      my_part[g * (kHeadDim + 2) + kHeadDim + 1] = L;
    }
  }

}

// Merge of the split partials of one (sequence, KV head) per workgroup, in
// split order; empty selections give out = 0 and lse = -inf.
template <int G>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const int32_t* __restrict__ cnt, const float* __restrict__ part, float* __restrict__ out,
    float* __restrict__ lse_out, int H, int max_budget, int nsplit, int ppw) {
  constexpr int kPart = G * (kHeadDim + 2);
  __shared__ float sh_f[kAttnMaxSplits * G];  // per split and query: max, then merge factor
  __shared__ float sh_l[kAttnMaxSplits * G];  // per split and query: sum
  __shared__ float sh_M[2 * G];               // global max and total sum per query
  const int64_t sh_idx = (int64_t)blockIdx.y * H + blockIdx.x;
  const int tid = threadIdx.x;
  const int n = clampi(cnt[sh_idx], 0, max_budget);
  const int nact = min((n + kAttnWaves * ppw - 1) / (kAttnWaves * ppw), nsplit);
  float* o_base = out + (sh_idx * G) * kHeadDim;
  if (nact == 0) {
    for (int i = tid; i < G * kHeadDim; i += blockDim.x) o_base[i] = 0.f;
    if (lse_out && tid < G) lse_out[sh_idx * G + tid] = -__builtin_inff();
    return;
  }
  const float* parts = part + sh_idx * nsplit * kPart;
  // per-split maxima and sums -> LDS (all loads independent)
  for (int i = tid; i < nact * G; i += blockDim.x) {
    const int y = i / G, g = i % G;
    const float* py = parts + y * kPart + g * (kHeadDim + 2) + kHeadDim;
    sh_f[i] = py[0];
    sh_l[i] = py[1];
  }
  __syncthreads();
  if (tid < G) {
    float M = -__builtin_inff();
    for (int y = 0; y < nact; ++y) M = fmaxf(M, sh_f[y * G + tid]);
    float Lsum = 0.f;
    for (int y = 0; y < nact; ++y) {
      const float f = (M == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(sh_f[y * G + tid] - M);
      sh_f[y * G + tid] = f;
      Lsum += f * sh_l[y * G + tid];
    }
    sh_M[tid] = M;
    sh_M[G + tid] = Lsum;
  }
  __syncthreads();
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) {
    const int g = i / kHeadDim, d = i % kHeadDim;
    float a = 0.f;
#pragma unroll 8
    for (int y = 0; y < nact; ++y) a += sh_f[y * G + g] * parts[y * kPart + g * (kHeadDim + 2) + d];
    const float Lsum = sh_M[G + g];
    o_base[g * kHeadDim + d] = (Lsum > 0.f) ? a / Lsum : 0.f;
    if (lse_out && d == 0)
      lse_out[sh_idx * G + g] =
          (Lsum > 0.f) ? (sh_M[g] + __builtin_amdgcn_logf(Lsum)) * kLn2 : -__builtin_inff();
  }
}

hipError_t launch_attn(int G, const void* q, const void* kpool, const void* vpool,
                       const int32_t* table, const int32_t* lens, const int32_t* sel,
                       const int32_t* cnt, float* part, float* out, float* lse_out, int64_t nb,
                       int S, int H, int MP, int max_budget, int nsplit, int ppw, hipStream_t st) {
  dim3 grid(nsplit, H, S), mgrid(H, S);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(kpool);
  const uint16_t* vv = static_cast<const uint16_t*>(vpool);
  switch (G) {
#define LOCKS_G(GG)                                                                               \
  case GG:                                                                                        \
    hipLaunchKernelGGL(attn_kernel<GG>, grid, dim3(64 * kAttnWaves), 0, st, qq, kk, vv, table,   \
                       lens, sel, cnt, part, nb, H, MP, max_budget, nsplit, ppw);                 \
    hipLaunchKernelGGL(attn_merge_kernel<GG>, mgrid, dim3(256), 0, st, cnt, part, out, lse_out,  \
                       H, max_budget, nsplit, ppw);                                               \
    break;
    LOCKS_G(1) LOCKS_G(2) LOCKS_G(4)
#undef LOCKS_G
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace locks
