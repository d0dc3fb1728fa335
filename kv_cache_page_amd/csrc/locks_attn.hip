// LOCKS sparse decode attention over the selected pages only (gfx950).
//
// [N] = LOCKS reading notes (zhongzhuzhou.org 2026-07-29), §4.4 Algorithm 2
// (last steps) and §3.1 eq. 1: every query head of a GQA group attends, with
// ordinary softmax renormalised over S, to the full K/V of the pages in S.
//
// Split-K flash decoding. A workgroup of 4 waves takes 4 * PPW consecutive
// entries of the (sequence, KV head) selection list; each wave streams PPW
// pages with an online softmax, the 4 waves merge in LDS, and the workgroup
// writes one partial (acc[G][d], max, sum) to the workspace. A second kernel
// merges the partials of each (sequence, KV head) in split order, so the
// result does not depend on scheduling.
#include "locks_attn_core.h"

namespace locks {

constexpr int kAttnWaves = 4;
constexpr int kAttnMaxSplits = 128;  // host raises pages per wave to stay within this
constexpr int kAttnChunk = 8;        // pages a wave keeps in flight per chunk

template <int G>
__global__ __launch_bounds__(64 * kAttnWaves) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kpool,
    const uint16_t* __restrict__ vpool, const int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, float* __restrict__ part, int64_t num_blocks, int H,
    int MP, int max_budget, int nsplit, int ppw, int hdiv) {
  __shared__ float sh_acc[kAttnWaves][G][kHeadDim];
  __shared__ float sh_ml[kAttnWaves][G][2];

  const int h = blockIdx.x, x = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t sh_idx = (int64_t)s * H + h;
  const int len = clampi(seq_lens[s], 0, MP * kPage);
  const int P = (len + kPage - 1) / kPage;
  const int n = clampi(cnt[sh_idx], 0, max_budget);
  const int per_wg = kAttnWaves * ppw;
  const int nact = (n + per_wg - 1) / per_wg;
  if (x >= nact) return;

  AttnQ qw;
  attn_load_q<G>(qw, q + sh_idx * G * kHeadDim, lane);
  AttnAcc acc;
  attn_init(acc);
  const int32_t* row = sel + sh_idx * max_budget;
  const int base = x * per_wg + wave * ppw;
  const int mine = clampi(n - base, 0, ppw);
  for (int c0 = 0; c0 < mine; c0 += kAttnChunk) {
    auto page_at = [&](int i, int64_t& off, int& nv) {
      const int j = row[base + c0 + i];
      if (j < 0 || j >= P) return;
      const int blk = table[(int64_t)s * MP + j];
      if (blk < 0 || blk >= num_blocks) return;
      off = ((int64_t)blk * (H / hdiv) + h / hdiv) * (kPage * kHeadDim);  // the pools' head (score_head_div)
      nv = (j == P - 1) ? len - kPage * (P - 1) : kPage;
    };
    attn_wave_pages<kAttnChunk>(acc, qw, kpool, vpool, min(kAttnChunk, mine - c0), page_at,
                                   lane);
  }
  attn_wave_to_lds<G>(acc, sh_acc[wave], sh_ml[wave], lane);
  __syncthreads();
  if (wave == 0)
    wg_partial_store<G>(sh_acc, sh_ml, kAttnWaves, part + (sh_idx * nsplit + x) * G * kPartStride,
                        lane);
}

// Merge of the split partials of one (sequence, KV head) per workgroup, in
// split order; empty selections give out = 0 and lse = -inf.
template <int G>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const int32_t* __restrict__ cnt, const float* __restrict__ part, float* __restrict__ out,
    float* __restrict__ lse_out, int H, int max_budget, int nsplit, int ppw) {
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
  const float* parts = part + sh_idx * nsplit * G * kPartStride;
  for (int i = tid; i < nact * G; i += blockDim.x) {
    const float2 ml = *reinterpret_cast<const float2*>(parts + i * kPartStride + kHeadDim);
    sh_f[i] = ml.x;
    sh_l[i] = ml.y;
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
    for (int y = 0; y < nact; ++y) a += sh_f[y * G + g] * parts[(y * G + g) * kPartStride + d];
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
                       int S, int H, int MP, int max_budget, int nsplit, int ppw, int hdiv,
                       hipStream_t st) {
  if (hdiv < 1 || H % hdiv != 0) return hipErrorInvalidValue;
  dim3 grid(H, nsplit, S), mgrid(H, S);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(kpool);
  const uint16_t* vv = static_cast<const uint16_t*>(vpool);
  switch (G) {
#define LOCKS_G(GG)                                                                               \
  case GG:                                                                                        \
    hipLaunchKernelGGL(attn_kernel<GG>, grid, dim3(64 * kAttnWaves), 0, st, qq, kk, vv, table,   \
                       lens, sel, cnt, part, nb, H, MP, max_budget, nsplit, ppw, hdiv);           \
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
