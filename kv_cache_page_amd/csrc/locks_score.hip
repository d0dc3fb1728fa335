// LOCKS page scoring and page selection kernels (gfx950).
//
// Score ([N] = LOCKS reading notes, zhongzhuzhou.org 2026-07-29, §4.2 eq. 4):
//   s_hat_j(q_g) = LSE_i ((q_g . mu_j + (V_j^T q_g) . c_i) / sqrt(d))
// computed from the summary slot only. Shares and selection (§4.2 eq. 5 and
// §4.4 Algorithm 2): Z_g = LSE_j s_hat_jg, key_j = log mean_g exp(s_hat_jg -
// Z_g), S = {0, P-1} + top-(k-2) keys among pages 1..P-2 (lower page first on
// equal keys).
//
// Score kernel mapping. Four lanes (a quad) share one page; lane l4 of the
// quad owns dims [32*l4, 32*l4 + 32) of the centroid and of every basis
// column, and tokens [4*l4, 4*l4 + 4) of the coefficients. The group's G
// queries stay in registers for the whole kernel, pre-scaled by a power of two
// and stored as fp16 pairs. Basis nibbles (xor 8 -> offset-binary 0..15) and
// centroid bytes (xor 0x80 -> 0..255) become fp16 denormals (n * 2^-24) with
// one AND per pair, and v_dot2c_f32_f16 accumulates n * q exactly-rounded in
// fp32; the offsets (8 and 128 times sum q) are subtracted through the
// accumulator's initial value. One quad butterfly completes V^T q and q . mu,
// then each lane forms the logits of its four tokens and a second quad
// reduction finishes the length-16 log-sum-exp.
#include "locks_device.h"

namespace locks {

// ---------------------------------------------------------------------------
// score
// ---------------------------------------------------------------------------
template <int R, int G>
__global__ __launch_bounds__(256) void score_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ summ,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, int64_t num_blocks, int H, int MP, int pages_per_wg,
    int fill_nan) {
  constexpr SlotLayout L = slot_layout(R);
  constexpr float kTwoM24 = 5.9604644775390625e-08f;  // 2^-24
  const int s = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l4 = lane & 3;
  const int len = clampi(seq_lens[s], 0, MP * kPage);
  const int F = len / kPage;
  const int j_lo = blockIdx.x * pages_per_wg;
  const int j_hi = min(j_lo + pages_per_wg, MP);
  float* srow = scores + ((int64_t)s * H + h) * MP * G;
  if (fill_nan) {
    const int first = max(j_lo, F);
    for (int idx = threadIdx.x; idx < (j_hi - first) * G; idx += blockDim.x)
      srow[(int64_t)first * G + idx] = __builtin_nanf("");
  }
  if (j_lo >= F) return;
  const int j_end = min(j_hi, F);

  // ---- queries of the group: lane's 32 dims, power-of-two scaled fp16 pairs
  half2v Q[G][4][4];
  float vinit[G], minit[G], fscale[G];
  for (int g = 0; g < G; ++g) {
    const uint4* qp = reinterpret_cast<const uint4*>(
        q + ((int64_t)s * H * G + (int64_t)h * G + g) * kHeadDim + 32 * l4);
    float x[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 w = qp[c];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * c + 2 * e] = bf16_lo(ww[e]);
        x[8 * c + 2 * e + 1] = bf16_hi(ww[e]);
      }
    }
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) mx = fmaxf(mx, fabsf(x[e]));
    mx = quad_max(mx);
    const int ex = (mx > 0.f && mx < __builtin_inff()) ? ilogbf(mx) : 0;
    const float up = ldexpf(1.f, 14 - ex);  // max |q| * up < 2^15
    float qs = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) qs += x[e] * up;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float* y = x + 8 * t;
      Q[g][t][0] = half2v{(_Float16)(y[0] * up), (_Float16)(y[2] * up)};
      Q[g][t][1] = half2v{(_Float16)(y[1] * up * 0.0625f), (_Float16)(y[3] * up * 0.0625f)};
      Q[g][t][2] = half2v{(_Float16)(y[4] * up), (_Float16)(y[6] * up)};
      Q[g][t][3] = half2v{(_Float16)(y[5] * up * 0.0625f), (_Float16)(y[7] * up * 0.0625f)};
    }
    vinit[g] = -8.f * kTwoM24 * qs;
    minit[g] = -128.f * kTwoM24 * qs;
    // logits in log2 units: 2^(24 - (14 - ex)) * log2(e) / sqrt(d)
    fscale[g] = ldexpf(kLog2e * 0.08838834764831845f, 10 + ex);
  }

  for (int jb = j_lo + wave * 16; jb < j_end; jb += 64) {
    const int j = jb + (lane >> 2);
    const bool in = j < j_end;
    const int blk = in ? table[(int64_t)s * MP + j] : 0;
    const bool ok = in && blk >= 0 && blk < num_blocks;
    const uint8_t* slot = static_cast<const uint8_t*>(__builtin_assume_aligned(
        summ + ((int64_t)(ok ? blk : 0) * H + h) * L.stride, 16));

    uint4 vq[R];
#pragma unroll
    for (int k = 0; k < R; ++k) vq[k] = *reinterpret_cast<const uint4*>(slot + 64 * k + 16 * l4);
    const uint4 mq0 = *reinterpret_cast<const uint4*>(slot + L.mu + 32 * l4);
    const uint4 mq1 = *reinterpret_cast<const uint4*>(slot + L.mu + 32 * l4 + 16);
    uint32_t cq[R];
#pragma unroll
    for (int e = 0; e < R; ++e)
      cq[e] = *reinterpret_cast<const uint32_t*>(slot + L.c + 4 * R * l4 + 4 * e);
    uint16_t sv[R];
#pragma unroll
    for (int k = 0; k < R; ++k) sv[k] = *reinterpret_cast<const uint16_t*>(slot + L.sv + 2 * k);
    uint16_t scw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      scw[i] = *reinterpret_cast<const uint16_t*>(slot + L.sc + 8 * l4 + 2 * i);
    const uint16_t smw = *reinterpret_cast<const uint16_t*>(slot + L.smu);

    // ---- V^T q (partial over the lane's 32 dims)
    float acc[R][G];
#pragma unroll
    for (int k = 0; k < R; ++k) {
#pragma unroll
      for (int g = 0; g < G; ++g) acc[k][g] = vinit[g];
      const uint32_t words[4] = {vq[k].x, vq[k].y, vq[k].z, vq[k].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t w = words[t] ^ 0x88888888u;
        const uint32_t w8 = w >> 8;
        const half2v p0 = __builtin_bit_cast(half2v, w & 0x000F000Fu);
        const half2v p1 = __builtin_bit_cast(half2v, w & 0x00F000F0u);
        const half2v p2 = __builtin_bit_cast(half2v, w8 & 0x000F000Fu);
        const half2v p3 = __builtin_bit_cast(half2v, w8 & 0x00F000F0u);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float a = acc[k][g];
          a = __builtin_amdgcn_fdot2(p0, Q[g][t][0], a, false);
          a = __builtin_amdgcn_fdot2(p1, Q[g][t][1], a, false);
          a = __builtin_amdgcn_fdot2(p2, Q[g][t][2], a, false);
          a = __builtin_amdgcn_fdot2(p3, Q[g][t][3], a, false);
          acc[k][g] = a;
        }
      }
    }
    // ---- q . mu (partial)
    float a1[G], a16[G];
#pragma unroll
    for (int g = 0; g < G; ++g) { a1[g] = minit[g]; a16[g] = 0.f; }
    {
      const uint32_t mw[8] = {mq0.x, mq0.y, mq0.z, mq0.w, mq1.x, mq1.y, mq1.z, mq1.w};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t w = mw[m] ^ 0x80808080u;
        const half2v e0 = __builtin_bit_cast(half2v, w & 0x00FF00FFu);
        const half2v e1 = __builtin_bit_cast(half2v, (w >> 8) & 0x00FF00FFu);
        const int t = m >> 1, o = (m & 1) * 2;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          a1[g] = __builtin_amdgcn_fdot2(e0, Q[g][t][o], a1[g], false);
          a16[g] = __builtin_amdgcn_fdot2(e1, Q[g][t][o + 1], a16[g], false);
        }
      }
    }
    // ---- finish the dot products across the quad
    float A[G];
    const float smu = (float)__builtin_bit_cast(_Float16, smw);
#pragma unroll
    for (int g = 0; g < G; ++g) A[g] = quad_sum(fmaf(16.f, a16[g], a1[g])) * smu;
    float p[R][G];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const float svk = (float)__builtin_bit_cast(_Float16, sv[k]);
#pragma unroll
      for (int g = 0; g < G; ++g) p[k][g] = quad_sum(acc[k][g]) * svk;
    }
    // ---- logits of the lane's 4 tokens, LSE over the page's 16
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = (float)__builtin_bit_cast(_Float16, scw[i]);
    float lg[4][G];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float cf[R];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int byte = i * R + k;
        cf[k] = (float)(int8_t)(cq[byte >> 2] >> (8 * (byte & 3)));
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float x = 0.f;
#pragma unroll
        for (int k = 0; k < R; ++k) x = fmaf(p[k][g], cf[k], x);
        lg[i][g] = fscale[g] * fmaf(sc[i], x, A[g]);
      }
    }
    float outv = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float m = fmaxf(fmaxf(lg[0][g], lg[1][g]), fmaxf(lg[2][g], lg[3][g]));
      m = quad_max(m);
      float e = __builtin_amdgcn_exp2f(lg[0][g] - m) + __builtin_amdgcn_exp2f(lg[1][g] - m) +
                __builtin_amdgcn_exp2f(lg[2][g] - m) + __builtin_amdgcn_exp2f(lg[3][g] - m);
      e = quad_sum(e);
      const float shat = (m + __builtin_amdgcn_logf(e)) * kLn2;
      if (l4 == g) outv = shat;
    }
    if (in && l4 < G) srow[(int64_t)j * G + l4] = ok ? outv : -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------
// block-wide helpers for 1024-thread workgroups
// ---------------------------------------------------------------------------
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

// Histogram increment with wave aggregation of repeated digits: the first
// few distinct digits of the wave are counted with one LDS atomic each, the
// remaining lanes add individually.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t digit, bool act) {
  const int lane = threadIdx.x & 63;
  unsigned long long live = __ballot(act);
#pragma unroll 1
  for (int it = 0; it < 4 && live; ++it) {
    const int leader = __ffsll(live) - 1;
    const uint32_t d0 = __shfl((int)digit, leader, 64);
    const bool same = act && digit == d0;
    const unsigned long long grp = __ballot(same);
    if (lane == leader) atomicAdd(&hist[d0], (uint32_t)__popcll(grp));
    if (same) act = false;
    live &= ~grp;
  }
  if (act) atomicAdd(&hist[digit], 1u);
}

// ---------------------------------------------------------------------------
// select: one 1024-thread workgroup per (sequence, KV head)
// ---------------------------------------------------------------------------
constexpr int kSelectThreads = 1024;
constexpr int kSelectLdsPages = 12288;  // keys of up to this many pages live in LDS (48 KB)

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

// Online (max, sum-exp) merge: (m, s) absorbs (m2, s2).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -__builtin_inff()) return;
  s = s * __expf(m - M) + s2 * __expf(m2 - M);
  m = M;
}

template <int G, bool kLdsKeys>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ budgets, int32_t* __restrict__ sel_pages,
    int32_t* __restrict__ sel_count, uint32_t* __restrict__ keybuf, int H, int MP,
    int max_budget) {
  extern __shared__ uint32_t sh_keys[];
  __shared__ uint32_t hist[256];
  __shared__ float red_m[16][G], red_s[16][G];
  __shared__ int sh_waves[16];
  __shared__ int sh_pick[2];
  const int s = blockIdx.y, h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int nthr = kSelectThreads;
  const int len = clampi(seq_lens[s], 0, MP * kPage);
  const int P = (len + kPage - 1) / kPage;
  const int F = len / kPage;
  const int k = clampi(budgets[s], 2, max_budget);
  int32_t* out = sel_pages + ((int64_t)s * H + h) * max_budget;
  if (P == 0 || k >= P) {
    for (int i = tid; i < max_budget; i += nthr) out[i] = i < P ? i : -1;
    if (tid == 0) sel_count[(int64_t)s * H + h] = P;
    return;
  }
  // From here P >= 3, k < P and pages 0..P-2 are full (F >= P-1).
  const float* sc = scores + ((int64_t)s * H + h) * MP * G;
  uint32_t* ukey = kLdsKeys ? sh_keys : keybuf + ((int64_t)s * H + h) * MP;

  // ---- Z_g = LSE over the F summarised pages, one pass, 4 loads in flight
  float zm[G], zs[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { zm[g] = -__builtin_inff(); zs[g] = 0.f; }
  for (int j0 = tid; j0 < F; j0 += 4 * nthr) {
    float v[4][G];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * nthr;
      if (j < F) {
        load_scores<G>(sc + (int64_t)j * G, v[u]);
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) v[u][g] = -__builtin_inff();
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int g = 0; g < G; ++g) lse_merge(zm[g], zs[g], v[u][g], 1.f);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float m2 = __shfl_xor(zm[g], d, 64), s2 = __shfl_xor(zs[g], d, 64);
      lse_merge(zm[g], zs[g], m2, s2);
    }
    if (lane == 0) { red_m[wave][g] = zm[g]; red_s[wave][g] = zs[g]; }
  }
  __syncthreads();
  float logZ[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = red_m[0][g], t = red_s[0][g];
    for (int w = 1; w < nthr / 64; ++w) lse_merge(m, t, red_m[w][g], red_s[w][g]);
    logZ[g] = m + __logf(t);
  }

  // ---- key_j = log mean_g exp(s_hat_jg - Z_g) for candidates 1..P-2
  const float logG = __logf((float)G);
  for (int j0 = 1 + tid; j0 <= P - 2; j0 += 4 * nthr) {
    float v[4][G];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * nthr;
      if (j <= P - 2) load_scores<G>(sc + (int64_t)j * G, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * nthr;
      if (j > P - 2) continue;
      float d[G], m = -__builtin_inff();
#pragma unroll
      for (int g = 0; g < G; ++g) {
        d[g] = v[u][g] - logZ[g];
        m = fmaxf(m, d[g]);
      }
      float t = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) t += __expf(d[g] - m);
      float key = m + __logf(t) - logG;
      if (!(key == key) || m == -__builtin_inff()) key = -__builtin_inff();
      ukey[j] = float_to_ordered(key);
    }
  }
  __syncthreads();

  // ---- radix select of the (k-2)-th largest ordered key, 8 bits per pass
  uint32_t prefix = 0u, mask = 0u;
  int need = k - 2;
  if (need == 0) prefix = 0xFFFFFFFFu;  // k == 2: sink and recent only
  for (int shift = 24; shift >= 0 && need > 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    if (tid == 0) { sh_pick[0] = 0; sh_pick[1] = 0; }
    __syncthreads();
    for (int j0 = 1; j0 <= P - 2; j0 += nthr) {
      const int j = j0 + tid;
      const bool in = j <= P - 2;
      const uint32_t u = in ? ukey[j] : 0u;
      hist_add(hist, (u >> shift) & 255u, in && (u & mask) == prefix);
    }
    __syncthreads();
    // thread t < 256 handles digit 255 - t, so its inclusive prefix over t is
    // the count of keys whose digit is >= 255 - t
    int incl = 0;
    if (tid < 256) {
      incl = (int)hist[255 - tid];
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
      }
      if (lane == 63) sh_waves[wave] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < wave; ++w) incl += sh_waves[w];
      const int c = (int)hist[255 - tid];
      if (incl >= need && incl - c < need) {
        sh_pick[0] = 255 - tid;
        sh_pick[1] = incl - c;
      }
    }
    __syncthreads();
    const uint32_t D = (uint32_t)sh_pick[0];
    need -= sh_pick[1];
    prefix |= D << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;  // keys > T are in; `need` of the keys == T (lowest pages)

  // ---- mark and compact in ascending page order (contiguous chunk per thread)
  const int cpt = (P + nthr - 1) / nthr;  // pages per thread, <= 64
  const int c0 = tid * cpt, c1 = min(c0 + cpt, P);
  int eq = 0;
  for (int j = c0; j < c1; ++j)
    if (j >= 1 && j <= P - 2 && ukey[j] == T) ++eq;
  int tot;
  int eq_before = block_exclusive_scan(eq, sh_waves, &tot);
  unsigned long long bits = 0ull;
  int nsel = 0;
  for (int j = c0; j < c1; ++j) {
    bool take;
    if (j == 0 || j == P - 1) {
      take = true;
    } else {
      const uint32_t u = ukey[j];
      take = u > T || (u == T && eq_before++ < need);
    }
    if (take) { bits |= 1ull << (j - c0); ++nsel; }
  }
  int pos = block_exclusive_scan(nsel, sh_waves, &tot);
  tot = min(tot, max_budget);  // never more than k <= max_budget by construction
  for (int j = c0; j < c1; ++j)
    if ((bits >> (j - c0) & 1ull) && pos < max_budget) out[pos++] = j;
  for (int i = tot + tid; i < max_budget; i += nthr) out[i] = -1;
  if (tid == 0) sel_count[(int64_t)s * H + h] = tot;
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
template <int R, int G>
static hipError_t launch_score_rg(const uint16_t* q, const uint8_t* summ, const int32_t* table,
                                  const int32_t* lens, float* scores, int64_t nb, int S, int H,
                                  int MP, int fill_nan, hipStream_t st) {
  const int ppw = 128;
  dim3 grid((MP + ppw - 1) / ppw, H, S);
  hipLaunchKernelGGL((score_kernel<R, G>), grid, dim3(256), 0, st, q, summ, table, lens, scores,
                     nb, H, MP, ppw, fill_nan);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_score_g(int r, const uint16_t* q, const uint8_t* summ,
                                 const int32_t* table, const int32_t* lens, float* scores,
                                 int64_t nb, int S, int H, int MP, int fill_nan, hipStream_t st) {
  switch (r) {
#define LOCKS_R(RR) \
  case RR:          \
    return launch_score_rg<RR, G>(q, summ, table, lens, scores, nb, S, H, MP, fill_nan, st);
    LOCKS_R(1) LOCKS_R(2) LOCKS_R(3) LOCKS_R(4) LOCKS_R(5) LOCKS_R(6) LOCKS_R(7) LOCKS_R(8)
    LOCKS_R(9) LOCKS_R(10) LOCKS_R(11) LOCKS_R(12) LOCKS_R(13) LOCKS_R(14) LOCKS_R(15) LOCKS_R(16)
#undef LOCKS_R
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_score(int r, int G, const void* q, const void* summ, const int32_t* table,
                        const int32_t* lens, float* scores, int64_t nb, int S, int H, int MP,
                        int fill_nan, hipStream_t st) {
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint8_t* ss = static_cast<const uint8_t*>(summ);
  switch (G) {
    case 1: return launch_score_g<1>(r, qq, ss, table, lens, scores, nb, S, H, MP, fill_nan, st);
    case 2: return launch_score_g<2>(r, qq, ss, table, lens, scores, nb, S, H, MP, fill_nan, st);
    case 4: return launch_score_g<4>(r, qq, ss, table, lens, scores, nb, S, H, MP, fill_nan, st);
    default: return hipErrorInvalidValue;
  }
}

template <int G>
static void launch_select_g(dim3 grid, int MP, const float* scores, const int32_t* lens,
                            const int32_t* budgets, int32_t* sel, int32_t* cnt, uint32_t* keybuf,
                            int H, int max_budget, hipStream_t st) {
  if (MP <= kSelectLdsPages) {
    hipLaunchKernelGGL((select_kernel<G, true>), grid, dim3(kSelectThreads),
                       (size_t)MP * sizeof(uint32_t), st, scores, lens, budgets, sel, cnt, keybuf,
                       H, MP, max_budget);
  } else {
    hipLaunchKernelGGL((select_kernel<G, false>), grid, dim3(kSelectThreads), 0, st, scores, lens,
                       budgets, sel, cnt, keybuf, H, MP, max_budget);
  }
}

hipError_t launch_select(int G, const float* scores, const int32_t* lens, const int32_t* budgets,
                         int32_t* sel, int32_t* cnt, uint32_t* keybuf, int S, int H, int MP,
                         int max_budget, hipStream_t st) {
  dim3 grid(H, S);
  switch (G) {
    case 1: launch_select_g<1>(grid, MP, scores, lens, budgets, sel, cnt, keybuf, H, max_budget, st); break;
    case 2: launch_select_g<2>(grid, MP, scores, lens, budgets, sel, cnt, keybuf, H, max_budget, st); break;
    case 4: launch_select_g<4>(grid, MP, scores, lens, budgets, sel, cnt, keybuf, H, max_budget, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace locks
