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
#include "locks_select.h"

namespace locks {

// ---------------------------------------------------------------------------
// score
// ---------------------------------------------------------------------------
// kScorePagesPerWg = 4 waves x 16 pages x 2 batches

// BITS: the basis width (4; 8 and 2 for the precision ablation). The lane's
// 32 dims of a basis column take BITS 32-bit words.
template <int R, int BITS>
struct SlotRegs {
  uint32_t vq[R][BITS];
  uint4 mq0, mq1;
  uint32_t cq[R];
  uint16_t sv[R];
  uint16_t scw[4];
  uint16_t smw;
};

// Loads the lane's share of one slot. blk < 0 (page outside the range or a
// block id out of range) loads block 0's slot as a stand-in.
template <int R, int BITS>
__device__ __forceinline__ void load_slot(SlotRegs<R, BITS>& d, const uint8_t* __restrict__ summ,
                                          int H, int h, int blk, int l4) {
  constexpr SlotLayout L = slot_layout(R, BITS);
  const uint8_t* slot = static_cast<const uint8_t*>(
      __builtin_assume_aligned(summ + ((int64_t)(blk >= 0 ? blk : 0) * H + h) * L.stride, 16));
#pragma unroll
  for (int k = 0; k < R; ++k) {
    // column k is 16 BITS bytes; the lane's 32 dims are 4 BITS bytes of it
    const uint8_t* col = slot + 16 * BITS * k + 4 * BITS * l4;
    if constexpr (BITS == 2) {
      const uint2 w = *reinterpret_cast<const uint2*>(col);
      d.vq[k][0] = w.x;
      d.vq[k][1] = w.y;
    } else {
#pragma unroll
      for (int c = 0; c < BITS / 4; ++c) {
        const uint4 w = *reinterpret_cast<const uint4*>(col + 16 * c);
        d.vq[k][4 * c] = w.x;
        d.vq[k][4 * c + 1] = w.y;
        d.vq[k][4 * c + 2] = w.z;
        d.vq[k][4 * c + 3] = w.w;
      }
    }
  }
  d.mq0 = *reinterpret_cast<const uint4*>(slot + L.mu + 32 * l4);
  d.mq1 = *reinterpret_cast<const uint4*>(slot + L.mu + 32 * l4 + 16);
#pragma unroll
  for (int e = 0; e < R; ++e)
    d.cq[e] = *reinterpret_cast<const uint32_t*>(slot + L.c + 4 * R * l4 + 4 * e);
#pragma unroll
  for (int k = 0; k < R; ++k) d.sv[k] = *reinterpret_cast<const uint16_t*>(slot + L.sv + 2 * k);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d.scw[i] = *reinterpret_cast<const uint16_t*>(slot + L.sc + 8 * l4 + 2 * i);
  d.smw = *reinterpret_cast<const uint16_t*>(slot + L.smu);
}

// Grid (H, ceil(MP / kScorePagesPerWg), S): consecutive workgroup ids walk
// the heads first, so with 8 heads all tiles of a head land on one XCD (ids
// are dealt to the 8 XCDs round-robin) and its scores stay in that L2.
// zpart (optional): per workgroup and query head, the base-2 (max, sum of
// 2^(s - max)) of its pages' scores, so that Z_g needs no second pass.
// mxout (optional, decode layout): scores then receives, per page and query,
// e_g = 2^(s_g - max_g s_g) (base-2 s), and mxout[page] that maximum; the
// selection then needs one log2 per page instead of G exponentials.
// Otherwise scores receives s_hat in natural-log units.
// knew/vnew (optional): the workgroup with tile index 0 of each (sequence,
// head) first appends the new token's key and value for that head.
template <int R, int G, int BITS>
__global__ __launch_bounds__(256) void score_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ summ,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, int64_t num_blocks, int H, int MP, int pages_per_wg,
    int flags, float2* __restrict__ zpart, const uint16_t* __restrict__ knew,
    const uint16_t* __restrict__ vnew, uint16_t* __restrict__ kpool,
    uint16_t* __restrict__ vpool, float* __restrict__ mxout, CoopZero coop) {
  static_assert(BITS == 2 || BITS == 4 || BITS == 8, "basis width");
  constexpr float kTwoM24 = 5.9604644775390625e-08f;  // 2^-24
  zero_coop_mailbox(coop, (int64_t)blockIdx.z * H + blockIdx.x, blockIdx.y, gridDim.y);
  const int s = blockIdx.z, h = blockIdx.x, tile = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l4 = lane & 3;
  const int len = clampi(seq_lens[s], 0, MP * kPage);
  const int F = scored_pages(len, (flags & kScoreDeferred) ? 1 : 0);
  const int j_lo = tile * pages_per_wg;
  // the pools' head of this head (score_head_div)
  const int hdiv = score_head_div(flags), hd = h / hdiv, Hd = H / hdiv;
  if (knew && tile == 0 && h % hdiv == 0 && threadIdx.x < 2 * (kHeadDim / 8) && len >= 1) {
    // decode-step append of the new token (position len - 1) for this head
    const int blk = table[(int64_t)s * MP + (len - 1) / kPage];
    if (blk >= 0 && blk < num_blocks) {
      const int c = threadIdx.x % (kHeadDim / 8);
      const int64_t src = ((int64_t)s * Hd + hd) * kHeadDim + 8 * c;
      const int64_t dst = (((int64_t)blk * Hd + hd) * kPage + (len - 1) % kPage) * kHeadDim + 8 * c;
      if (threadIdx.x < kHeadDim / 8)
        *reinterpret_cast<uint4*>(kpool + dst) = *reinterpret_cast<const uint4*>(knew + src);
      else
        *reinterpret_cast<uint4*>(vpool + dst) = *reinterpret_cast<const uint4*>(vnew + src);
    }
  }
  const int j_hi = min(j_lo + pages_per_wg, MP);
  float* srow = scores + ((int64_t)s * H + h) * MP * G;
  if (flags & kScoreFillNan) {
    const int first = max(j_lo, F);
    for (int idx = threadIdx.x; idx < (j_hi - first) * G; idx += blockDim.x)
      srow[(int64_t)first * G + idx] = __builtin_nanf("");
  }
  if (j_lo >= F) return;
  const int j_end = min(j_hi, F);

  // ---- queries of the group: lane's 32 dims, power-of-two scaled fp16 pairs
  half2v Q[G][4][4];
  // int2 basis: the pairs of dims (16 h + e, 16 h + e + 8) that one mask of a
  // word's two-bit fields yields
  half2v Q2[BITS == 2 ? G : 1][2][8];
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
    if constexpr (BITS == 2) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          Q2[g][hh][e] = half2v{(_Float16)(x[16 * hh + e] * up), (_Float16)(x[16 * hh + e + 8] * up)};
    }
    // offset-binary codes: value = code - 8 (int4), - 128 (int8), - 2 (int2)
    vinit[g] = -(BITS == 4 ? 8.f : BITS == 8 ? 128.f : 2.f) * kTwoM24 * qs;
    minit[g] = -128.f * kTwoM24 * qs;
    // logits in log2 units: 2^(24 - (14 - ex)) * log2(e) / sqrt(d)
    fscale[g] = ldexpf(kLog2e * 0.08838834764831845f, 10 + ex);
  }

  // Block ids of all the lane's pages are read first (independent loads);
  // then a software pipeline loads the slot data of the next 16-page batch
  // into registers while the current batch is computed.
  constexpr int kMaxIter = kScorePagesPerWg / 64;
  const int jw = j_lo + wave * 16 + (lane >> 2);
  int blks[kMaxIter];
#pragma unroll
  for (int it = 0; it < kMaxIter; ++it) {
    const int j = jw + 64 * it;
    const int b = (j < j_end) ? table[(int64_t)s * MP + j] : -1;
    blks[it] = (b >= 0 && b < num_blocks) ? b : -1;
  }
  float zm = -__builtin_inff(), zs = 0.f;  // running LSE of query head l4 over the pages
  SlotRegs<R, BITS> cur, nxt;
  load_slot<R, BITS>(cur, summ, Hd, hd, blks[0], l4);
#pragma unroll
  for (int it = 0; it < kMaxIter; ++it) {
    const int j = jw + 64 * it;
    if (j - (lane >> 2) >= j_end) break;  // wave-uniform
    const bool in = j < j_end;
    const bool ok = blks[it] >= 0;
    if (it + 1 < kMaxIter) load_slot<R, BITS>(nxt, summ, Hd, hd, blks[it + 1 < kMaxIter ? it + 1 : it], l4);
    const uint4 mq0 = cur.mq0, mq1 = cur.mq1;
    const uint32_t* cq = cur.cq;
    const uint16_t* sv = cur.sv;
    const uint16_t* scw = cur.scw;
    const uint16_t smw = cur.smw;

    // ---- V^T q (partial over the lane's 32 dims)
    float acc[R][G];
#pragma unroll
    for (int k = 0; k < R; ++k) {
#pragma unroll
      for (int g = 0; g < G; ++g) acc[k][g] = vinit[g];
      if constexpr (BITS == 4) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t w = cur.vq[k][t] ^ 0x88888888u;
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
      } else if constexpr (BITS == 8) {
        // bytes as the centroid's: offset binary, even and odd dims of a word
        float a16[G];
#pragma unroll
        for (int g = 0; g < G; ++g) a16[g] = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t w = cur.vq[k][m] ^ 0x80808080u;
          const half2v e0 = __builtin_bit_cast(half2v, w & 0x00FF00FFu);
          const half2v e1 = __builtin_bit_cast(half2v, (w >> 8) & 0x00FF00FFu);
          const int t = m >> 1, o = (m & 1) * 2;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            acc[k][g] = __builtin_amdgcn_fdot2(e0, Q[g][t][o], acc[k][g], false);
            a16[g] = __builtin_amdgcn_fdot2(e1, Q[g][t][o + 1], a16[g], false);
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) acc[k][g] = fmaf(16.f, a16[g], acc[k][g]);
      } else {
        // two-bit fields: offset binary after flipping each field's top bit;
        // mask e yields the fields e and e + 8 of a word
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t w = cur.vq[k][hh] ^ 0xAAAAAAAAu;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const half2v p = __builtin_bit_cast(half2v, (w >> (2 * e)) & 0x00030003u);
#pragma unroll
            for (int g = 0; g < G; ++g) acc[k][g] = __builtin_amdgcn_fdot2(p, Q2[g][hh][e], acc[k][g], false);
          }
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
    // s_hat of query l4 in base-2 units (log2 of the page's sum of 2^logit)
    float out2 = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float m = fmaxf(fmaxf(lg[0][g], lg[1][g]), fmaxf(lg[2][g], lg[3][g]));
      m = quad_max(m);
      float e = __builtin_amdgcn_exp2f(lg[0][g] - m) + __builtin_amdgcn_exp2f(lg[1][g] - m) +
                __builtin_amdgcn_exp2f(lg[2][g] - m) + __builtin_amdgcn_exp2f(lg[3][g] - m);
      e = quad_sum(e);
      const float shat2 = m + __builtin_amdgcn_logf(e);
      if (l4 == g && ok) out2 = shat2;
    }
    if (mxout) {
      // decode layout: e_g = 2^(s_g - max_g s_g) per query and the page max
      const float mx = quad_max(out2);
      const float ev = (l4 < G && mx != -__builtin_inff()) ? __builtin_amdgcn_exp2f(out2 - mx) : 0.f;
      if (in && l4 < G) srow[(int64_t)j * G + l4] = ev;
      if (in && l4 == 0) mxout[((int64_t)s * H + h) * MP + j] = mx;
    } else if (in && l4 < G) {
      srow[(int64_t)j * G + l4] = out2 * kLn2;
    }
    if (in && ok) lse2_merge(zm, zs, out2, 1.f);
    cur = nxt;
  }
  if (zpart) {
    // reduce over the lanes that hold the same query head, then over waves
    __shared__ float zred[4][4][2];
#pragma unroll
    for (int m = 4; m < 64; m <<= 1) {
      const float m2 = __shfl_xor(zm, m, 64), s2 = __shfl_xor(zs, m, 64);
      lse2_merge(zm, zs, m2, s2);
    }
    if (lane < G) { zred[wave][lane][0] = zm; zred[wave][lane][1] = zs; }
    __syncthreads();
    if (threadIdx.x < G) {
      float m = zred[0][threadIdx.x][0], t = zred[0][threadIdx.x][1];
      for (int w = 1; w < 4; ++w) lse2_merge(m, t, zred[w][threadIdx.x][0], zred[w][threadIdx.x][1]);
      zpart[(((int64_t)s * H + h) * gridDim.y + tile) * G + threadIdx.x] = make_float2(m, t);
    }
  }
}

// ---------------------------------------------------------------------------
// select: one 1024-thread workgroup per (sequence, KV head)
//
// 1. scores -> registers; Z_g by a block max then a block exp-sum;
// 2. key_j in LDS (or global memory for very wide tables), block max K;
// 3. histogram of bin_j = min(511, floor((K - key_j) * 32)): bins are 1/32
//    nat wide and order-preserving (key_a > key_b implies bin_a <= bin_b), so
//    every candidate in a bin below the crossing bin t is selected;
// 4. inside bin t the remaining slots go to the candidates of largest key,
//    lower page first on ties, found by pairwise ranking (or, when more than
//    1024 candidates share bin t, by an exact 8-bit radix select on the
//    order-preserving key bits);
// 5. membership bits in an LDS bitmap, one 32-page word per thread, and a
//    block scan of word popcounts write the page ids in ascending order.
// ---------------------------------------------------------------------------
constexpr int kSelectThreads = 1024;
constexpr int kSelectLdsPages = 10240;  // keys of up to this many pages live in LDS (40 KB)
constexpr int kSelectRegPages = 8;      // pages per thread held in registers per chunk
constexpr int kMaxBitmapWords = 65536 / 32;

template <int G, bool kLdsKeys>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ budgets, int32_t* __restrict__ sel_pages,
    int32_t* __restrict__ sel_count, float* __restrict__ keybuf, int H, int MP,
    int max_budget, int lag, int rule) {
  extern __shared__ float sh_keys[];
  __shared__ uint32_t bits[kMaxBitmapWords];
  __shared__ uint32_t hist[kBins];
  __shared__ float cand_key[kSelectThreads];
  __shared__ int cand_page[kSelectThreads];
  __shared__ float red[16][4];
  __shared__ int sh_waves[16];
  __shared__ int sh_int[4];
  const int s = blockIdx.y, h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int nthr = kSelectThreads;
  const int len = clampi(seq_lens[s], 0, MP * kPage);
  const int P = (len + kPage - 1) / kPage;
  const int F = scored_pages(len, lag);
  const int k = clampi(budgets[s], 2, max_budget);
  int32_t* out = sel_pages + ((int64_t)s * H + h) * max_budget;
  if (P == 0 || k >= P) {
    for (int i = tid; i < max_budget; i += nthr) out[i] = i < P ? i : -1;
    if (tid == 0) sel_count[(int64_t)s * H + h] = P;
    return;
  }
  // From here P >= 3, k < P and pages 0..P-2 are full (F >= P-1).
  const float* sc = scores + ((int64_t)s * H + h) * MP * G;
  float* key = kLdsKeys ? sh_keys : keybuf + ((int64_t)s * H + h) * MP;
  const int nwords = (P + 31) / 32;
  for (int w = tid; w < nwords; w += nthr) bits[w] = 0u;
  constexpr int kChunk = kSelectRegPages * nthr;
  const bool one_chunk = F <= kChunk;

  // ---- 1. Z_g
  float v[kSelectRegPages][G];
  float mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = -__builtin_inff();
  for (int c0 = 0; c0 < F; c0 += kChunk) {
#pragma unroll
    for (int u = 0; u < kSelectRegPages; ++u) {
      const int j = c0 + u * nthr + tid;
      if (j < F) {
        load_scores<G>(sc + (int64_t)j * G, v[u]);
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) v[u][g] = -__builtin_inff();
      }
#pragma unroll
      for (int g = 0; g < G; ++g) mx[g] = fmaxf(mx[g], v[u][g]);
    }
  }
  block_max_g<G>(mx, red);
#pragma unroll
  for (int g = 0; g < G; ++g) if (mx[g] == -__builtin_inff()) mx[g] = 0.f;
  float sm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) sm[g] = 0.f;
  for (int c0 = 0; c0 < F; c0 += kChunk) {
#pragma unroll
    for (int u = 0; u < kSelectRegPages; ++u) {
      const int j = c0 + u * nthr + tid;
      if (!one_chunk && j < F) load_scores<G>(sc + (int64_t)j * G, v[u]);
      if (j < F)
#pragma unroll
        for (int g = 0; g < G; ++g) sm[g] += __expf(v[u][g] - mx[g]);
    }
  }
  block_sum_g<G>(sm, red);
  float logZ[G];
#pragma unroll
  for (int g = 0; g < G; ++g) logZ[g] = mx[g] + __logf(sm[g]);
  float logZtot = logZ[0];  // log sum_g Z_g (group-mass)
#pragma unroll
  for (int g = 1; g < G; ++g) {
    const float a = fmaxf(logZtot, logZ[g]), b = fminf(logZtot, logZ[g]);
    logZtot = a + log1pf(__expf(b - a));
  }

  // ---- 2. keys of the candidates 1..P-2 and their maximum
  const float logG = __logf((float)G);
  float kmax = -__builtin_inff();
  for (int c0 = 0; c0 < P - 1; c0 += kChunk) {
#pragma unroll
    for (int u = 0; u < kSelectRegPages; ++u) {
      const int j = c0 + u * nthr + tid;
      if (j < 1 || j > P - 2) continue;
      if (!one_chunk) load_scores<G>(sc + (int64_t)j * G, v[u]);
      const float kj = group_key_rule<G>(v[u], logZ, logG, rule, logZtot);
      key[j] = kj;
      kmax = fmaxf(kmax, kj);
    }
  }
  {
    float km[1] = {kmax};
    block_max_g<1>(km, red);
    kmax = km[0];
  }
  // ---- 3. histogram of the order-preserving bins below the best key
  for (int i = tid; i < kBins; i += nthr) hist[i] = 0u;
  __syncthreads();
  auto bin_of = [&](float kj) -> int {
    const float d = (kmax - kj) * kBinsPerNat;  // >= 0, +inf for -inf keys
    return d < (float)(kBins - 1) ? (int)d : kBins - 1;
  };
  for (int j = 1 + tid; j <= P - 2; j += nthr) atomicAdd(&hist[bin_of(key[j])], 1u);
  __syncthreads();
  int need = k - 2;
  int tbin = -1;  // crossing bin (-1: nothing to select beyond sink/recent)
  if (need > 0) {
    const int c = (tid < kBins) ? (int)hist[tid] : 0;
    int tot;
    const int before = block_exclusive_scan(c, sh_waves, &tot);
    if (tid < kBins && before < need && before + c >= need) {
      sh_int[0] = tid;
      sh_int[1] = need - before;
    }
    __syncthreads();
    tbin = sh_int[0];
    need = sh_int[1];
  }
  __syncthreads();
  // ---- 4. resolve inside bin tbin: take the `need` largest keys there
  if (tbin >= 0) {
    const int ct = (int)hist[tbin];
    if (ct <= nthr) {
      if (tid == 0) sh_int[2] = 0;
      __syncthreads();
      for (int j = 1 + tid; j <= P - 2; j += nthr) {
        const float kj = key[j];
        if (bin_of(kj) == tbin) {
          const int slot = atomicAdd(&sh_int[2], 1);
          cand_key[slot] = kj;
          cand_page[slot] = j;
        }
      }
      __syncthreads();
      if (tid < ct) {
        const float me = cand_key[tid];
        const int mp = cand_page[tid];
        int rank = 0;
        for (int e = 0; e < ct; ++e) {
          const float o = cand_key[e];
          rank += (o > me || (o == me && cand_page[e] < mp)) ? 1 : 0;
        }
        if (rank < need) atomicOr(&bits[mp >> 5], 1u << (mp & 31));
      }
    } else {
      // many candidates share the crossing bin (degenerate key distributions):
      // exact 8-bit radix select on the order-preserving key bits
      uint32_t prefix = 0u;
      for (int sh = 24; sh >= 0; sh -= 8) {
        for (int i = tid; i < 256; i += nthr) hist[i] = 0u;
        __syncthreads();
        for (int j = 1 + tid; j <= P - 2; j += nthr) {
          const float kj = key[j];
          const uint32_t u = float_to_ordered(kj);
          if (bin_of(kj) == tbin && (sh == 24 || (u >> (sh + 8)) == prefix))
            atomicAdd(&hist[255 - ((u >> sh) & 255u)], 1u);  // descending order
        }
        __syncthreads();
        const int c = (tid < 256) ? (int)hist[tid] : 0;
        int tot;
        const int before = block_exclusive_scan(c, sh_waves, &tot);
        if (tid < 256 && before < need && before + c >= need) {
          sh_int[0] = 255 - tid;
          sh_int[1] = need - before;
        }
        __syncthreads();
        prefix = (prefix << 8) | (uint32_t)sh_int[0];
        need = sh_int[1];
        __syncthreads();
      }
      // keys above `prefix` in bin tbin are in; `need` of those equal, lowest pages
      const int cpt = (P + nthr - 1) / nthr;
      const int c0 = tid * cpt, c1 = min(c0 + cpt, P - 1);
      int eq = 0;
      for (int j = max(c0, 1); j < c1; ++j) {
        const float kj = key[j];
        eq += (bin_of(kj) == tbin && float_to_ordered(kj) == prefix) ? 1 : 0;
      }
      int tot;
      int eq_before = block_exclusive_scan(eq, sh_waves, &tot);
      for (int j = max(c0, 1); j < c1; ++j) {
        const float kj = key[j];
        if (bin_of(kj) != tbin) continue;
        const uint32_t u = float_to_ordered(kj);
        if (u > prefix || (u == prefix && eq_before++ < need))
          atomicOr(&bits[j >> 5], 1u << (j & 31));
      }
    }
  }
  __syncthreads();
  // ---- 5. membership bitmap -> ascending page list
  for (int w = tid; w < nwords; w += nthr) {
    uint32_t b = bits[w];
    for (int e = 0; e < 32; ++e) {
      const int j = 32 * w + e;
      if (j >= P) break;
      bool in = (j == 0 || j == P - 1);
      if (!in && tbin >= 0) in = bin_of(key[j]) < tbin;
      if (in) b |= 1u << e;
    }
    bits[w] = b;
  }
  __syncthreads();
  // each thread owns words tid*wpt .. +wpt (wpt <= 2 for 65536 pages)
  const int wpt = (nwords + nthr - 1) / nthr;
  const int w0 = tid * wpt, w1 = min(w0 + wpt, nwords);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
  int tot;
  int pos = block_exclusive_scan(cnt, sh_waves, &tot);
  tot = min(tot, max_budget);  // == k <= max_budget by construction
  for (int w = w0; w < w1; ++w) {
    uint32_t b = bits[w];
    while (b) {
      const int e = __ffs(b) - 1;
      b &= b - 1;
      if (pos < max_budget) out[pos] = 32 * w + e;
      ++pos;
    }
  }
  for (int i = tot + tid; i < max_budget; i += nthr) out[i] = -1;
  if (tid == 0) sel_count[(int64_t)s * H + h] = tot;
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
template <int R, int G, int BITS>
static hipError_t launch_score_rg(const uint16_t* q, const uint8_t* summ, const int32_t* table,
                                  const int32_t* lens, float* scores, int64_t nb, int S, int H,
                                  int MP, int flags, float2* zpart, const void* knew,
                                  const void* vnew, void* kpool, void* vpool, float* mxout,
                                  CoopZero coop, hipStream_t st) {
  const int ppw = kScorePagesPerWg;
  dim3 grid(H, (MP + ppw - 1) / ppw, S);
  hipLaunchKernelGGL((score_kernel<R, G, BITS>), grid, dim3(256), 0, st, q, summ, table, lens, scores,
                     nb, H, MP, ppw, flags, zpart, static_cast<const uint16_t*>(knew),
                     static_cast<const uint16_t*>(vnew), static_cast<uint16_t*>(kpool),
                     static_cast<uint16_t*>(vpool), mxout, coop);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_score_g(int r, int bits, const uint16_t* q, const uint8_t* summ,
                                 const int32_t* table, const int32_t* lens, float* scores,
                                 int64_t nb, int S, int H, int MP, int flags, float2* zpart,
                                 const void* knew, const void* vnew, void* kpool, void* vpool,
                                 float* mxout, CoopZero coop, hipStream_t st) {
#define LOCKS_ARGS q, summ, table, lens, scores, nb, S, H, MP, flags, zpart, knew, vnew, kpool, vpool, mxout, coop, st
  if (bits != 4) {
    // the precision ablation: ranks 4, 8 and 16
#define LOCKS_RB(RR)                                                                   \
  case RR:                                                                             \
    return bits == 8 ? launch_score_rg<RR, G, 8>(LOCKS_ARGS)                           \
                     : bits == 2 ? launch_score_rg<RR, G, 2>(LOCKS_ARGS) : hipErrorInvalidValue;
    switch (r) {
      LOCKS_RB(4) LOCKS_RB(8) LOCKS_RB(16)
      default:
        return hipErrorInvalidValue;
    }
#undef LOCKS_RB
  }
  switch (r) {
#define LOCKS_R(RR) \
  case RR:          \
    return launch_score_rg<RR, G, 4>(LOCKS_ARGS);
    LOCKS_R(1) LOCKS_R(2) LOCKS_R(3) LOCKS_R(4) LOCKS_R(5) LOCKS_R(6) LOCKS_R(7) LOCKS_R(8)
    LOCKS_R(9) LOCKS_R(10) LOCKS_R(11) LOCKS_R(12) LOCKS_R(13) LOCKS_R(14) LOCKS_R(15) LOCKS_R(16)
#undef LOCKS_R
    default:
      return hipErrorInvalidValue;
  }
#undef LOCKS_ARGS
}

bool score_mfma_supported(int r);
hipError_t launch_score_mfma(int r, int G, const void* q, const void* summ, const int32_t* table,
                             const int32_t* lens, float* scores, int64_t nb, int S, int H, int MP,
                             int flags, float2* zpart, const void* knew, const void* vnew,
                             void* kpool, void* vpool, float* mxout, CoopZero coop,
                             hipStream_t st);

// bits: the basis width of the slots (4; 8 and 2 go through score_kernel).
hipError_t launch_score(int r, int bits, int G, const void* q, const void* summ,
                        const int32_t* table, const int32_t* lens, float* scores, int64_t nb,
                        int S, int H, int MP, int flags, float2* zpart, const void* knew,
                        const void* vnew, void* kpool, void* vpool, float* mxout, CoopZero coop,
                        hipStream_t st) {
  if (bits == 4 && score_mfma_supported(r))
    return launch_score_mfma(r, G, q, summ, table, lens, scores, nb, S, H, MP, flags, zpart,
                             knew, vnew, kpool, vpool, mxout, coop, st);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint8_t* ss = static_cast<const uint8_t*>(summ);
  switch (G) {
#define LOCKS_ARGS qq, ss, table, lens, scores, nb, S, H, MP, flags, zpart, knew, vnew, kpool, vpool, mxout, coop, st
    case 1: return launch_score_g<1>(r, bits, LOCKS_ARGS);
    case 2: return launch_score_g<2>(r, bits, LOCKS_ARGS);
    case 4: return launch_score_g<4>(r, bits, LOCKS_ARGS);
#undef LOCKS_ARGS
    default: return hipErrorInvalidValue;
  }
}

template <int G>
static void launch_select_g(dim3 grid, int MP, const float* scores, const int32_t* lens,
                            const int32_t* budgets, int32_t* sel, int32_t* cnt, float* keybuf,
                            int H, int max_budget, int lag, int rule, hipStream_t st) {
  if (MP <= kSelectLdsPages) {
    hipLaunchKernelGGL((select_kernel<G, true>), grid, dim3(kSelectThreads),
                       (size_t)MP * sizeof(float), st, scores, lens, budgets, sel, cnt, keybuf,
                       H, MP, max_budget, lag, rule);
  } else {
    hipLaunchKernelGGL((select_kernel<G, false>), grid, dim3(kSelectThreads), 0, st, scores, lens,
                       budgets, sel, cnt, keybuf, H, MP, max_budget, lag, rule);
  }
}

// lag = 1: only the pages full before the current token are scored (deferred
// build). rule: the GQA merge rule (kMergeShare, kMergeMax, kMergeMass).
hipError_t launch_select(int G, const float* scores, const int32_t* lens, const int32_t* budgets,
                         int32_t* sel, int32_t* cnt, float* keybuf, int S, int H, int MP,
                         int max_budget, int lag, int rule, hipStream_t st) {
  dim3 grid(H, S);
  switch (G) {
    case 1: launch_select_g<1>(grid, MP, scores, lens, budgets, sel, cnt, keybuf, H, max_budget, lag, rule, st); break;
    case 2: launch_select_g<2>(grid, MP, scores, lens, budgets, sel, cnt, keybuf, H, max_budget, lag, rule, st); break;
    case 4: launch_select_g<4>(grid, MP, scores, lens, budgets, sel, cnt, keybuf, H, max_budget, lag, rule, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace locks
