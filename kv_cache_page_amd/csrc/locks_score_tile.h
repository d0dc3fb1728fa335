// LOCKS page scores on the matrix cores (gfx950), for ranks 4, 8 and 16: the
// per-tile device code shared by the score kernel and the fused decode step.
//
// [N] = LOCKS reading notes (zhongzhuzhou.org 2026-07-29), §4.2 eq. 4: for
// every full page j and query g of the GQA group,
//   s_hat_jg = LSE_t ((q_g . mu_j + c_t . (V_j^T q_g)) / sqrt(d))
// from the int4 basis, int8 coefficients and int8 centroid of the slot.
//
// Same contract and tiles as the VALU score kernel (128-page tiles of one
// (sequence, KV head), one Z partial per tile, one 256-thread workgroup per
// tile); wave w of a tile takes the 32 pages j_lo + 32 w + [0, 32) as 8
// groups of 4 pages. Lane l = 16 q16 + r16.
//
// Stage 1, W = V^T q on v_mfma_f32_16x16x32_f16, per group and quarter of
//   the ranks (ranks 4hh .. 4hh+3): A rows m = r16 are (page m / 4, rank
//   4hh + m % 4), K = the 128 dims. The int4 codes become exact fp16
//   denormals (c + 8) 2^-24 with two masks per nibble pair, and the K order
//   inside a lane follows the slot's nibble order (lane q16 of chunk c holds
//   dims 8 (4 q16 + c) .. +7, i.e. byte 16 q16 + 4c of the basis row), so each
//   lane reads one 16-byte piece of one row. The B columns n carry query
//   n % 4 (the G queries repeated), scaled by a power of two into fp16. The
//   D layout then leaves, in lane (q16 = a, r16), the 4 ranks of that quarter
//   for page a of the group and query r16 % 4: over the quarters, a lane holds
//   the whole W of its page for its query, with no data exchange.
// The centroid term mu . q uses one more MFMA chain per 16 pages with A rows
//   in the order page 4 (m % 4) + m / 4, so that register i of lane q16 holds
//   page 4 i + q16 for query r16 % 4; one lane permute per register hands it
//   to the lanes of stage 2's column (page r16 / 4).
// Stage 2, the logits c_t . W, on the matrix cores too: one product per
//   group (two for rank 16) with rows = the 16 tokens, K = (page, rank) and
//   columns n = (page n / 4, query n % 4). The B operand is block diagonal:
//   lane (a, r16) holds the W of page a for query r16 % 4, which is column
//   r16's block exactly when a == r16 / 4, and zeros otherwise. W enters as
//   an fp16 high part plus an fp16 low part (two products, about 21 bits),
//   scaled by 2^12 into fp16's normal range (|W| < 2 s_k in these units, so
//   basis-column scales s_k below 8 stay finite; unit basis columns give
//   s_k <= 1/7); the int8 coefficients become
//   exact fp16 through the 1024 + byte pattern. D leaves tokens 4a .. 4a+3 of
//   page r16 / 4 for query r16 % 4 in lane (a, r16); the LSE over the page's
//   16 tokens combines the four rows (row swaps, no LDS).
// The query rows are loaded together with the block ids; the slot loads of
// the first two groups and of the centroids are issued as soon as the ids
// arrive, the query operands are built meanwhile, and a 3-deep pipeline keeps
// two groups in flight while one is computed. Each loop iteration is one
// straight-line block (no early exit, outputs stored after the loop, loads
// unconditional) fenced by scheduling barriers: the compiler's memory wait
// counts then stay exact and every group waits only for its own loads.
#pragma once

#include "locks_device.h"

namespace locks {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// 8 int4 codes of one basis word -> (c + 8) 2^-24 as fp16 denormals, in the
// order [d0, d2, 16 d1, 16 d3, d4, d6, 16 d5, 16 d7] (bytes of the word hold
// the dim pairs (0,1), (4,5), (2,3), (6,7), low nibble first).
__device__ __forceinline__ half8 nib8(uint32_t w) {
  // (x ^ 8) & 15 per nibble: one three-input bit operation per output word
  const uint32_t w8 = w >> 8;
  return __builtin_bit_cast(half8, make_uint4((w ^ 0x00080008u) & 0x000F000Fu,
                                              (w ^ 0x00800080u) & 0x00F000F0u,
                                              (w8 ^ 0x00080008u) & 0x000F000Fu,
                                              (w8 ^ 0x00800080u) & 0x00F000F0u));
}

typedef _Float16 half4 __attribute__((ext_vector_type(4)));

// 4 int8 codes (one word, byte order) -> 2 words of exact fp16 values: the
// byte b = c + 128 becomes the half 0x64bb = 1024 + b, minus 1152.
__device__ __forceinline__ void coef4(uint32_t w, uint32_t& h0, uint32_t& h1) {
  const uint32_t y = w ^ 0x80808080u;
  const half2v k = half2v{(_Float16)-1152.f, (_Float16)-1152.f};
  h0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, y, 0x04010400u)) + k);
  h1 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, y, 0x04030402u)) + k);
}

// 8 int8 codes (two words, byte order) -> (c + 128) 2^-24 as fp16
// denormals, in the order [b0, b2, b1, b3, b4, b6, b5, b7].
__device__ __forceinline__ half8 byte8(uint32_t w0, uint32_t w1) {
  w0 ^= 0x80808080u;
  w1 ^= 0x80808080u;
  return __builtin_bit_cast(half8, make_uint4(w0 & 0x00FF00FFu, (w0 >> 8) & 0x00FF00FFu,
                                              w1 & 0x00FF00FFu, (w1 >> 8) & 0x00FF00FFu));
}

// Value of lane (r + K) mod 16 of the same 16-lane row (DPP row rotation).
template <int K>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 | K, 0xF, 0xF, true));
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Slot data of one 4-page group as one lane needs it.
template <int R>
struct GroupRegs {
  uint4 v[R / 4];        // basis: row 4 hh + r16 % 4 of page r16 / 4, bytes 16 q16 ..
  uint32_t c[R / 4];     // coefficients of token r16 of page q16
  uint32_t sv[R / 2];    // fp16 basis-column scales of page q16
  uint2 sc;              // fp16 scales of tokens 4 q16 .. 4 q16 + 3 of page r16 / 4
  uint32_t smu;          // fp16 centroid scale of page r16 / 4 (low half)
};

template <int R>
__device__ __forceinline__ void load_group(GroupRegs<R>& g, const uint8_t* __restrict__ slotV,
                                           const uint8_t* __restrict__ slotC, int r16, int q16) {
  constexpr SlotLayout L = slot_layout(R);
  const uint8_t* pv = slotV + L.v + 64 * (r16 & 3) + 16 * q16;
#pragma unroll
  for (int hh = 0; hh < R / 4; ++hh) g.v[hh] = *reinterpret_cast<const uint4*>(pv + 256 * hh);
  const uint8_t* pc = slotC + L.c + R * r16;  // the R code bytes of token r16
  if constexpr (R == 4) {
    g.c[0] = *reinterpret_cast<const uint32_t*>(pc);
  } else if constexpr (R == 8) {
    const uint2 t = *reinterpret_cast<const uint2*>(pc);
    g.c[0] = t.x;
    g.c[1] = t.y;
  } else {
    const uint4 t = *reinterpret_cast<const uint4*>(pc);
    g.c[0] = t.x;
    g.c[1] = t.y;
    g.c[2] = t.z;
    g.c[3] = t.w;
  }
#pragma unroll
  for (int e = 0; e < R / 2; ++e) g.sv[e] = *reinterpret_cast<const uint32_t*>(slotC + L.sv + 4 * e);
  g.sc = *reinterpret_cast<const uint2*>(slotV + L.sc + 8 * q16);
  g.smu = *reinterpret_cast<const uint16_t*>(slotV + L.smu);
}

// Splits the products p0 = w0 s0 and p1 = w1 s1 into fp16 high parts and
// fp16 low parts that together carry about 21 bits: hi = fp16(p) rounded
// toward zero by one packed conversion, lo = fp16(p - hi) (the remainder is
// exact in fp32). Both parts come from the one converted hi: when the
// compiler was free to round the product to fp16 twice (once fused into a
// mixed-precision FMA, once from the fp32 product), the two roundings could
// differ by an fp16 ulp on a rounding tie and hi + lo was then off by twice
// the low part.
__device__ __forceinline__ void split_hi_lo2(float w0, float s0, float w1, float s1, uint32_t& hi,
                                             uint32_t& lo) {
  const float p0 = w0 * s0, p1 = w1 * s1;
  const auto h = __builtin_amdgcn_cvt_pkrtz(p0, p1);
  const auto l = __builtin_amdgcn_cvt_pkrtz(p0 - (float)h[0], p1 - (float)h[1]);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

// One tile of TP pages (128, or 32 in a fused decode step over a short
// table), by 4 waves (wave = 0..3, tid = 64 wave + lane). Leaves the wave's Z
// partial of query gq = lane % 4 in (zm, zs) of lanes 0..3.
template <int R, int G, int TP = kScorePagesPerWg>
__device__ __forceinline__ void score_tile(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ summ,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, int64_t num_blocks, int H, int MP, int rowp,
    int flags, const uint16_t* __restrict__ knew, const uint16_t* __restrict__ vnew,
    uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool, float* __restrict__ mxout,
    int s, int h, int tile, int wave, int tid, float& zm, float& zs) {
  static_assert(R == 4 || R == 8 || R == 16, "matrix-core path covers ranks 4, 8, 16");
  static_assert(TP == 32 || TP == 64 || TP == 128, "a wave takes 8 pages or whole 16-page halves");
  constexpr SlotLayout L = slot_layout(R);
  constexpr int NHR = R / 4;
  constexpr float kTwoM24 = 5.9604644775390625e-08f;  // 2^-24
  constexpr int kWavePages = TP / 4;                  // pages per wave
  constexpr int kHalves = (kWavePages + 15) / 16;     // 16-page halves (centroid MFMAs)
  constexpr int kGroups = kWavePages / 4;             // 4-page groups per wave
  const int lane = tid & 63;
  const int r16 = lane & 15, q16 = lane >> 4;
  const int gq = r16 & 3;  // this lane's query (B column r16 carries query r16 % 4)
  const int j_lo = tile * TP;
  const int P0 = j_lo + kWavePages * wave;  // this wave's first page
  // block ids of the pages P0 + 16 u + r16, read together with the length
  int traw[kHalves];
#pragma unroll
  for (int u = 0; u < kHalves; ++u) {
    const int j = P0 + 16 * u + r16;
    traw[u] = (j < MP) ? table[(int64_t)s * MP + j] : -1;
  }
  // raw query rows (independent of the block ids): column r16 carries query
  // gq; lane q16 holds dims [32 q16, 32 q16 + 32) of it. Issued here, ahead
  // of the wait for the block ids (the empty asm keeps the compiler from
  // sinking the loads below it).
  const bool qok = gq < G;
  uint4 qraw[4];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(
        q + ((int64_t)s * H * G + (int64_t)h * G + (qok ? gq : 0)) * kHeadDim + 32 * q16);
#pragma unroll
    for (int c = 0; c < 4; ++c) qraw[c] = qp[c];
  }
  asm volatile("" ::: "memory");
  const int len = clampi(seq_lens[s], 0, MP * kPage);
  const int F = scored_pages(len, (flags & kScoreDeferred) ? 1 : 0);
  // the pools' head of this head (score_head_div)
  const int hdiv = score_head_div(flags), hd = h / hdiv, Hd = H / hdiv;
  if (knew && tile == 0 && h % hdiv == 0 && tid < 2 * (kHeadDim / 8) && len >= 1) {
    // decode-step append of the new token (position len - 1) for this head
    const int blk = table[(int64_t)s * MP + (len - 1) / kPage];
    if (blk >= 0 && blk < num_blocks) {
      const int c = tid % (kHeadDim / 8);
      const int64_t src = ((int64_t)s * Hd + hd) * kHeadDim + 8 * c;
      const int64_t dst = (((int64_t)blk * Hd + hd) * kPage + (len - 1) % kPage) * kHeadDim + 8 * c;
      if (tid < kHeadDim / 8)
        st_agent(reinterpret_cast<uint4*>(kpool + dst), *reinterpret_cast<const uint4*>(knew + src));
      else
        st_agent(reinterpret_cast<uint4*>(vpool + dst), *reinterpret_cast<const uint4*>(vnew + src));
    }
  }
  const int j_hi = min(j_lo + TP, MP);
  // output rows of rowp >= MP pages (a fused decode step rounds them up so
  // that every tile writes whole 128-byte lines)
  float* srow = scores + ((int64_t)s * H + h) * rowp * G;
  if (flags & kScoreFillNan) {
    const int first = max(j_lo, F);
    for (int idx = tid; idx < (j_hi - first) * G; idx += 256)
      reinterpret_cast<uint32_t*>(srow)[(int64_t)first * G + idx] = 0x7FC00000u;  // quiet NaN
  }
  if (j_lo >= F) return;
  const int j_end = min(j_hi, F);

  // ---- live block ids (-1: page past the end, of the next wave (8-page
  // waves fill half a 16-page half) or id out of range); the slot addresses
  // each role needs come by lane permutes. vbits[u] bit i: page P0 + 16 u + i
  // is live.
  int bo[kHalves];
  uint32_t vbits[kHalves];
#pragma unroll
  for (int u = 0; u < kHalves; ++u) {
    const int j = P0 + 16 * u + r16;
    const int b = traw[u];
    bo[u] = (j < j_end && 16 * u + r16 < kWavePages && b >= 0 && b < num_blocks) ? b : -1;
    vbits[u] = (uint32_t)__ballot(bo[u] >= 0) & 0xFFFFu;
  }

  // slot of block b for this head: summ_h + b * (H * stride), one 32 x 32 -> 64 multiply-add
  const uint8_t* summ_h = summ + (size_t)hd * L.stride;
  const uint32_t hs = (uint32_t)Hd * (uint32_t)L.stride;
  auto slot_ptr = [&](int b) -> const uint8_t* {
    return summ_h + (uint64_t)(uint32_t)(b < 0 ? 0 : b) * hs;
  };
  auto shfl_i = [&](int v, int src) -> int { return __shfl(v, src, 64); };

  // ---- centroid term per 16-page half: register i of lane q16 holds
  // page 16 u + 4 i + q16, query gq
  uint4 mw[kHalves][2];
  {
    const int src = 4 * (r16 & 3) + (r16 >> 2);  // A row r16 <- page src
#pragma unroll
    for (int u = 0; u < kHalves; ++u) {
      const uint8_t* o = slot_ptr(shfl_i(bo[u], src)) + L.mu + 32 * q16;
      mw[u][0] = *reinterpret_cast<const uint4*>(o);
      mw[u][1] = *reinterpret_cast<const uint4*>(o + 16);
    }
  }
  // ---- groups: pipeline of slot loads (three groups in flight while one is
  // computed; two for rank 16)
  float zv[kGroups];  // page LSEs (base 2) of query gq, for the tile's Z partial
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) zv[gi] = -__builtin_inff();
  constexpr int kDepth = (R >= 8) ? 3 : 4;  // a fourth group in flight measured no faster at rank 8
  GroupRegs<R> buf[kDepth];
  // block ids of every group's two lane roles, permuted once
  int bVg[kGroups], bCg[kGroups];
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    const int u = gi >> 2, base = 4 * (gi & 3);
    bVg[gi] = shfl_i(bo[u], base + (r16 >> 2));
    bCg[gi] = shfl_i(bo[u], base + q16);
  }
  auto issue = [&](int gi, GroupRegs<R>& gr) {
    load_group<R>(gr, slot_ptr(bVg[gi]), slot_ptr(bCg[gi]), r16, q16);
  };
  // Issues are unconditional (a group past the end reads block 0's slot,
  // which exists): a load behind a branch makes the compiler's wait counts
  // assume the worst case, and every group would then wait for all loads.
  // (the first kDepth - 1 groups, or every group of a wave that has fewer)
  constexpr int kFirst = (kDepth - 1 < kGroups) ? kDepth - 1 : kGroups;
#pragma unroll
  for (int gi = 0; gi < kFirst; ++gi) issue(gi, buf[gi]);
  __builtin_amdgcn_sched_barrier(0);  // keep the first issues ahead of the query-operand work
  // ---- query operands, power-of-two scaled into fp16 (built while the slot
  // loads are in flight)
  half8 B1[4], Bm[4];
  float vinit, minit, fs;
  {
    float x[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 w = qraw[c];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * c + 2 * e] = qok ? bf16_lo(ww[e]) : 0.f;
        x[8 * c + 2 * e + 1] = qok ? bf16_hi(ww[e]) : 0.f;
      }
    }
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) mx = fmaxf(mx, fabsf(x[e]));
    mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(mx), 0x401F)));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const int ex = (mx > 0.f && mx < __builtin_inff()) ? ilogbf(mx) : 0;
    const float up = ldexpf(1.f, 14 - ex);  // max |q| * up < 2^15
    float qs = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) qs += x[e] * up;
    qs += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(qs), 0x401F));
    qs += __shfl_xor(qs, 32, 64);
    // stage-1 operand, chunk c: dims 8 (4 q16 + c) + [0,2,1,3,4,6,5,7] with the
    // high nibbles' factor 16 divided out
    // centroid operand, chunk c: dims 32 q16 + 8 c + [0,2,1,3,4,6,5,7]
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // the lane's dims: local index 8 c' + e covers dim 32 q16 + 8 c' + e
      const float* y = x + 8 * c;  // dims 32 q16 + 8 c .. : word (4 q16 + c)
      B1[c] = half8{(_Float16)(y[0] * up), (_Float16)(y[2] * up),
                    (_Float16)(y[1] * up * 0.0625f), (_Float16)(y[3] * up * 0.0625f),
                    (_Float16)(y[4] * up), (_Float16)(y[6] * up),
                    (_Float16)(y[5] * up * 0.0625f), (_Float16)(y[7] * up * 0.0625f)};
      Bm[c] = half8{(_Float16)(y[0] * up), (_Float16)(y[2] * up), (_Float16)(y[1] * up),
                    (_Float16)(y[3] * up), (_Float16)(y[4] * up), (_Float16)(y[6] * up),
                    (_Float16)(y[5] * up), (_Float16)(y[7] * up)};
    }
    vinit = -8.f * kTwoM24 * qs;
    minit = -128.f * kTwoM24 * qs;
    // logits in log2 units: 2^(24 - (14 - ex)) * log2(e) / sqrt(d)
    fs = ldexpf(kLog2e * 0.08838834764831845f, 10 + ex);
  }

  floatx4 Dm[kHalves];
  {
#pragma unroll
    for (int u = 0; u < kHalves; ++u) {
      const uint32_t w[8] = {mw[u][0].x, mw[u][0].y, mw[u][0].z, mw[u][0].w,
                             mw[u][1].x, mw[u][1].y, mw[u][1].z, mw[u][1].w};
      floatx4 d = {minit, minit, minit, minit};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(byte8(w[2 * c], w[2 * c + 1]), Bm[c], d, 0, 0, 0);
      Dm[u] = d;
    }
  }
  // Stage-2 lane constants: the diagonal mask and the factor 2^12 ride on the
  // basis-column scales (a packed fp16 multiply per scale pair).
  const bool diag = q16 == (r16 >> 2);
  const half2v msig = diag ? half2v{(_Float16)4096.f, (_Float16)4096.f}
                           : half2v{(_Float16)0.f, (_Float16)0.f};
  const float fsig = fs * (1.f / 4096.f);
  // centroid term of the lane's stage-2 column: page 4 i + r16 / 4 of half u,
  // query r16 % 4, from register i of lane 16 (r16 / 4) + r16 % 4
  float muq[kHalves][4];
  {
    const int src = 4 * (16 * (r16 >> 2) + (r16 & 3));
#pragma unroll
    for (int u = 0; u < kHalves; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        muq[u][i] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(Dm[u][i])));
  }

#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    // no early exit for groups past the end (their pages are not live, so
    // nothing they compute is written): straight-line code keeps the
    // compiler from sinking the early slot loads into later blocks
    __builtin_amdgcn_sched_barrier(0);  // one iteration = the issue, then this group
    if (gi + kDepth - 1 < kGroups) issue(gi + kDepth - 1, buf[(gi + kDepth - 1) % kDepth]);
    __builtin_amdgcn_sched_barrier(0);
    const GroupRegs<R>& gr = buf[gi % kDepth];
    const int u = gi >> 2, base = 4 * (gi & 3);
    // stage 1: W of page q16 of the group, query gq, ranks 4 hh + i, times
    // 2^12 on the diagonal lanes and zero on the others
    uint32_t svm[R / 2];
#pragma unroll
    for (int e = 0; e < R / 2; ++e)
      svm[e] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, gr.sv[e]) * msig);
    float W[R];  // the stage-1 result d_k and the scale s_k, split below
    float Ws[R];
#pragma unroll
    for (int hh = 0; hh < NHR; ++hh) {
      floatx4 d = {vinit, vinit, vinit, vinit};
      const uint32_t vw[4] = {gr.v[hh].x, gr.v[hh].y, gr.v[hh].z, gr.v[hh].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(nib8(vw[c]), B1[c], d, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = 4 * hh + i;
        W[k] = d[i];
        Ws[k] = (k & 1) ? half_hi(svm[k >> 1]) : half_lo(svm[k >> 1]);
      }
    }
    // stage 2: X[i] = 2^12 c_t . W for token t = 4 q16 + i of page r16 / 4 and
    // query r16 % 4 (W = high + low fp16 parts)
    floatx4 X = {0.f, 0.f, 0.f, 0.f};
    if constexpr (R == 4) {
      uint32_t a0, a1;
      coef4(gr.c[0], a0, a1);
      const half4 A = __builtin_bit_cast(half4, make_uint2(a0, a1));
      uint32_t bh[2], bl[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) split_hi_lo2(W[2 * e], Ws[2 * e], W[2 * e + 1], Ws[2 * e + 1], bh[e], bl[e]);
      const half4 Bh = __builtin_bit_cast(half4, make_uint2(bh[0], bh[1]));
      const half4 Bl = __builtin_bit_cast(half4, make_uint2(bl[0], bl[1]));
      X = __builtin_amdgcn_mfma_f32_16x16x16f16(A, Bh, X, 0, 0, 0);
      X = __builtin_amdgcn_mfma_f32_16x16x16f16(A, Bl, X, 0, 0, 0);
    } else {
#pragma unroll
      for (int hc = 0; hc < R / 8; ++hc) {
        uint32_t a[4];
        coef4(gr.c[2 * hc], a[0], a[1]);
        coef4(gr.c[2 * hc + 1], a[2], a[3]);
        const half8 A = __builtin_bit_cast(half8, make_uint4(a[0], a[1], a[2], a[3]));
        uint32_t bh[4], bl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 8 * hc + 2 * e;
          split_hi_lo2(W[k], Ws[k], W[k + 1], Ws[k + 1], bh[e], bl[e]);
        }
        const half8 Bh = __builtin_bit_cast(half8, make_uint4(bh[0], bh[1], bh[2], bh[3]));
        const half8 Bl = __builtin_bit_cast(half8, make_uint4(bl[0], bl[1], bl[2], bl[3]));
        X = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bh, X, 0, 0, 0);
        X = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bl, X, 0, 0, 0);
      }
    }
    // logits (base 2) of tokens 4 q16 + i: fs (s_t c_t . W + q . mu)
    const float bm = fs * (muq[u][gi & 3] * half_lo(gr.smu));
    float lg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t sw = (i < 2) ? gr.sc.x : gr.sc.y;
      const float sc = (i & 1) ? half_hi(sw) : half_lo(sw);
      lg[i] = fmaf(fsig * sc, X[i], bm);
    }
    // LSE over the page's 16 tokens: 4 here, 12 in the other rows' lanes of
    // the same column
    float m = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    m = xrow_max(m);
    float e = __builtin_amdgcn_exp2f(lg[0] - m) + __builtin_amdgcn_exp2f(lg[1] - m) +
              __builtin_amdgcn_exp2f(lg[2] - m) + __builtin_amdgcn_exp2f(lg[3] - m);
    e = xrow_sum(e);
    const bool ok = ((vbits[u] >> (base + (r16 >> 2))) & 1u) && gq < G;
    zv[gi] = (ok && q16 == 0) ? m + __builtin_amdgcn_logf(e) : -__builtin_inff();
  }
  // outputs after the loop: stores behind lane conditions are branches, and
  // a branch between a slot load and its use makes the compiler's wait
  // counts assume the worst case
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    const int jp = P0 + 4 * gi + (r16 >> 2);  // the lane's page
    const bool writer = q16 == 0 && jp < j_end;  // row 0 writes
    const float out2 = zv[gi];
    if (mxout) {
      // decode layout: e_g = 2^(s_g - max_g s_g) per query and the page max;
      // lanes r16 = 4p .. 4p+3 hold page p's 4 queries (a DPP quad)
      const float mx = quad_max(out2);
      const float ev = (gq < G && mx != -__builtin_inff()) ? __builtin_amdgcn_exp2f(out2 - mx) : 0.f;
      // (coherent stores: in a fused decode step, other workgroups of the same
      // launch read them)
      if (writer && gq < G) st_agent(&srow[(int64_t)jp * G + gq], ev);
      if (writer && gq == 0) st_agent(&mxout[((int64_t)s * H + h) * rowp + jp], mx);
    } else if (writer && gq < G) {
      srow[(int64_t)jp * G + gq] = out2 * kLn2;
    }
  }
  // the lane's page LSEs (row 0 only), then lanes 0..3 carry query gq = r16;
  // reduce over the other lanes of the same query (xor 4, 8: the group's
  // pages; xor 16, 32: rows 1..3, empty)
  zm = zv[0];
#pragma unroll
  for (int gi = 1; gi < kGroups; ++gi) zm = fmaxf(zm, zv[gi]);
  zs = 0.f;
  if (zm != -__builtin_inff()) {
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) zs += __builtin_amdgcn_exp2f(zv[gi] - zm);
  }
#pragma unroll
  for (int mm = 4; mm < 64; mm <<= 1) {
    const float m2 = __shfl_xor(zm, mm, 64), s2 = __shfl_xor(zs, mm, 64);
    lse2_merge(zm, zs, m2, s2);
  }
}

}  // namespace locks
