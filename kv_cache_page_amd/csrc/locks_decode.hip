// LOCKS decode step, second kernel: page selection, sparse attention over the
// selected pages, and the merge of the split partials, in one launch (gfx950).
//
// [N] = LOCKS reading notes (zhongzhuzhou.org 2026-07-29): §4.4 Algorithm 2
// (query-aware selection of the sink page, the most recent page and the
// top-(k-2) pages by the group-shared estimate of eq. 5), then §3.1 eq. 1
// (softmax attention renormalised over the selected set S).
//
// Grid (H, nsplit, S) with 512-thread workgroups; consecutive workgroup ids
// walk the KV heads first, so with 8 heads every split of a head runs on the
// same XCD as the score tiles of that head. Every workgroup of a (sequence,
// KV head) computes the whole selection itself: the computation is
// deterministic, so all of them obtain the same ascending page list without
// any inter-workgroup signal. Workgroup x then attends list entries
// [x * 8 * ppw, (x + 1) * 8 * ppw), one wave per ppw pages, and writes one
// partial (an empty one when it has no entries); a small second kernel merges
// the nsplit partials of each (sequence, KV head) in split order. (A merge by
// the last workgroup to arrive needs a release fence, an atomic round trip
// and an acquire in the critical path: measured slower than the extra launch.)
//
// Inputs from the score kernel (decode layout): per page j and query g,
// e_jg = 2^(s_jg - m_j) with m_j = max_g s_jg (base-2 scores), and m_j; per
// 128-page tile and query, the base-2 (max, sum) of the scores. Wave w owns
// the pages [64 kRP w, 64 kRP (w + 1)), lane l of it the pages 64 u + l of
// that range; their e, m and block ids are loaded at kernel start, before the
// sequence length is known.
//
// Selection, in base-2 units:
//   1. log2 Z_g from the tile partials (each wave reduces them by itself);
//   2. key_j = log2 mean_g 2^(s_jg - log2 Z_g)
//            = m_j - Zx + log2(sum_g e_jg W_g) - log2 G, W_g = 2^(Zx - log2 Z_g),
//      Zx = max_g log2 Z_g, for candidates 1..P-2 (one log2 per page; exact
//      while the group's log2 Z_g lie within 126 of each other). Keys are
//      log-shares, so key_j <= 0;
//   3. histogram of bin_j = floor(-key_j * 16), clamped to [0, 511] (1/16
//      wide, order-preserving; bin 511, which holds the far tail and -inf
//      keys, is counted by difference); every wave scans it for the bin t
//      where the top-(k-2) count is crossed;
//   4. list part A = sink, recent and the candidates below bin t (all of bin
//      t when it fits), in ascending page order, positions from the wave
//      totals and the wave's own ballots;
//   5. part B = the `need` largest keys of bin t, lower page first on ties,
//      in ascending page order after part A. Up to 64 candidates every wave
//      ranks them in registers (while the loads of its first part-A page are
//      already in flight); up to 512 they are ranked pairwise through LDS;
//      beyond, an exact 8-bit radix select on the order-preserving key bits.
// The attention partition (list positions per workgroup and wave) is thus a
// deterministic function of the keys; the selection output, when asked for,
// is rewritten as one ascending list.
#include "locks_attn_core.h"
#include "locks_select.h"

namespace locks {

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecMaxBudget = 2048;  // selection list held in LDS
constexpr int kDecMaxSplits = 32;
constexpr int kDecMaxPpw = 8;  // pages per wave
constexpr float kDecBinsPerUnit = 16.f;
constexpr int kHistCopies = 8;  // lanes spread their histogram atomics over 8 copies
constexpr int kFastRank = 64;   // crossing bins up to this size are ranked in registers
static_assert(kBins == kDecThreads, "one histogram bin per thread");

// Exclusive prefix sum over one wave.
__device__ __forceinline__ int wave_exclusive_scan(int v, int lane) {
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x - v;
}

template <int G, int kRP>
__global__ __launch_bounds__(kDecThreads) void decode_attn_kernel(
    const float* __restrict__ escore, const float* __restrict__ pmax,
    const float2* __restrict__ zpart, int ntiles, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ budgets, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kpool, const uint16_t* __restrict__ vpool,
    const int32_t* __restrict__ table, int64_t num_blocks, int H, int MP, int max_budget,
    int nsplit, int ppw, float* __restrict__ part, int32_t* __restrict__ sel_pages,
    int32_t* __restrict__ sel_count) {
  constexpr int kWords = kRP * kDecThreads / 32;  // page bitmap words (<= 512)
  static_assert(kWords <= kDecThreads, "bitmap words");
  constexpr int kWavePages = 64 * kRP;  // wave w owns pages [w * kWavePages, (w + 1) * kWavePages)
  __shared__ uint32_t histc[kHistCopies][kBins + 1];  // padded: copy c of bin b in bank (b + c) % 32
  __shared__ __align__(16) uint32_t hist[kBins];
  __shared__ uint32_t bits[kWords];      // members of a large crossing bin
  __shared__ uint32_t bits_out[kWords];  // whole selection (selection output only)
  __shared__ uint4 sh_q[G * kHeadDim / 8];
  __shared__ float cand_key[kDecThreads];
  __shared__ uint32_t cand_page[kDecThreads];  // also the tie bitmap of the radix path
  __shared__ int cand_blk[kDecThreads];
  __shared__ int sel_list[kDecMaxBudget];
  __shared__ int sel_blk[kDecMaxBudget];
  __shared__ int sh_waves[16];
  __shared__ int sh_wcnt[kDecWaves];
  __shared__ int sh_int[4];
  __shared__ float sh_acc[kDecWaves][G][kHeadDim];
  __shared__ float sh_ml[kDecWaves][G][2];

  const int h = blockIdx.x, x = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t sh_idx = (int64_t)s * H + h;
  // page of register slot u of this thread
  auto page_of = [&](int u) { return wave * kWavePages + 64 * u + lane; };

  // ---- every independent load first
  const int len_raw = seq_lens[s];
  const int bud_raw = budgets[s];
  // tile Z partials first: the Z reduction can start while the page loads
  // are still in flight
  const float2* zp = zpart + sh_idx * ntiles * G;
  constexpr int kZl = (kRP * kDecThreads + 64 * kScorePagesPerWg - 1) / (64 * kScorePagesPerWg);
  float2 zl[kZl][G];  // tile partials t = lane + 64 c
#pragma unroll
  for (int c = 0; c < kZl; ++c) {
    const int t = lane + 64 * c;
#pragma unroll
    for (int g = 0; g < G; ++g)
      zl[c][g] = (t < ntiles) ? zp[t * G + g] : make_float2(-__builtin_inff(), 0.f);
  }
  float ev[kRP][G], mv[kRP];
  int bk[kRP];
  {
    const float* er = escore + sh_idx * MP * G;
    const float* mr = pmax + sh_idx * MP;
    const int32_t* tr = table + (int64_t)s * MP;
#pragma unroll
    for (int u = 0; u < kRP; ++u) {
      const int j = page_of(u);
      if (j < MP) {
        load_scores<G>(er + (int64_t)j * G, ev[u]);
        mv[u] = mr[j];
        bk[u] = tr[j];
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) ev[u][g] = 0.f;
        mv[u] = -__builtin_inff();
        bk[u] = -1;
      }
    }
  }
  if (tid < G * kHeadDim / 8) sh_q[tid] = reinterpret_cast<const uint4*>(q + sh_idx * G * kHeadDim)[tid];
  // histogram and bitmap cleared while the loads are in flight (the first
  // barrier of the selection publishes this)
  for (int i = tid; i < kHistCopies * (kBins + 1); i += kDecThreads) (&histc[0][0])[i] = 0u;
  if (tid < kWords) { bits[tid] = 0u; bits_out[tid] = 0u; }
  if (tid == 0) sh_int[3] = 0;

  const int len = clampi(len_raw, 0, MP * kPage);
  const int P = (len + kPage - 1) / kPage;
  const int F = len / kPage;
  const int k = clampi(bud_raw, 2, max_budget);
  int n, nA;
  int tbin = -1, need = 0, ct = 0;  // crossing bin, slots left in it, its size
  bool part_bin = false, fast_b = false;
  const bool sel_all = (P == 0 || k >= P);
  uint64_t bal[kRP];
  if (sel_all) {
    n = P;  // every page (P <= k <= max_budget)
    nA = n;
#pragma unroll
    for (int u = 0; u < kRP; ++u) {
      const int j = page_of(u);
      if (j < P) {
        sel_list[j] = j;
        sel_blk[j] = bk[u];
      }
    }
  } else {
    // From here P >= 3, k < P and pages 0..P-2 are full (F >= P-1).
    // ---- 1. log2 Z_g over the F full pages (tiles beyond F hold nothing)
    const int ntu = (F + kScorePagesPerWg - 1) / kScorePagesPerWg;
    float lz[G], zx = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mt = -__builtin_inff();
#pragma unroll
      for (int c = 0; c < kZl; ++c)
        if (lane + 64 * c < ntu) mt = fmaxf(mt, zl[c][g].x);
      const float M = wave_allmax(mt);
      float c = 0.f;
#pragma unroll
      for (int cc = 0; cc < kZl; ++cc) {
        const float mc = (lane + 64 * cc < ntu) ? zl[cc][g].x : -__builtin_inff();
        if (mc != -__builtin_inff()) c += zl[cc][g].y * __builtin_amdgcn_exp2f(mc - M);
      }
      const float S = wave_allsum(c);
      lz[g] = S > 0.f ? M + __builtin_amdgcn_logf(S) : -__builtin_inff();
      zx = fmaxf(zx, lz[g]);
    }
    float wg[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
      wg[g] = (lz[g] == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(fminf(zx - lz[g], 126.f));
    const float log2G = (G == 1) ? 0.f : (G == 2) ? 1.f : 2.f;
    // ---- 2. keys (<= 0) and their bins
    auto is_cand = [&](int j) { return j >= 1 && j <= P - 2; };
    float key[kRP];
    int bin[kRP];
#pragma unroll
    for (int u = 0; u < kRP; ++u) {
      const int j = page_of(u);
      float t = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) t = fmaf(ev[u][g], wg[g], t);
      float kj = (mv[u] - zx) + (__builtin_amdgcn_logf(t) - log2G);
      kj = (is_cand(j) && kj == kj) ? kj : -__builtin_inff();
      key[u] = kj;
      const float d = -kj * kDecBinsPerUnit;  // >= 0 up to rounding; +inf for -inf keys
      bin[u] = d < (float)(kBins - 1) ? (d > 0.f ? (int)d : 0) : kBins - 1;
    }
    // ---- 3. histogram (bin 511 by difference)
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kRP; ++u)
      if (bin[u] < kBins - 1) atomicAdd(&histc[lane & (kHistCopies - 1)][bin[u]], 1u);
    __syncthreads();
    {
      uint32_t t = 0u;
#pragma unroll
      for (int c = 0; c < kHistCopies; ++c) t += histc[c][tid];
      hist[tid] = t;
    }
    __syncthreads();
    // ---- 4. crossing bin: every wave scans the histogram itself (lane l
    // holds bins 8l .. 8l+7), so no broadcast is needed
    const int need0 = k - 2;
    if (need0 > 0) {
      const uint4 h0 = *reinterpret_cast<const uint4*>(&hist[8 * lane]);
      const uint4 h1 = *reinterpret_cast<const uint4*>(&hist[8 * lane + 4]);
      int c8[8] = {(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w, (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
      int tot = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) tot += c8[e];
      int before = wave_inclusive_scan(tot) - tot;
      if (lane == 63) c8[7] = (P - 2) - (before + tot - c8[7]);  // bin 511: the rest
      int fb = -1, fn = 0, fc = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (before < need0 && before + c8[e] >= need0) { fb = 8 * lane + e; fn = need0 - before; fc = c8[e]; }
        before += c8[e];
      }
      const uint64_t found = __ballot(fb >= 0);
      if (found) {  // wave-uniform; one lane holds the crossing
        const int src = __builtin_ctzll(found);
        tbin = __builtin_amdgcn_readlane(fb, src);
        need = __builtin_amdgcn_readlane(fn, src);
        ct = __builtin_amdgcn_readlane(fc, src);
      }
    }
    // ---- 5. list part A: sink, recent and the candidates below the crossing
    // bin (with the whole crossing bin when it fits), in ascending page order;
    // the crossing bin's candidates go to LDS when only part of it is taken
    part_bin = (tbin >= 0) && (need < ct);
    int wA = 0;
#pragma unroll
    for (int u = 0; u < kRP; ++u) {
      const int j = page_of(u);
      const bool cand = (j >= 1) & (j <= P - 2);
      const bool in = (j == 0) | (j == P - 1) | (cand & (bin[u] < tbin)) |
                      ((tbin >= 0) & (need == ct) & cand & (bin[u] == tbin));
      bal[u] = __ballot(in);
      wA += __popcll(bal[u]);
    }
    if (part_bin && ct <= kDecThreads) {
#pragma unroll
      for (int u = 0; u < kRP; ++u) {
        const int j = page_of(u);
        if (is_cand(j) && bin[u] == tbin) {
          const int slot = atomicAdd(&sh_int[3], 1);
          cand_key[slot] = key[u];
          cand_page[slot] = (uint32_t)j;
          cand_blk[slot] = bk[u];
        }
      }
    }
    if (lane == 0) sh_wcnt[wave] = wA;
    __syncthreads();
    nA = 0;
    {
      int pos = 0;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const int c = sh_wcnt[w];
        pos += (w < wave) ? c : 0;
        nA += c;
      }
#pragma unroll
      for (int u = 0; u < kRP; ++u) {
        if ((bal[u] >> lane) & 1ull) {
          const int p = pos + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[u] >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bal[u], 0u));
          if (p < kDecMaxBudget) {
            sel_list[p] = page_of(u);
            sel_blk[p] = bk[u];
          }
        }
        pos += __popcll(bal[u]);
      }
    }
    n = min(nA + (part_bin ? need : 0), max_budget);  // == k by construction
    if (part_bin && ct > kFastRank) {
      // ---- 6 (large crossing bin). Members into the bitmap, then their
      // positions nA + (members with a lower page) written by their owners
      if (ct <= kDecThreads) {
        if (tid < ct) {
          const float me = cand_key[tid];
          const uint32_t mp = cand_page[tid];
          int rank = 0;
#pragma unroll 8
          for (int e = 0; e < ct; ++e) {
            const float o = cand_key[e];
            rank += (o > me || (o == me && cand_page[e] < mp)) ? 1 : 0;
          }
          if (rank < need) atomicOr(&bits[mp >> 5], 1u << (mp & 31));
        }
      } else {
        // exact 8-bit radix select on the order-preserving key bits
        uint32_t prefix = 0u;
#pragma unroll 1
        for (int shift = 24; shift >= 0; shift -= 8) {
          __syncthreads();
          if (tid < 256) hist[tid] = 0u;
          __syncthreads();
#pragma unroll
          for (int u = 0; u < kRP; ++u) {
            const int j = page_of(u);
            const uint32_t o = float_to_ordered(key[u]);
            if (is_cand(j) && bin[u] == tbin && (shift == 24 || (o >> (shift + 8)) == prefix))
              atomicAdd(&hist[255 - ((o >> shift) & 255u)], 1u);  // descending order
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
        }
        // keys above `prefix` are in; of those equal to it, the `need` lowest pages
        uint32_t* eqb = cand_page;
        if (tid < kWords) eqb[tid] = 0u;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kRP; ++u) {
          const int j = page_of(u);
          if (!is_cand(j) || bin[u] != tbin) continue;
          const uint32_t o = float_to_ordered(key[u]);
          if (o > prefix) atomicOr(&bits[j >> 5], 1u << (j & 31));
          else if (o == prefix) atomicOr(&eqb[j >> 5], 1u << (j & 31));
        }
        __syncthreads();
        const uint32_t ew = (tid < kWords) ? eqb[tid] : 0u;
        int tot;
        const int before = block_exclusive_scan(__popc(ew), sh_waves, &tot);
        if (before < need) {
          uint32_t w = ew, take = 0u;
          for (int left = need - before; w && left > 0; --left) {
            const uint32_t low = w & (0u - w);
            take |= low;
            w ^= low;
          }
          if (take) atomicOr(&bits[tid], take);
        }
      }
      __syncthreads();
      {
        const uint32_t bw = (tid < kWords) ? bits[tid] : 0u;
        int tot;
        const int before = block_exclusive_scan(__popc(bw), sh_waves, &tot);
        if (tid < kWords) hist[tid] = (uint32_t)before;  // word offsets (kWords <= kBins)
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kRP; ++u) {
        const int j = page_of(u);
        if (!is_cand(j) || bin[u] != tbin) continue;
        const uint32_t w = bits[j >> 5];
        if ((w >> (j & 31)) & 1u) {
          const int p = nA + (int)hist[j >> 5] + __popc(w & ((1u << (j & 31)) - 1u));
          if (p < kDecMaxBudget) {
            sel_list[p] = j;
            sel_blk[p] = bk[u];
          }
        }
      }
      nA = n;  // the whole list now sits in LDS
    }
    fast_b = part_bin && ct <= kFastRank;
  }
  __syncthreads();

  // ---- the wave's pages: list positions base .. base + ppw - 1. Positions
  // below nA come from LDS; the rest (a partly taken crossing bin of at most
  // 64 candidates) from a ranking every wave repeats in registers, while the
  // loads of its first page are already in flight
  const int per_wg = kDecWaves * ppw;
  const int base = x * per_wg + wave * ppw;
  const int mine = clampi(n - base, 0, ppw);
  uint32_t qw[G][16];
  attn_load_q<G>(qw, reinterpret_cast<const uint16_t*>(sh_q), lane);
  auto page_off = [&](int j, int blk, int64_t& off, int& nv) {
    off = -1;
    nv = 0;
    if (j < 0 || j >= P || blk < 0 || blk >= num_blocks) return;
    off = ((int64_t)blk * H + h) * (kPage * kHeadDim);
    nv = (j == P - 1) ? len - kPage * (P - 1) : kPage;
  };
  int64_t off[kDecMaxPpw];
  int nv[kDecMaxPpw];
#pragma unroll
  for (int i = 0; i < kDecMaxPpw; ++i) { off[i] = -1; nv[i] = 0; }
#pragma unroll
  for (int i = 0; i < kDecMaxPpw; ++i)
    if (i < mine && base + i < nA) page_off(sel_list[base + i], sel_blk[base + i], off[i], nv[i]);
  PageRegs cur, nxt;
  if (mine > 0 && off[0] >= 0) attn_load_page(cur, kpool, vpool, off[0], lane);
  if (fast_b && base + mine > nA) {
    // lane e < ct holds candidate e; rank by key (lower page first on ties),
    // then the members' positions nA + (members with a lower page)
    float ck = -__builtin_inff();
    uint32_t cp = 0xFFFFFFFFu;
    int cb = -1;
    if (lane < ct) { ck = cand_key[lane]; cp = cand_page[lane]; cb = cand_blk[lane]; }
    int rank = 0;
    for (int e = 0; e < ct; ++e) {
      const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ck), e));
      const uint32_t op = (uint32_t)__builtin_amdgcn_readlane((int)cp, e);
      rank += ((o > ck) | ((o == ck) & (op < cp))) ? 1 : 0;
    }
    const bool inB = (lane < ct) & (rank < need);
    const uint64_t bm = __ballot(inB);
    int bpos = nA;
    for (int e = 0; e < ct; ++e) {
      const uint32_t op = (uint32_t)__builtin_amdgcn_readlane((int)cp, e);
      bpos += (((bm >> e) & 1ull) && op < cp) ? 1 : 0;
    }
#pragma unroll
    for (int i = 0; i < kDecMaxPpw; ++i) {
      if (i < mine && base + i >= nA) {
        const uint64_t hit = __ballot(inB && bpos == base + i);
        if (hit) {
          const int src = __builtin_ctzll(hit);
          page_off(__builtin_amdgcn_readlane((int)cp, src), __builtin_amdgcn_readlane(cb, src), off[i], nv[i]);
        }
      }
    }
    if (mine > 0 && base >= nA && off[0] >= 0) attn_load_page(cur, kpool, vpool, off[0], lane);
  }
  // ---- attention over the wave's pages (next page loading while one is computed)
  {
    AttnAcc<G> acc;
    attn_init<G>(acc);
#pragma unroll
    for (int i = 0; i < kDecMaxPpw; ++i) {
      if (i >= mine) break;
      if (i + 1 < kDecMaxPpw && i + 1 < mine && off[i + 1 < kDecMaxPpw ? i + 1 : i] >= 0)
        attn_load_page(nxt, kpool, vpool, off[i + 1 < kDecMaxPpw ? i + 1 : i], lane);
      if (off[i] >= 0) attn_page<G>(acc, cur, qw, nv[i], lane);
      cur = nxt;
    }
    attn_wave_to_lds<G>(acc, sh_acc[wave], sh_ml[wave], lane);
  }
  // ---- selection output (first workgroup only): the ascending page list
  if (x == 0 && sel_pages) {
    int32_t* o = sel_pages + sh_idx * max_budget;
    if (!sel_all) {
      // membership bitmap: part A from the wave ballots, then the crossing
      // bin's members (already in `bits` on the large-bin path)
      if (lane == 0) {
#pragma unroll
        for (int u = 0; u < kRP; ++u) {
          const int w0 = (wave * kWavePages + 64 * u) >> 5;
          bits_out[w0] = (uint32_t)bal[u];
          bits_out[w0 + 1] = (uint32_t)(bal[u] >> 32);
        }
      }
      __syncthreads();
      if (fast_b && wave == 0 && lane < ct) {
        const float ck = cand_key[lane];
        const uint32_t cp = cand_page[lane];
        int rank = 0;
        for (int e = 0; e < ct; ++e) {
          const float o2 = cand_key[e];
          rank += ((o2 > ck) | ((o2 == ck) & (cand_page[e] < cp))) ? 1 : 0;
        }
        if (rank < need) atomicOr(&bits_out[cp >> 5], 1u << (cp & 31));
      }
      if (part_bin && !fast_b && tid < kWords) atomicOr(&bits_out[tid], bits[tid]);
      __syncthreads();
      const uint32_t bw = (tid < kWords) ? bits_out[tid] : 0u;
      int tot;
      int before = block_exclusive_scan(__popc(bw), sh_waves, &tot);
      uint32_t w = bw;
      while (w) {
        const int b = __builtin_ctz(w);
        w &= w - 1u;
        if (before < max_budget) o[before] = 32 * tid + b;
        ++before;
      }
      for (int i = tot + tid; i < max_budget; i += kDecThreads) o[i] = -1;
    } else {
      for (int i = tid; i < max_budget; i += kDecThreads) o[i] = i < n ? sel_list[i] : -1;
    }
    if (tid == 0) sel_count[sh_idx] = n;
  }
  __syncthreads();
  // ---- the workgroup's partial: thread (g, d) combines the 8 wave partials
  if (tid < G * kHeadDim) {
    const int g = tid / kHeadDim, d = tid % kHeadDim;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, sh_ml[w][g][0]);
    float a = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = (M == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(sh_ml[w][g][0] - M);
      a += f * sh_acc[w][g][d];
      L += f * sh_ml[w][g][1];
    }
    float* p = part + (sh_idx * nsplit + x) * G * kPartStride + g * kPartStride;
    p[d] = a;
    if (d == 0) *reinterpret_cast<float2*>(p + kHeadDim) = make_float2(M, L);
  }
}

// Merge of the nsplit partials of one (sequence, KV head) in split order:
// thread (g, c) owns output elements 4c .. 4c+3 of query g. All partials exist
// (empty ones carry max -inf, sum 0, acc 0); an empty selection gives out = 0
// and lse = -inf. kMaxS >= nsplit bounds the unrolled load loop.
template <int G, int kMaxS>
__global__ __launch_bounds__(G * kHeadDim / 4) void decode_merge_kernel(
    const float* __restrict__ part, float* __restrict__ out, float* __restrict__ lse_out, int H,
    int nsplit) {
  const int64_t sh_idx = (int64_t)blockIdx.y * H + blockIdx.x;
  const int tid = threadIdx.x;
  const int g = tid / (kHeadDim / 4), d = 4 * (tid % (kHeadDim / 4));
  const float* parts = part + sh_idx * nsplit * G * kPartStride;
  float4 pa[kMaxS];
  float pm[kMaxS], pl[kMaxS];
#pragma unroll
  for (int y = 0; y < kMaxS; ++y) {
    // unconditional (clamped) loads, masked afterwards: all in flight at once
    const float* py = parts + (min(y, nsplit - 1) * G + g) * kPartStride;
    pa[y] = *reinterpret_cast<const float4*>(py + d);
    const float2 ml = *reinterpret_cast<const float2*>(py + kHeadDim);
    pm[y] = ml.x;
    pl[y] = ml.y;
  }
#pragma unroll
  for (int y = 0; y < kMaxS; ++y)
    if (y >= nsplit) { pa[y] = make_float4(0.f, 0.f, 0.f, 0.f); pm[y] = -__builtin_inff(); pl[y] = 0.f; }
  // one common maximum, then every split's weight independently (no chain
  // of rescalings), summed in split order
  float M = -__builtin_inff();
#pragma unroll
  for (int y = 0; y < kMaxS; ++y) M = fmaxf(M, pm[y]);
  float L = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int y = 0; y < kMaxS; ++y) {
    const float f = (M == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(pm[y] - M);
    L = fmaf(pl[y], f, L);
    a.x = fmaf(pa[y].x, f, a.x);
    a.y = fmaf(pa[y].y, f, a.y);
    a.z = fmaf(pa[y].z, f, a.z);
    a.w = fmaf(pa[y].w, f, a.w);
  }
  const bool some = L > 0.f;
  *reinterpret_cast<float4*>(out + (sh_idx * G + g) * kHeadDim + d) =
      some ? make_float4(a.x / L, a.y / L, a.z / L, a.w / L) : make_float4(0.f, 0.f, 0.f, 0.f);
  if (lse_out && d == 0)
    lse_out[sh_idx * G + g] = (L > 0.f) ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -__builtin_inff();
}

// Launch shape of the fused kernel for a table of MP pages and a budget of KB
// pages: false when it does not apply (the caller then runs the separate
// select and attention kernels).
bool decode_shape(int MP, int KB, int* ppw, int* nsplit) {
  if (MP > 32 * kDecThreads || KB > kDecMaxBudget) return false;
  int p = 1;
  while (p < kDecMaxPpw && (KB + kDecWaves * p - 1) / (kDecWaves * p) > 16) p *= 2;
  const int ns = (KB + kDecWaves * p - 1) / (kDecWaves * p);
  if (ns > kDecMaxSplits) return false;
  *ppw = p;
  *nsplit = ns;
  return true;
}

int decode_max_splits() { return kDecMaxSplits; }

template <int G, int kRP>
static void launch_decode_rp(const float* escore, const float* pmax, const float2* zpart,
                             int ntiles, const int32_t* lens, const int32_t* budgets,
                             const uint16_t* q, const uint16_t* kpool, const uint16_t* vpool,
                             const int32_t* table, int64_t nb, int S, int H, int MP, int KB,
                             int nsplit, int ppw, float* part, float* out, float* lse_out,
                             int32_t* sel, int32_t* cnt, hipStream_t st) {
  hipLaunchKernelGGL((decode_attn_kernel<G, kRP>), dim3(H, nsplit, S), dim3(kDecThreads), 0, st,
                     escore, pmax, zpart, ntiles, lens, budgets, q, kpool, vpool, table, nb, H, MP,
                     KB, nsplit, ppw, part, sel, cnt);
  const dim3 mg(H, S), mb(G * kHeadDim / 4);
  if (nsplit <= 8)
    hipLaunchKernelGGL((decode_merge_kernel<G, 8>), mg, mb, 0, st, part, out, lse_out, H, nsplit);
  else if (nsplit <= 16)
    hipLaunchKernelGGL((decode_merge_kernel<G, 16>), mg, mb, 0, st, part, out, lse_out, H, nsplit);
  else
    hipLaunchKernelGGL((decode_merge_kernel<G, kDecMaxSplits>), mg, mb, 0, st, part, out, lse_out, H,
                       nsplit);
}

template <int G>
static void launch_decode_g(const float* escore, const float* pmax, const float2* zpart,
                            int ntiles, const int32_t* lens, const int32_t* budgets,
                            const uint16_t* q, const uint16_t* kpool, const uint16_t* vpool,
                            const int32_t* table, int64_t nb, int S, int H, int MP, int KB,
                            int nsplit, int ppw, float* part, float* out, float* lse_out,
                            int32_t* sel, int32_t* cnt, hipStream_t st) {
#define LOCKS_ARGS escore, pmax, zpart, ntiles, lens, budgets, q, kpool, vpool, table, nb, S, H, \
                   MP, KB, nsplit, ppw, part, out, lse_out, sel, cnt, st
  if (MP <= 4 * kDecThreads)
    launch_decode_rp<G, 4>(LOCKS_ARGS);
  else if (MP <= 16 * kDecThreads)
    launch_decode_rp<G, 16>(LOCKS_ARGS);
  else
    launch_decode_rp<G, 32>(LOCKS_ARGS);
#undef LOCKS_ARGS
}

hipError_t launch_decode(int G, const float* escore, const float* pmax, const float2* zpart,
                         int ntiles, const int32_t* lens, const int32_t* budgets, const void* q,
                         const void* kpool, const void* vpool, const int32_t* table, int64_t nb,
                         int S, int H, int MP, int KB, int nsplit, int ppw, float* part,
                         float* out, float* lse_out, int32_t* sel, int32_t* cnt, hipStream_t st) {
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(kpool);
  const uint16_t* vv = static_cast<const uint16_t*>(vpool);
#define LOCKS_ARGS escore, pmax, zpart, ntiles, lens, budgets, qq, kk, vv, table, nb, S, H, MP, KB, \
                   nsplit, ppw, part, out, lse_out, sel, cnt, st
  switch (G) {
    case 1: launch_decode_g<1>(LOCKS_ARGS); break;
    case 2: launch_decode_g<2>(LOCKS_ARGS); break;
    case 4: launch_decode_g<4>(LOCKS_ARGS); break;
    default: return hipErrorInvalidValue;
  }
#undef LOCKS_ARGS
  return hipGetLastError();
}

}  // namespace locks
