// LOCKS decode step in one launch (gfx950): for ranks 4, 8 and 16 the page
// scores (score workgroups first in the grid, the tile code of the score
// kernel), then page selection, sparse attention over the selected pages and
// the merge of the split partials; for other ranks the same selection and
// attention after a separate score kernel.
//
// [N] = LOCKS reading notes (zhongzhuzhou.org 2026-07-29): §4.4 Algorithm 2
// (query-aware selection of the sink page, the most recent page and the
// top-(k-2) pages by the group-shared estimate of eq. 5), then §3.1 eq. 1
// (softmax attention renormalised over the selected set S).
//
// nsplit in {8, 16, 32} workgroups of 512 threads per (sequence, KV head),
// whose ids interleave up to 8 heads (id = h % 8 + 8 x + ...): with the score
// grid's heads-first order, every workgroup of head h then runs on the XCD
// that wrote its inputs. The nsplit workgroups of one head split the work:
// workgroup x
// owns the page slice [x * slice, (x + 1) * slice) (slice <= 512, one page
// per thread), selects within it and attends its own selected pages. They
// exchange data through a per-(sequence, head) mailbox in the workspace whose
// slots carry their own "written" tag (the score workgroups or the score
// kernel of the same step zero them), so a reader waits for exactly the data
// it needs:
//   1. slice histograms of the key bins (count + 1 per bin), each with the
//      slice's top candidates (key, page + 1) up to a cut-off bin: every
//      workgroup sums the histograms, finds the crossing bin t of the
//      top-(k-2) count, and knows each slice's count in t;
//   2. when only part of bin t is taken, its candidates: from the top lists
//      when every cut-off lies beyond t, else published by each slice. Every
//      workgroup ranks them (part B) while its part-A pages are already being
//      attended, then attends its slice's part-B members;
//   3. the workgroup partials, normalised (o = acc / l, lse = m + log2 l),
//      one word per element that carries o and the complemented bits of the
//      log-sum (its tag): each workgroup polls those of its 1/nsplit share of
//      the output elements and merges them in split order.
// Mailbox accesses are agent-scope relaxed atomics (coherent across the XCDs
// without cache write-back or invalidation); a tagged 64-bit slot is written
// and read whole, so its value is valid once its tag is. Waits poll with a
// bound: a timeout (it needs a member of the group that never starts, e.g.
// when another kernel holds the compute units) skips the rest of the
// selection, writes NaN instead of hanging and poisons the workspace (see the
// step region below). Progress: the members of a group lie within a window of
// HL nsplit (<= 256, HL = min(H, 8)) consecutive workgroup ids and each XCD
// starts its workgroups in id order, so the lowest unfinished group always has
// all its members running while the device can hold HL nsplit workgroups at
// once; the host takes the separate select and attention launches on a device
// that cannot (decode_resident_capacity). A crossing bin of more than 512
// candidates (degenerate keys) goes through a counted barrier instead and an
// exact 8-bit radix select on the order-preserving key bits.
//
// Inputs from the score part (decode layout): per page j and query g,
// e_jg = 2^(s_jg - m_j) with m_j = max_g s_jg (base-2 scores), and m_j; per
// score tile (128 pages, or 32 in a fused launch with 8 splits) and query,
// the base-2 (max, sum) of the scores.
//
// Selection, in base-2 units:
//   1. log2 Z_g from the tile partials (every wave reduces them by itself);
//   2. key_j = log2 mean_g 2^(s_jg - log2 Z_g)
//            = m_j - Zx + log2(sum_g e_jg W_g) - log2 G, W_g = 2^(Zx - log2 Z_g),
//      Zx = max_g log2 Z_g, for candidates 1..P-2 (one log2 per page; exact
//      while the group's log2 Z_g lie within 126 of each other). Keys are
//      log-shares, so key_j <= 0;
//   3. bin_j = floor(-key_j * 16), clamped to [0, 511] (1/16 wide,
//      order-preserving); exchange 1; every wave scans the summed histogram;
//   4. part A = sink, recent and the candidates below bin t (all of bin t
//      when it fits);
//   5. part B = the `need` largest keys of bin t, lower page first on ties:
//      ranked from the slices' top candidates (published with exchange 1)
//      when they hold all of bin t, else after exchange 2 of its candidates.
// When every page is selected (k >= P) there is no selection and workgroup x
// attends the pages [x * per_wg, (x + 1) * per_wg) instead. The selection
// output, when asked for, is the ascending list: each workgroup writes its
// slice's pages after the part-A counts of the earlier slices (published with
// their tag) and their part-B members.
#include <atomic>

#include "locks_attn_core.h"
#include "locks_score_tile.h"
#include "locks_select.h"
#include "locks_step.h"

namespace locks {

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecMaxBudget = 2048;
constexpr int kDecMaxSplits = 32;
constexpr int kDecMaxPpw = 8;       // positions per wave when every page is selected
constexpr float kDecBinsPerUnit = 16.f;
constexpr int kHistCopies = 8;      // lanes spread their histogram atomics over 8 copies
constexpr int kFastCand = kDecThreads;  // crossing-bin candidates exchanged through tagged slots
constexpr int kSpinMax = 1 << 22;   // polls, each a coherent load and a 64-clock sleep
static_assert(kBins == kDecThreads, "one histogram bin per thread");
constexpr uint64_t kTopEmpty = 0xFFFFFFFFull << 32;  // unused top-candidate slot

// Bin of a key (<= 0, or -inf): floor(-key * 16) clamped to [0, 511]. The
// publisher of a top candidate and its readers call this same function.
__device__ __forceinline__ int dec_bin(float key) {
  const float d = -key * kDecBinsPerUnit;  // >= 0 up to rounding; +inf for -inf keys
  return d < (float)(kBins - 1) ? (d > 0.f ? (int)d : 0) : kBins - 1;
}

// Mailbox words of one (sequence, KV head) and G queries per head. Zeroed by
// the score part of the step (score workgroups or the score kernel): the counters [kCoopCounters][kCoopCtrWords], slice
// histograms [nsplit][512], part-A counts [32], fast candidates [512], the
// slices' top candidates [nsplit][512 / nsplit] and the split partials
// [nsplit][G][128] (the last three 64-bit; a partial word carries its
// split's log-sum, see the merge).
// Not zeroed: the large-bin candidates (key bits, page) [MP] each.
__host__ __device__ inline int64_t coop_part_offset(int nsplit) {
  return (int64_t)kCoopCounters * kCoopCtrWords + (int64_t)nsplit * kBins + kDecMaxSplits + 2 * kFastCand +
         2 * kDecThreads;
}
__host__ __device__ inline int64_t coop_zero_words(int nsplit, int G) {
  return coop_part_offset(nsplit) + 2LL * nsplit * G * kHeadDim;
}
// After the zeroed words: the step region (not zeroed) of a fused launch,
// [0] the epoch (see step_tag), [1] the poison word and [32 ..) one
// completion flag per score workgroup of the head; then the large-bin
// candidates. A workgroup whose bounded wait timed out stores kPoison in the
// poison word; every later launch on the workspace then skips its waits and
// writes NaN, until the caller zeroes the workspace. (After a timeout a late
// score workgroup of the same launch may read the next epoch and leave a flag
// that the next launch would take for its own.)
constexpr int kStepWords = 128;
constexpr uint32_t kPoison = 0x504F4953u;  // not a value a zeroed or stale-filled workspace holds by chance
constexpr int kMaxScorePairs = 64;  // one polling lane each
// Pages per score tile in a fused launch with nsplit selection workgroups per
// head: 32 for the smallest split count (tables of at most 8 x 512 pages), so
// that a short table still spreads its summary reads over enough compute
// units (a workgroup's reads are bounded by the loads it keeps in flight,
// not by the memory's bandwidth); 128 otherwise.
__host__ __device__ constexpr int step_tile_pages(int nsplit) { return nsplit <= 8 ? 32 : 128; }
__host__ __device__ inline int64_t coop_mailbox_words(int nsplit, int G, int MP) {
  return (coop_zero_words(nsplit, G) + kStepWords + 2LL * MP + 31) / 32 * 32;
}
// Completion tag of epoch E: a bijective scramble, so a flag left by another
// epoch, zeroed memory or a small count never reads as this epoch's tag.
__host__ __device__ inline uint32_t step_tag(uint32_t E) { return (E * 0x9E3779B1u) ^ 0x5BD1E995u; }
__device__ __forceinline__ uint64_t* mb_part(uint32_t* mb, int nsplit) {
  return reinterpret_cast<uint64_t*>(mb + coop_part_offset(nsplit));
}

// ---- coherent mailbox accesses (agent-scope relaxed atomics)
__device__ __forceinline__ void st_coh(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coh64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_cohf(float* p, float v) {
  st_coh(reinterpret_cast<uint32_t*>(p), __float_as_uint(v));
}
__device__ __forceinline__ float ld_cohf(const float* p) {
  return __uint_as_float(ld_coh(reinterpret_cast<const uint32_t*>(p)));
}

// Arrival of the whole workgroup at counter c after every wave's mailbox
// stores have completed; returns the count before this arrival to every thread.
__device__ __forceinline__ uint32_t coop_arrive(uint32_t* c, uint32_t* sh) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) *sh = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *sh;
}

// Bounded wait (thread 0 polls) until counter c reaches `target`; false on a timeout.
__device__ __forceinline__ bool coop_wait(const uint32_t* c, uint32_t target, uint32_t* sh) {
  if (threadIdx.x == 0) {
    uint32_t okv = 0u;
    for (int it = 0; it < kSpinMax; ++it) {
      if (ld_coh(c) >= target) { okv = 1u; break; }
      __builtin_amdgcn_s_sleep(1);
    }
    *sh = okv;
  }
  __syncthreads();
  return *sh != 0u;
}

// Attention of one wave over list entries e = first, first + step, ... < cnt
// (pages and block ids in LDS), the next page loading while one is computed.
// Chunks of up to four pages are unrolled with two register buffers: every
// load is either followed by its use on the straight path or skipped by a
// forward exit, so the compiler's memory wait counts stay exact (a loop back
// edge would make it wait for everything at the top of every iteration).
__device__ __forceinline__ void attn_list(AttnAcc& acc, const AttnQ& qw,
                                          const uint16_t* __restrict__ kpool,
                                          const uint16_t* __restrict__ vpool, const int* lpage,
                                          const int* lblk, int first, int step, int cnt, int P,
                                          int len, int H, int h, int64_t num_blocks, int lane) {
  constexpr int kU = 4;  // pages per unrolled chunk
  // element offset of entry e (0 for an invalid entry, whose page is skipped)
  auto off_of = [&](int e, int& nv) -> int64_t {
    const int pj = lpage[e], blk = lblk[e];
    const bool valid = pj >= 0 && pj < P && blk >= 0 && blk < num_blocks;
    nv = !valid ? 0 : (pj == P - 1) ? len - kPage * (P - 1) : kPage;
    return valid ? ((int64_t)blk * H + h) * (kPage * kHeadDim) : 0;
  };
  for (int base = first; base < cnt; base += kU * step) {
    PageRegs b0, b1;
    int nv0, nv1;
    attn_load_page(b0, kpool, vpool, off_of(base, nv0), lane);
    if (base + step >= cnt) {
      if (nv0 > 0) attn_page(acc, b0, qw, nv0, lane);
      continue;
    }
    attn_load_page(b1, kpool, vpool, off_of(base + step, nv1), lane);
    if (nv0 > 0) attn_page(acc, b0, qw, nv0, lane);
    if (base + 2 * step >= cnt) {
      if (nv1 > 0) attn_page(acc, b1, qw, nv1, lane);
      continue;
    }
    attn_load_page(b0, kpool, vpool, off_of(base + 2 * step, nv0), lane);
    if (nv1 > 0) attn_page(acc, b1, qw, nv1, lane);
    if (base + 3 * step >= cnt) {
      if (nv0 > 0) attn_page(acc, b0, qw, nv0, lane);
      continue;
    }
    attn_load_page(b1, kpool, vpool, off_of(base + 3 * step, nv1), lane);
    if (nv0 > 0) attn_page(acc, b0, qw, nv0, lane);
    if (nv1 > 0) attn_page(acc, b1, qw, nv1, lane);
  }
}

// Score pairs (two tiles of TP pages) that hold scored pages of a sequence
// of len tokens: at least one (it appends the new token and sets a flag).
__device__ __forceinline__ int step_pairs_needed(int len, int lag, int TP, int npairs) {
  const int tiles = (scored_pages(len, lag) + TP - 1) / TP;
  return min(max((tiles + 1) / 2, 1), npairs);
}

// Decode workgroups of a head that hold pages (or, when every page is
// selected, positions) of a sequence of P pages: the others leave at once
// and the exchanges and the merge run over these only (at least one, which
// writes the outputs of an empty sequence).
__device__ __forceinline__ int decode_wgs_needed(int P, bool sel_all, int slice, int per_wg, int nsplit) {
  const int a = sel_all ? (P + per_wg - 1) / per_wg : (P + slice - 1) / slice;
  return min(max(a, 1), nsplit);
}

// The score part of a fused launch: workgroup (h, pair) scores the tiles
// 2 pair and 2 pair + 1 of head h (waves 0-3 and 4-7), writes the decode-layout
// outputs and the tiles' Z partials, zeroes its share of the head's mailbox,
// and, once every store of the workgroup has completed, sets its completion
// flag to the tag of the head's current epoch. Everything a decode workgroup
// reads from it (score outputs, Z partials, the appended K/V row, mailbox
// zeros) is written with agent-scope stores, which reach memory before the
// flag, so the two may run on different XCDs.
template <int R, int G, int TP>
__device__ __forceinline__ void step_score_part(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ summ,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ escore, float* __restrict__ pmax, float2* __restrict__ zpart, int ntiles,
    int64_t num_blocks, int H, int MP, int npairs, const uint16_t* __restrict__ knew,
    const uint16_t* __restrict__ vnew, uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool,
    CoopZero coop, uint32_t* step, int lag, int hdiv, int bid, int s, bool trim) {
  const int h = bid % H, pair = bid / H;
  const int64_t sh_idx = (int64_t)s * H + h;
  // With trim (a launch over several sequences, sized by the longest), the
  // pairs past this sequence's scored pages leave at once: the selection
  // workgroups wait only for the flags of the first npz pairs, which zero
  // the mailbox among themselves.
  int npz = npairs;
  if (trim) {
    npz = step_pairs_needed(clampi(seq_lens[s], 0, MP * kPage), lag, TP, npairs);
    if (pair >= npz) return;
  }
  uint32_t E = 0u;  // the head's epoch, read and used by thread 0 only
  if (threadIdx.x == 0) E = ld_coh(step);
  zero_coop_mailbox(coop, sh_idx, pair, npz);
  const int sub = threadIdx.x >> 8, tid = threadIdx.x & 255, wave = tid >> 6, lane = tid & 63;
  const int tile = 2 * pair + sub;
  float zm = -__builtin_inff(), zs = 0.f;
  if (tile < ntiles)
    score_tile<R, G, TP>(q, summ, table, seq_lens, escore, num_blocks, H, MP, step_row_pages(MP),
                     (lag ? kScoreDeferred : 0) | (hdiv << kScoreHeadDivShift), knew, vnew, kpool, vpool, pmax, s, h, tile, wave,
                     tid, zm, zs);
  __shared__ float zred[2][4][4][2];
  if (lane < G) {
    zred[sub][wave][lane][0] = zm;
    zred[sub][wave][lane][1] = zs;
  }
  __syncthreads();
  if (tid < G && tile < ntiles) {
    float m = zred[sub][0][tid][0], t = zred[sub][0][tid][1];
    for (int w = 1; w < 4; ++w) lse2_merge(m, t, zred[sub][w][tid][0], zred[sub][w][tid][1]);
    // padded layout: 64 bytes per tile, so a 128-byte line holds the two
    // tiles of one workgroup and no other writer's data
    st_coh64(reinterpret_cast<uint64_t*>(zpart + (sh_idx * 2 * npairs + tile) * 8 + tid),
             (uint64_t)__float_as_uint(m) | ((uint64_t)__float_as_uint(t) << 32));
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) st_coh(&step[32 + pair], step_tag(E));
}

// R > 0: one fused launch per step, the score workgroups first (H x npairs,
// heads first), then the decode workgroups, which wait for their head's
// score workgroups. R = 0: the decode workgroups alone, after a separate
// score kernel. Grid row z holds sequence z's score workgroups, then the
// decode workgroups of sequence z - dshift. With several sequences and a
// score part, dshift = 1 (S + 1 rows): the dispatcher starts workgroups in
// row order, so a sequence's decode workgroups start after the next
// sequence's score workgroups, when their own scores are about done, instead
// of holding compute units that the next score reads wait for. Each
// workgroup still waits only for earlier ones (its sequence's score
// workgroups) and its own contiguous decode group.
template <int R, int G, int kS>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(
    float* __restrict__ escore, float* __restrict__ pmax, float2* __restrict__ zpart, int ntiles,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ budgets,
    const uint16_t* __restrict__ q, uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool,
    const int32_t* __restrict__ table, int64_t num_blocks, int H, int MP, int max_budget,
    int slice, int per_wg, uint32_t* __restrict__ mbox, float* __restrict__ out,
    float* __restrict__ lse_out, int32_t* __restrict__ sel_pages, int32_t* __restrict__ sel_count,
    const uint8_t* __restrict__ summ, int npairs, const uint16_t* __restrict__ knew,
    const uint16_t* __restrict__ vnew, CoopZero coop, int lag, int rule, int hdiv, int dshift) {
  constexpr int nsplit = kS;
  constexpr int kTop = kDecThreads / kS;  // top-candidate slots per slice
  static_assert(kTop * kS == kDecThreads, "one top-candidate slot per thread");
  const int n_score = (R > 0) ? H * npairs : 0;
  if constexpr (R > 0) {
    if ((int)blockIdx.x < n_score) {
      // (the score part of the extra last row, dshift = 1, is empty)
      if ((int)blockIdx.z >= (int)gridDim.z - dshift) return;
      uint32_t* step = mbox + ((int64_t)blockIdx.z * H + (int)blockIdx.x % H) * coop_mailbox_words(nsplit, G, MP) +
                       coop_zero_words(nsplit, G);
      step_score_part<R, G, step_tile_pages(kS)>(q, summ, table, seq_lens, escore, pmax, zpart, ntiles, num_blocks, H, MP,
                            npairs, knew, vnew, kpool, vpool, coop, step, lag, hdiv, (int)blockIdx.x, (int)blockIdx.z,
                            dshift != 0);
      return;
    }
  }
  __shared__ uint32_t histc[kHistCopies][kBins + 1];  // padded: copy c of bin b in bank (b + c) % 32
  __shared__ __align__(16) uint32_t hist[kBins];
  __shared__ uint4 sh_q[G * kHeadDim / 8];
  __shared__ float cand_key[kFastCand];
  __shared__ uint32_t cand_page[kFastCand];
  __shared__ int att_page[kDecThreads];  // part-A pages to attend (or the positions) and their blocks
  __shared__ int att_blk[kDecThreads];
  __shared__ int b_page[kDecThreads];    // this slice's part-B members and their blocks
  __shared__ int b_blk[kDecThreads];
  __shared__ int cs_page[kDecWaves], cs_blk[kDecWaves];  // the slice's first crossing-bin candidates
  __shared__ int cs_mem[kDecWaves];                      // ... and whether they are members
  __shared__ int my_blk[kDecThreads];    // block id of slice page tid
  __shared__ uint32_t slice_bits[kDecThreads / 32];  // selected pages of the slice (output)
  __shared__ int sh_cbase[kS + 1];  // crossing-bin candidates before slice y
  __shared__ int sh_waves[16];
  __shared__ int sh_wa[kDecWaves], sh_wc[kDecWaves], sh_wt[kDecWaves];
  __shared__ uint32_t sh_vote[kDecWaves];  // exchange 1: a wave still missing data
  __shared__ int sh_nocov;  // some slice's top candidates stop before the crossing bin
  __shared__ int sh_int[8];
  __shared__ uint32_t sh_u[2];
  __shared__ uint32_t sh_ready;
  __shared__ float sh_acc[kDecWaves][G][kHeadDim];
  __shared__ float sh_ml[kDecWaves][G][2];

  // workgroup ids interleave up to HL = 8 heads: id = h % HL + HL (x + nsplit (h / HL))
  const int HL = H < 8 ? H : 8;
  const int bid = (int)blockIdx.x - n_score;
  const int hr = bid / (HL * nsplit), rr = bid % (HL * nsplit);
  const int h = hr * HL + rr % HL, x = rr / HL, s = (int)blockIdx.z - dshift;
  if (s < 0) return;  // the decode part of the first row, dshift = 1, is empty
  if (h >= H) return;  // padding of the last head row
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t sh_idx = (int64_t)s * H + h;
  const int hd = h / hdiv, Hd = H / hdiv;  // the pools' head of this head (score_head_div)
  uint32_t* mb = mbox + sh_idx * coop_mailbox_words(nsplit, G, MP);
  uint32_t* ctr = mb;                                            // [kCoopCounters][kCoopCtrWords]
  uint32_t* mb_hist = ctr + kCoopCounters * kCoopCtrWords;       // [nsplit][512], count + 1
  uint32_t* mb_acnt = mb_hist + nsplit * kBins;                  // [32], part-A count + 1
  uint64_t* mb_cand = reinterpret_cast<uint64_t*>(mb_acnt + kDecMaxSplits);  // [512]: key | (page + 1) << 32
  uint64_t* mb_top = mb_cand + kFastCand;  // [nsplit][kTop]: key | (page + 1) << 32, last: sbin | 1 << 32
  uint32_t* mb_step = mb + coop_zero_words(nsplit, G);                       // epoch, score flags
  uint32_t* mb_bkey = mb_step + kStepWords;                                   // [MP] (large bin)
  uint32_t* mb_bpage = mb_bkey + MP;                                          // [MP] (large bin)

  // ---- loads that need no score output first: length, budget, the block id
  // of this thread's page (clamped, so the loads are unconditional), queries
  // (the epoch and the poison word, adjacent, by one lane per wave: every
  // workgroup of the head reads them, and one request per wave keeps their
  // line from being a hot spot)
  uint64_t epw = 0ull;
  if (lane == 0) epw = ld_coh64(reinterpret_cast<const uint64_t*>(mb_step));
  epw = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(epw >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)epw);
  const uint32_t epoch = (R > 0) ? (uint32_t)epw : 0u;
  const bool poisoned = (uint32_t)(epw >> 32) == kPoison;
  const int len_raw = seq_lens[s];
  const int bud_raw = budgets[s];
  const int len = clampi(len_raw, 0, MP * kPage);
  const int P = (len + kPage - 1) / kPage;
  const int k = clampi(bud_raw, 2, max_budget);
  const bool sel_all = (P == 0 || k >= P);
  // the head's workgroups with pages of this sequence (the others have
  // nothing to attend or publish: they leave below, before the flags wait and
  // without touching the mailbox, once the loads here are all issued)
  const int act = decode_wgs_needed(P, sel_all, slice, per_wg, nsplit);
  // (over several sequences, a workgroup without pages leaves before any
  // other load: short sequences leave many of them)
  if (dshift && x >= act) return;
  const int j = x * slice + tid;  // this thread's page
  const bool jin = tid < slice && j < MP;
  const int jj = jin ? j : 0;
  const int bk = table[(int64_t)s * MP + jj];
  if (tid < G * kHeadDim / 8) sh_q[tid] = reinterpret_cast<const uint4*>(q + sh_idx * G * kHeadDim)[tid];
  for (int i = tid; i < kHistCopies * (kBins + 1); i += kDecThreads) (&histc[0][0])[i] = 0u;
  if (tid < kDecThreads / 32) slice_bits[tid] = 0u;
  if (tid == 0) {
    sh_nocov = 0;
    sh_int[4] = 0;  // part B: members of this slice and of the slices before it
    sh_int[5] = 0;
    sh_u[1] = 1u;   // the fast ranking received every candidate
  }
  my_blk[tid] = bk;
  if (x >= act) return;
  bool ok = !poisoned;  // false after a timed-out wait (here or in an earlier launch)
  if constexpr (R > 0) {
    // ---- wait (bounded) for the head's score workgroups of this epoch
    // the score pairs of this sequence that set a flag (all of them unless
    // the launch trims them, as the score part does)
    const int npz = dshift ? step_pairs_needed(len, lag, step_tile_pages(kS), npairs) : npairs;
    if (wave == 0 && !poisoned) {
      const uint32_t want = step_tag(epoch);
      uint32_t done = 0u;
      for (int it = 0; it < kSpinMax; ++it) {
        const uint32_t v = (lane < npz) ? ld_coh(&mb_step[32 + lane]) : want;
        if (__ballot(v != want) == 0ull) {
          done = 1u;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane == 0) sh_ready = done;
    }
    else if (wave == 0 && lane == 0) sh_ready = 0u;
    __syncthreads();
    ok = sh_ready != 0u;
  }
  // ---- the tile Z partials, and the e and m of this thread's page. In a
  // fused launch they come from this launch's score workgroups, complete now:
  // each 128-byte line of them has one writer (a score workgroup, which stored
  // it coherently), and no workgroup on this XCD read the line earlier in the
  // launch, so plain loads return the written values (the caches hold no copy
  // from before the launch).
  const float2* zp = zpart + ((R > 0) ? sh_idx * 2 * npairs * 8 : sh_idx * ntiles * G);
  const int zstride = (R > 0) ? 8 : G;  // float2 per tile
  constexpr int kTP = (R > 0) ? step_tile_pages(kS) : kScorePagesPerWg;  // pages per tile
  // the table holds at most kS x 512 pages (decode_shape)
  constexpr int kZl = (kS * kDecThreads + 64 * kTP - 1) / (64 * kTP);
  float2 zl[kZl][G];  // tile partials t = lane + 64 c
#pragma unroll
  for (int c = 0; c < kZl; ++c) {
    const int t = min(lane + 64 * c, ntiles - 1);
#pragma unroll
    for (int g = 0; g < G; ++g) zl[c][g] = zp[t * zstride + g];
  }
  float ev[G];
  const int rowp = (R > 0) ? step_row_pages(MP) : MP;  // score output row length
  load_scores<G>(escore + (sh_idx * rowp + jj) * G, ev);
  const float mv = pmax[sh_idx * rowp + jj];

  const int F = scored_pages(len, lag);  // summarised pages (pages 0..P-2 are among them)
  bool in = false;      // this thread's page is in part A
  int natt = 0;         // pages in att_page (part A, or the positions when every page is selected)
  int tbin = -1, need = 0, ct = 0;
  bool part_bin = false;
  bool lds_b = false;   // the crossing bin's candidates came with exchange 1 (in cand_key/cand_page)

  AttnQ qw;
  AttnAcc acc;
  attn_init(acc);

  if (sel_all) {
    // positions = pages: workgroup x attends [x * per_wg, (x + 1) * per_wg)
    const int lo = x * per_wg;
    natt = clampi(P - lo, 0, per_wg);
    if (tid < natt) {
      att_page[tid] = lo + tid;
      att_blk[tid] = table[(int64_t)s * MP + lo + tid];
    }
    __syncthreads();
  } else {
    // From here P >= 3, k < P and pages 0..P-2 are full (F >= P-1).
    // ---- 1. log2 Z_g over the F full pages (tiles beyond F hold nothing)
    const int ntu = (F + kTP - 1) / kTP;
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
    // group-mass: log2 sum_g Z_g
    float ztot = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) ztot += (lz[g] == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(lz[g] - zx);
    ztot = zx + __builtin_amdgcn_logf(ztot);
    // ---- 2. key (<= 0) and bin of this thread's page: the share average of
    // eq. 5, or the group-max / group-mass alternatives
    const bool cand = jin && j >= 1 && j <= P - 2;
    float key;
    int bin;
    {
      float t = 0.f;
      if (rule == kMergeMax) {
#pragma unroll
        for (int g = 0; g < G; ++g) t = fmaxf(t, ev[g] * wg[g]);
      } else if (rule == kMergeMass) {
#pragma unroll
        for (int g = 0; g < G; ++g) t += ev[g];
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) t = fmaf(ev[g], wg[g], t);
      }
      float kj = (rule == kMergeMax)    ? (mv - zx) + __builtin_amdgcn_logf(t)
                 : (rule == kMergeMass) ? mv + __builtin_amdgcn_logf(t) - ztot
                                        : (mv - zx) + (__builtin_amdgcn_logf(t) - log2G);
      kj = (cand && kj == kj) ? kj : -__builtin_inff();
      key = kj;
      bin = dec_bin(kj);
    }
    // ---- 3. slice histogram (candidates only), published; exchange 1
    // (the zeroed copies are visible here: in a fused launch the barrier of
    // the flags wait came after the zeroing)
    if constexpr (R == 0) __syncthreads();
    if (cand) atomicAdd(&histc[lane & (kHistCopies - 1)][bin], 1u);
    __syncthreads();
    {
      uint32_t t = 1u;  // the written tag
#pragma unroll
      for (int c = 0; c < kHistCopies; ++c) t += histc[c][tid];
      st_coh(&mb_hist[x * kBins + tid], t);
      hist[tid] = t - 1u;
    }
    // ---- the slice's top candidates, published beside its histogram: the
    // candidates of the bins before sbin, the first bin at which the slice's
    // running count exceeds kTop - 1, in page order; the last slot holds sbin.
    // When every slice's sbin lies beyond the crossing bin, all the crossing
    // bin's candidates are among them and its ranking needs no second exchange.
    __syncthreads();
    {
      const uint4 h0 = *reinterpret_cast<const uint4*>(&hist[8 * lane]);
      const uint4 h1 = *reinterpret_cast<const uint4*>(&hist[8 * lane + 4]);
      const int c8[8] = {(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w,
                         (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
      int tot = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) tot += c8[e];
      int run = wave_inclusive_scan(tot) - tot, fb = -1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        run += c8[e];
        if (fb < 0 && run > kTop - 1) fb = 8 * lane + e;
      }
      const uint64_t found = __ballot(fb >= 0);
      const int sbin = found ? __builtin_amdgcn_readlane(fb, __builtin_ctzll(found)) : kBins;
      const bool pub = cand && bin < sbin;  // at most kTop - 1 of them
      const uint64_t balP = __ballot(pub);
      if (lane == 0) sh_wt[wave] = __popcll(balP);
      __syncthreads();
      int preP = 0, totP = 0;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        preP += (w < wave) ? sh_wt[w] : 0;
        totP += sh_wt[w];
      }
      uint64_t* top = mb_top + x * kTop;
      if (pub) {
        const int pos = preP + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(balP >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)balP, 0u));
        st_coh64(&top[pos], (uint64_t)__float_as_uint(key) | ((uint64_t)(j + 1) << 32));
      }
      if (tid >= totP && tid < kTop - 1) st_coh64(&top[tid], kTopEmpty);
      if (tid == kTop - 1) st_coh64(&top[tid], (1ull << 32) | (uint32_t)sbin);
    }
    // every slice's count of bin tid (kept in registers) and top-candidate
    // slot tid (slice tid / kTop)
    uint32_t hy[kS] = {};
    uint64_t tv = 0ull;
    {
      uint32_t pending = ok ? 1u : 0u;  // a workgroup that already failed does not wait
      for (int it = 0; pending && it < kSpinMax; ++it) {
        pending = 0u;
#pragma unroll
        for (int y = 0; y < kS; ++y) {
          // (an absent slice reads as empty; its load is kept unconditional:
          // the mailbox holds every slice's words, zeroed in this step)
          const uint32_t w = ld_coh(&mb_hist[y * kBins + tid]);
          hy[y] = (y < act) ? w : 1u;
          pending |= (hy[y] == 0u) ? 1u : 0u;
        }
        // (the top list of an absent slice: empty, cut off at no bin)
        const uint64_t tw = ld_coh64(&mb_top[tid]);
        tv = (tid / kTop < act) ? tw : (tid % kTop == kTop - 1) ? ((1ull << 32) | (uint32_t)kBins) : kTopEmpty;
        pending |= ((tv >> 32) == 0ull) ? 1u : 0u;
        if (pending) __builtin_amdgcn_s_sleep(1);
      }
      // the summed histogram and every wave's vote on "all arrived" share one
      // barrier (the counts are only used when the vote passes)
      const uint64_t miss = __ballot(pending != 0u);
      uint32_t t = 0u;
#pragma unroll
      for (int y = 0; y < kS; ++y) {
        hy[y] -= 1u;
        t += hy[y];
      }
      hist[tid] = t;
      if (lane == 0) sh_vote[wave] = miss != 0ull ? 1u : 0u;
    }
    __syncthreads();
    {
      uint32_t any = 0u;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) any |= sh_vote[w];
      ok = ok && any == 0u;
    }
    if (ok) {
      // ---- crossing bin: every wave scans the histogram itself (lane l
      // holds bins 8l .. 8l+7), so no broadcast is needed
      const int need0 = k - 2;
      if (need0 > 0) {
        const uint4 h0 = *reinterpret_cast<const uint4*>(&hist[8 * lane]);
        const uint4 h1 = *reinterpret_cast<const uint4*>(&hist[8 * lane + 4]);
        const int c8[8] = {(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w,
                           (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
        int tot = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) tot += c8[e];
        int before = wave_inclusive_scan(tot) - tot;
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
      part_bin = (tbin >= 0) && (need < ct);
      if (tid == tbin) {  // crossing-bin candidates before each slice
        int c = 0;
#pragma unroll
        for (int y = 0; y < kS; ++y) {
          sh_cbase[y] = c;
          c += (int)hy[y];
        }
        sh_cbase[kS] = c;
      }
      // ---- 4. part A of this slice, in page order (wave ballots), and the
      // crossing bin's candidates, published
      in = jin && j < P &&
           ((j == 0) | (j == P - 1) | (cand & (bin < tbin)) | ((tbin >= 0) & (need == ct) & cand & (bin == tbin)));
      const uint64_t balA = __ballot(in);
      // the crossing bin's candidates among the published top candidates
      const bool tmark = tid % kTop == kTop - 1;
      const float tkey = __uint_as_float((uint32_t)tv);
      const bool te = part_bin && ct <= 64 && !tmark && (tv & kTopEmpty) != kTopEmpty && dec_bin(tkey) == tbin;
      const uint64_t balT = __ballot(te);
      if (lane == 0) {
        sh_wa[wave] = __popcll(balA);
        sh_wt[wave] = __popcll(balT);
      }
      if (tmark && part_bin && (int)(uint32_t)tv <= tbin) sh_nocov = 1;
      __syncthreads();
      int preA = 0, totA = 0, preT = 0, totT = 0;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        preA += (w < wave) ? sh_wa[w] : 0;
        totA += sh_wa[w];
        preT += (w < wave) ? sh_wt[w] : 0;
        totT += sh_wt[w];
      }
      // the same decision in every workgroup of the head: all its inputs are
      // the exchanged histograms and top candidates
      lds_b = part_bin && ct <= 64 && sh_nocov == 0 && totT == ct;
      if (lds_b && te) {  // the candidate list, in slice and page order
        const int pos = preT + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(balT >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)balT, 0u));
        const uint32_t pg = (uint32_t)(tv >> 32) - 1u;
        cand_key[pos] = tkey;
        cand_page[pos] = pg;
        // this slice's first candidates, loaded ahead by wave kc (part 5)
        const int kc = pos - sh_cbase[x];
        if (kc >= 0 && kc < kDecWaves && kc < sh_cbase[x + 1] - sh_cbase[x]) {
          cs_page[kc] = (int)pg;
          cs_blk[kc] = my_blk[clampi((int)pg - x * slice, 0, kDecThreads - 1)];
        }
      }
      if (in) {
        const int pos = preA + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(balA >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)balA, 0u));
        att_page[pos] = j;
        att_blk[pos] = bk;
        atomicOr(&slice_bits[tid >> 5], 1u << (tid & 31));
      }
      natt = totA;
      if (tid == 0) st_coh(&mb_acnt[x], (uint32_t)totA + 1u);
      if (part_bin && !lds_b) {
        const bool isc = cand && bin == tbin;
        const uint64_t balC = __ballot(isc);
        if (lane == 0) sh_wc[wave] = __popcll(balC);
        __syncthreads();
        int preC = 0;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) preC += (w < wave) ? sh_wc[w] : 0;
        if (isc) {
          const int kc = preC + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(balC >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)balC, 0u));
          const int cpos = sh_cbase[x] + kc;
          if (kc < kDecWaves) {  // loaded ahead by wave kc, in case it is a member
            cs_page[kc] = j;
            cs_blk[kc] = bk;
          }
          if (ct <= kFastCand)
            st_coh64(&mb_cand[cpos], (uint64_t)__float_as_uint(key) | ((uint64_t)(j + 1) << 32));
          else {
            st_coh(&mb_bkey[cpos], __float_as_uint(key));
            st_coh(&mb_bpage[cpos], (uint32_t)j);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- 5. part B: membership of every candidate of the crossing bin (page
  // order); this slice's members go to b_page, members before this slice are
  // counted. A bin of up to 64 candidates is ranked by the last wave while
  // the others already attend part A; larger bins by the whole workgroup after.
  const int cb_lo = part_bin ? sh_cbase[x] : 0, cb_hi = part_bin ? sh_cbase[x + 1] : 0;
  const bool fast_b = !sel_all && ok && part_bin && ct <= 64;
  attn_load_q<G>(qw, reinterpret_cast<const uint16_t*>(sh_q), lane);
  // the K/V of the slice's first crossing-bin candidates load now (wave k
  // takes candidate k) and are attended if ranking makes them members
  const int nc = fast_b ? min(cb_hi - cb_lo, kDecWaves) : 0;
  PageRegs bspec;
  if (wave < nc) {
    const int pj = cs_page[wave], blk = cs_blk[wave];
    const bool valid = blk >= 0 && blk < num_blocks;  // candidates are full pages
    attn_load_page(bspec, kpool, vpool, valid ? ((int64_t)blk * Hd + hd) * (kPage * kHeadDim) : 0, lane);
  }
  if (fast_b && wave == kDecWaves - 1) {
    // lane e < ct holds candidate e; rank by key (lower page first on ties)
    uint64_t v = 0ull;
    if (lds_b) {
      if (lane < ct) v = (uint64_t)__float_as_uint(cand_key[lane]) | ((uint64_t)(cand_page[lane] + 1u) << 32);
    } else if (lane < ct) {
      for (int it = 0; it < kSpinMax; ++it) {
        v = ld_coh64(&mb_cand[lane]);
        if ((v >> 32) != 0ull) break;
        __builtin_amdgcn_s_sleep(1);
      }
    }
    const bool got = __ballot(lane < ct && (v >> 32) == 0ull) == 0ull;
    const float ck = (lane < ct) ? __uint_as_float((uint32_t)v) : -__builtin_inff();
    const uint32_t cp = (lane < ct) ? (uint32_t)(v >> 32) - 1u : 0xFFFFFFFFu;
    int rank = 0;
    for (int e = 0; e < ct; ++e) {
      const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ck), e));
      const uint32_t op = (uint32_t)__builtin_amdgcn_readlane((int)cp, e);
      rank += ((o > ck) | ((o == ck) & (op < cp))) ? 1 : 0;
    }
    const bool mem = got && lane < ct && rank < need;
    const bool mine_m = mem && lane >= cb_lo && lane < cb_hi;
    const int kc = lane - cb_lo;  // candidate index within the slice
    if (kc >= 0 && kc < nc) {
      const int r = (int)cp - x * slice;
      cs_mem[kc] = (mine_m && my_blk[r] >= 0 && my_blk[r] < num_blocks) ? 1 : 0;
    }
    // members beyond the preloaded ones go to the list
    const bool listed = mine_m && kc >= nc;
    const uint64_t bmine = __ballot(listed);
    if (listed) {
      const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bmine >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bmine, 0u));
      const int r = (int)cp - x * slice;
      b_page[pos] = (int)cp;
      b_blk[pos] = my_blk[r];
    }
    if (mine_m) {
      const int r = (int)cp - x * slice;
      atomicOr(&slice_bits[r >> 5], 1u << (r & 31));
    }
    const uint64_t bbef = __ballot(mem && lane < cb_lo);
    if (lane == 0) {
      sh_int[4] = __popcll(bmine);
      sh_int[5] = __popcll(bbef);
      if (!got) sh_u[1] = 0u;
    }
  }
  // ---- attention over part A (or the positions)
  attn_list(acc, qw, kpool, vpool, att_page, att_blk, wave, kDecWaves, natt, P, len, Hd, hd,
               num_blocks, lane);
  if (!sel_all && ok && part_bin && !fast_b) {
    // membership `mem` of candidate t (page `page`), called by every thread
    // for one chunk of candidates: members before this slice are counted,
    // this slice's members appended (page order)
    auto take = [&](int t, bool mem, int page) {
      const bool mine_m = mem && t >= cb_lo && t < cb_hi;
      int tot;
      const int before = block_exclusive_scan(mine_m ? 1 : 0, sh_waves, &tot);
      if (mem && t < cb_lo) atomicAdd(&sh_int[5], 1);
      if (mine_m) {
        const int r = page - x * slice;
        b_page[sh_int[4] + before] = page;
        b_blk[sh_int[4] + before] = my_blk[r];
        atomicOr(&slice_bits[r >> 5], 1u << (r & 31));
      }
      __syncthreads();
      if (tid == 0) sh_int[4] += tot;
      __syncthreads();
    };
    if (ct <= kFastCand) {
      uint64_t v = 0ull;
      if (tid < ct) {
        for (int it = 0; it < kSpinMax; ++it) {
          v = ld_coh64(&mb_cand[tid]);
          if ((v >> 32) != 0ull) break;
          __builtin_amdgcn_s_sleep(1);
        }
        cand_key[tid] = __uint_as_float((uint32_t)v);
        cand_page[tid] = (uint32_t)(v >> 32) - 1u;
      }
      ok = __syncthreads_and(tid >= ct || (v >> 32) != 0ull);
      if (ok) {
        bool mem = false;
        if (tid < ct) {
          const float me = cand_key[tid];
          const uint32_t mp = cand_page[tid];
          int rank = 0;
          for (int e = 0; e < ct; ++e) {
            const float o = cand_key[e];
            rank += (o > me || (o == me && cand_page[e] < mp)) ? 1 : 0;
          }
          mem = rank < need;
        }
        take(tid, mem, tid < ct ? (int)cand_page[tid] : 0);
      }
    } else {
      // large crossing bin: counted barrier, then an exact 8-bit radix select
      // on the order-preserving key bits over the published candidates
      coop_arrive(&ctr[1 * kCoopCtrWords], &sh_u[0]);
      ok = coop_wait(&ctr[1 * kCoopCtrWords], (uint32_t)act, &sh_u[1]);
      if (ok) {
        uint32_t prefix = 0u;
        int needr = need;
#pragma unroll 1
        for (int shift = 24; shift >= 0; shift -= 8) {
          __syncthreads();
          if (tid < 256) hist[tid] = 0u;
          __syncthreads();
          for (int t = tid; t < ct; t += kDecThreads) {
            const uint32_t o = float_to_ordered(__uint_as_float(ld_coh(&mb_bkey[t])));
            if (shift == 24 || (o >> (shift + 8)) == prefix)
              atomicAdd(&hist[255 - ((o >> shift) & 255u)], 1u);  // descending order
          }
          __syncthreads();
          const int c = (tid < 256) ? (int)hist[tid] : 0;
          int tot;
          const int before = block_exclusive_scan(c, sh_waves, &tot);
          if (tid < 256 && before < needr && before + c >= needr) {
            sh_int[0] = 255 - tid;
            sh_int[1] = needr - before;
          }
          __syncthreads();
          prefix = (prefix << 8) | (uint32_t)sh_int[0];
          needr = sh_int[1];
        }
        // keys above `prefix` are in; of those equal to it, the `needr` first
        // in page order
        int ties = 0;
#pragma unroll 1
        for (int base = 0; base < ct; base += kDecThreads) {
          const int t = base + tid;
          uint32_t o = 0u;
          int page = 0;
          if (t < ct) {
            o = float_to_ordered(__uint_as_float(ld_coh(&mb_bkey[t])));
            page = (int)ld_coh(&mb_bpage[t]);
          }
          const bool eq = t < ct && o == prefix;
          int teq;
          const int tb = block_exclusive_scan(eq ? 1 : 0, sh_waves, &teq);
          take(t, t < ct && (o > prefix || (eq && ties + tb < needr)), page);
          ties += teq;
        }
      }
    }
  }
  __syncthreads();
  const int bbefore = sh_int[5];
  if (fast_b) ok = sh_u[1] != 0u;
  if (ok && wave < nc && cs_mem[wave]) attn_page(acc, bspec, qw, kPage, lane);
  attn_list(acc, qw, kpool, vpool, b_page, b_blk, wave, kDecWaves, sh_int[4], P, len, Hd, hd,
               num_blocks, lane);
  attn_wave_to_lds<G>(acc, sh_acc[wave], sh_ml[wave], lane);
  __syncthreads();

  // ---- the workgroup's partial, normalised: thread (g, d) combines the 8
  // wave partials into o = acc / l and lse = m + log2 l and publishes both in
  // one word, o | ~bits(lse) << 32, that the merging workgroups poll: the
  // complemented log-sum is never 0 (the one float whose complement is 0, a
  // NaN, is stored as the canonical NaN), so a zeroed word reads as absent,
  // and one load per split brings the value and its weight together
  uint64_t* mb_po = mb_part(mb, nsplit);  // [nsplit][G][128]
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
    float o = L > 0.f ? a / L : 0.f;
    if (!ok) o = __builtin_nanf("");
    const float lse = L > 0.f ? M + __builtin_amdgcn_logf(L) : -__builtin_inff();
    uint32_t lb = __float_as_uint(lse);
    if (lb == 0xFFFFFFFFu) lb = 0x7FC00000u;
    st_coh64(&mb_po[(x * G + g) * kHeadDim + d], ((uint64_t)(~lb) << 32) | __float_as_uint(o));
  }

  // ---- selection output: every workgroup writes its slice's selected pages
  // at their places in the ascending list
  if (sel_pages) {
    int32_t* o = sel_pages + sh_idx * max_budget;
    int n;
    if (sel_all) {
      n = P;
      const int lo = x * per_wg;
      if (tid < natt) o[lo + tid] = lo + tid;
    } else {
      // part-A counts of all slices (tagged), and this slice's bitmap
      __syncthreads();
      if (wave == 0) {
        uint32_t a = 1u;
        if (lane < act && ok) {
          for (int it = 0; it < kSpinMax; ++it) {
            a = ld_coh(&mb_acnt[lane]);
            if (a != 0u) break;
            __builtin_amdgcn_s_sleep(1);
          }
        }
        const int av = (a != 0u) ? (int)a - 1 : 0;
        const int ex = wave_inclusive_scan(av) - av;
        if (lane == x) sh_int[6] = ex;
        if (lane == 63) sh_int[7] = ex + av;  // all part-A members
      }
      __syncthreads();
      n = min(sh_int[7] + (part_bin ? need : 0), max_budget);
      const int words = (slice + 31) / 32;
      const uint32_t bw = (tid < words) ? slice_bits[tid] : 0u;
      int tot;
      int before = block_exclusive_scan(__popc(bw), sh_waves, &tot) + sh_int[6] + bbefore;
      uint32_t w = bw;
      while (w) {
        const int b = __builtin_ctz(w);
        w &= w - 1u;
        if (before < max_budget) o[before] = x * slice + 32 * tid + b;
        ++before;
      }
    }
    if (x == 0) {
      for (int i = n + tid; i < max_budget; i += kDecThreads) o[i] = -1;
      if (tid == 0) sel_count[sh_idx] = n;
    }
  }

  // ---- the merge, spread over the head's act workgroups: workgroup x takes
  // the elements [x N / act, (x + 1) N / act) of the N = G x 128 outputs (at
  // least one each, as N >= act); the thread of element e waits (bounded) for
  // the act partials of it and combines them in split order (an absent
  // split: empty)
  constexpr int kN = G * kHeadDim;
  const int e = x * kN / act + tid;
  if (e >= (x + 1) * kN / act) return;
  const int g = e / kHeadDim, d = e % kHeadDim;
  uint64_t po[kS];
  bool got = false;
  constexpr uint64_t kEmpty = (uint64_t)(~0xFF800000u) << 32;  // o = 0, lse = -inf
  for (int it = 0; it < kSpinMax; ++it) {
    uint32_t miss = 0u;
#pragma unroll
    for (int y = 0; y < kS; ++y) {
      // (unconditional loads: the mailbox holds every split's words)
      const uint64_t wo = ld_coh64(&mb_po[(y * G + g) * kHeadDim + d]);
      po[y] = (y < act) ? wo : kEmpty;
    }
#pragma unroll
    for (int y = 0; y < kS; ++y) miss |= (uint32_t)((po[y] >> 32) == 0ull);
    if (miss == 0u) {
      got = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  // one common maximum, then every split's weight 2^(lse_y - max), summed in
  // split order
  float M = -__builtin_inff();
#pragma unroll
  for (int y = 0; y < kS; ++y) M = fmaxf(M, __uint_as_float(~(uint32_t)(po[y] >> 32)));
  float W = 0.f, a = 0.f;
#pragma unroll
  for (int y = 0; y < kS; ++y) {
    const float ly = __uint_as_float(~(uint32_t)(po[y] >> 32));
    const float f = (ly == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(ly - M);
    W += f;
    a = fmaf(__uint_as_float((uint32_t)po[y]), f, a);
  }
  if (!got || !ok) {
    a = __builtin_nanf("");
    if (!poisoned) st_coh(mb_step + 1, kPoison);
  }
  const bool some = W > 0.f;
  out[(sh_idx * G + g) * kHeadDim + d] = some ? a / W : (a == a ? 0.f : a);
  if (lse_out && d == 0)
    lse_out[sh_idx * G + g] = some ? (M + __builtin_amdgcn_logf(W)) * kLn2 : -__builtin_inff();
  // every workgroup of the head has read the epoch (each published a partial
  // after reading it), so the next step's launch may use the next one
  if (R > 0 && x == act - 1 && tid == 0) st_coh(mb_step, epoch + 1u);
}

// Launch shape for a table of MP pages and a budget of KB pages: false when
// the fused step does not apply (the caller then runs the separate select and
// attention kernels). nsplit: the smallest of 8, 16, 32 with slices of at most
// 512 pages and, when every page is selected, at most 8 positions per wave.
bool decode_shape(int MP, int KB, int* per_wg, int* nsplit, int* slice) {
  if (MP > kDecMaxSplits * kDecThreads || KB > kDecMaxBudget) return false;
  int ns = 8;
  while (ns < kDecMaxSplits && ((MP + ns - 1) / ns > kDecThreads || (KB + ns - 1) / ns > kDecWaves * kDecMaxPpw))
    ns *= 2;
  *nsplit = ns;
  *slice = (MP + ns - 1) / ns;
  *per_wg = (KB + ns - 1) / ns;
  return true;
}

int decode_max_splits() { return kDecMaxSplits; }

// Score tiles of a fused launch over MP pages with nsplit selection
// workgroups per head (the kernel is instantiated for nsplit 8, 16, 32).
int step_score_tiles(int MP, int nsplit) {
  const int ns = nsplit <= 8 ? 8 : nsplit <= 16 ? 16 : 32;
  return (MP + step_tile_pages(ns) - 1) / step_tile_pages(ns);
}

int64_t decode_mailbox_words(int MP, int KB, int G) {
  int pw, ns, sl;
  if (!decode_shape(MP, KB, &pw, &ns, &sl)) return 0;
  return coop_mailbox_words(ns, G, MP);
}
int64_t decode_mailbox_zero_words(int MP, int KB, int G) {
  int pw, ns, sl;
  if (!decode_shape(MP, KB, &pw, &ns, &sl)) return 0;
  return coop_zero_words(ns, G);
}

template <int R, int G, int kS>
static void launch_step_rgs(const StepLaunch& a, hipStream_t st) {
  const int HL = a.H < 8 ? a.H : 8;
  const int ntiles = R > 0 ? step_score_tiles(a.MP, kS) : a.ntiles;
  const int npairs = (ntiles + 1) / 2;
  const int n_score = R > 0 ? a.H * npairs : 0;
  const int n_dec = HL * kS * ((a.H + HL - 1) / HL);
  const int dshift = (R > 0 && a.S > 1) ? 1 : 0;
  hipLaunchKernelGGL((decode_step_kernel<R, G, kS>), dim3(n_score + n_dec, 1, (unsigned)a.S + (unsigned)dshift), dim3(kDecThreads), 0, st,
                     a.escore, a.pmax, a.zpart, ntiles, a.lens, a.budgets,
                     static_cast<const uint16_t*>(a.q), static_cast<uint16_t*>(a.kpool),
                     static_cast<uint16_t*>(a.vpool), a.table, a.nb, a.H, a.MP, a.KB, a.slice, a.per_wg,
                     a.mbox, a.out, a.lse_out, a.sel, a.cnt, static_cast<const uint8_t*>(a.summ), npairs,
                     static_cast<const uint16_t*>(a.knew), static_cast<const uint16_t*>(a.vnew), a.coop,
                     a.lag, a.rule, a.hdiv > 0 ? a.hdiv : 1, dshift);
}

template <int R, int G>
static void launch_step_rg(const StepLaunch& a, hipStream_t st) {
  if (a.nsplit <= 8)
    launch_step_rgs<R, G, 8>(a, st);
  else if (a.nsplit <= 16)
    launch_step_rgs<R, G, 16>(a, st);
  else
    launch_step_rgs<R, G, 32>(a, st);
}

template <int G>
static hipError_t launch_step_g(const StepLaunch& a, hipStream_t st) {
  switch (a.r) {
    case 0: launch_step_rg<0, G>(a, st); break;
    case 4: launch_step_rg<4, G>(a, st); break;
    case 8: launch_step_rg<8, G>(a, st); break;
    case 16: launch_step_rg<16, G>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool decode_step_fuses_score(int r) { return r == 4 || r == 8 || r == 16; }

// Clears the step region (epoch, poison word, completion flags) of mailbox
// blockIdx.x.
__global__ __launch_bounds__(kStepWords) void step_reset_kernel(uint32_t* __restrict__ mbox,
                                                                int64_t stride, int64_t offset) {
  mbox[(int64_t)blockIdx.x * stride + offset + threadIdx.x] = 0u;
}

// The step regions of the `sh` (sequence, KV head) mailboxes of a fused
// decode step over MP pages and budgets up to KB; nothing for other shapes.
hipError_t launch_step_reset(uint32_t* mbox, int64_t sh, int MP, int KB, int G, hipStream_t st) {
  int pw, ns, sl;
  if (sh <= 0 || !decode_shape(MP, KB, &pw, &ns, &sl)) return hipSuccess;
  hipLaunchKernelGGL(step_reset_kernel, dim3((unsigned)sh), dim3(kStepWords), 0, st, mbox,
                     coop_mailbox_words(ns, G, MP), coop_zero_words(ns, G));
  return hipGetLastError();
}

template <int R, int G, int kS>
static int capacity_of(int dev) {
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&decode_step_kernel<R, G, kS>), kDecThreads, 0) !=
      hipSuccess)
    return -1;
  return cus * per_cu;
}

template <int R, int G>
static int capacity_rg(int dev, int si) {
  return si == 0 ? capacity_of<R, G, 8>(dev) : si == 1 ? capacity_of<R, G, 16>(dev) : capacity_of<R, G, 32>(dev);
}

template <int R>
static int capacity_r(int dev, int gi, int si) {
  return gi == 0 ? capacity_rg<R, 1>(dev, si) : gi == 1 ? capacity_rg<R, 2>(dev, si) : capacity_rg<R, 4>(dev, si);
}

// Workgroups of decode_step_kernel<r, G, nsplit> that the current device
// holds at once (compute units x workgroups resident per compute unit).
// Queried once per device and shape and kept in a small per-device table
// (the library's only process-wide state: device properties); 0 if a query
// fails.
int decode_resident_capacity(int r, int G, int nsplit) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices][4][3][3];  // 0: not queried yet, -1: failed
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  const int ri = r == 4 ? 1 : r == 8 ? 2 : r == 16 ? 3 : 0;
  const int gi = G == 1 ? 0 : G == 2 ? 1 : 2;
  const int si = nsplit <= 8 ? 0 : nsplit <= 16 ? 1 : 2;
  std::atomic<int>& slot = cache[dev][ri][gi][si];
  int c = slot.load(std::memory_order_relaxed);
  if (c == 0) {
    c = ri == 0 ? capacity_r<0>(dev, gi, si)
        : ri == 1 ? capacity_r<4>(dev, gi, si)
        : ri == 2 ? capacity_r<8>(dev, gi, si)
                  : capacity_r<16>(dev, gi, si);
    if (c == 0) c = -1;
    slot.store(c, std::memory_order_relaxed);
  }
  return c > 0 ? c : 0;
}

hipError_t launch_decode(int G, const StepLaunch& a, hipStream_t st) {
  if (a.r != 0 && (step_score_tiles(a.MP, a.nsplit) + 1) / 2 > kMaxScorePairs) return hipErrorInvalidValue;
  switch (G) {
    case 1: return launch_step_g<1>(a, st);
    case 2: return launch_step_g<2>(a, st);
    case 4: return launch_step_g<4>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace locks
