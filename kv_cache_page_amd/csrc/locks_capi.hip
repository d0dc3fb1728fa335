// C ABI of the LOCKS decode path: host-side validation, workspace carving and
// kernel dispatch. Declarations and the contract of every entry point are in
// include/locks.h.
#include "locks.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "locks_device.h"
#include "locks_step.h"

namespace locks {
hipError_t launch_score(int r, int bits, int G, const void* q, const void* summ,
                        const int32_t* table, const int32_t* lens, float* scores, int64_t nb,
                        int S, int H, int MP, int flags, float2* zpart, const void* knew,
                        const void* vnew, void* kpool, void* vpool, float* mxout, CoopZero coop,
                        hipStream_t st);
hipError_t launch_select(int G, const float* scores, const int32_t* lens, const int32_t* budgets,
                         int32_t* sel, int32_t* cnt, float* keybuf, int S, int H, int MP,
                         int max_budget, int lag, int rule, hipStream_t st);
hipError_t launch_attn(int G, const void* q, const void* kpool, const void* vpool,
                       const int32_t* table, const int32_t* lens, const int32_t* sel,
                       const int32_t* cnt, float* part, float* out, float* lse_out, int64_t nb,
                       int S, int H, int MP, int max_budget, int nsplit, int ppw, int hdiv,
                       hipStream_t st);
hipError_t launch_build(int r, const void* kpool, int64_t nb, int H, const int32_t* ids, int n,
                        const int32_t* table, const int32_t* lens, int MP, void* summ,
                        const void* knew, const void* vnew, void* vpool, int bits, hipStream_t st);
bool decode_shape(int MP, int KB, int* per_wg, int* nsplit, int* slice);
int64_t decode_mailbox_words(int MP, int KB, int G);
int64_t decode_mailbox_zero_words(int MP, int KB, int G);
hipError_t launch_decode(int G, const StepLaunch& a, hipStream_t st);
bool decode_step_fuses_score(int r);
int decode_resident_capacity(int r, int G, int nsplit);
int step_score_tiles(int MP, int nsplit);
hipError_t launch_step_reset(uint32_t* mbox, int64_t sh, int MP, int KB, int G, hipStream_t st);
hipError_t launch_append(const void* knew, const void* vnew, void* kpool, void* vpool, int64_t nb,
                         const int32_t* table, const int32_t* lens, int S, int H, int MP,
                         hipStream_t st);
}  // namespace locks

namespace {

constexpr int kMaxPagesSupported = 65536;  // select keeps one 64-bit page mask per thread
constexpr int kAttnWaves = 4;
constexpr int kAttnMaxSplits = 128;

// Pages each attention wave streams: one, unless the budget would need more
// than kAttnMaxSplits workgroups per (sequence, KV head).
int attn_pages_per_wave(int32_t KB) {
  return (KB + kAttnWaves * kAttnMaxSplits - 1) / (kAttnWaves * kAttnMaxSplits);
}

locks_status check_dims(const locks_dims* d) {
  if (!d) return LOCKS_ERR_INVALID_ARG;
  if (d->head_dim <= 0 || d->page_size <= 0 || d->rank <= 0 || d->num_kv_heads <= 0 ||
      d->group_size <= 0)
    return LOCKS_ERR_INVALID_ARG;
  if (d->head_dim != locks::kHeadDim || d->page_size != locks::kPage) return LOCKS_ERR_UNSUPPORTED;
  if (d->rank > locks::kPage) return LOCKS_ERR_UNSUPPORTED;
  if (d->group_size != 1 && d->group_size != 2 && d->group_size != 4) return LOCKS_ERR_UNSUPPORTED;
  if (d->basis_bits != 0 && d->basis_bits != 2 && d->basis_bits != 4 && d->basis_bits != 8)
    return LOCKS_ERR_INVALID_ARG;
  if (d->merge_rule < LOCKS_MERGE_SHARE || d->merge_rule > LOCKS_MERGE_PER_HEAD) return LOCKS_ERR_INVALID_ARG;
  if (d->merge_rule == LOCKS_MERGE_PER_HEAD && d->num_kv_heads > INT32_MAX / 4) return LOCKS_ERR_UNSUPPORTED;
  // the precision ablation's bases (int8, int2) are built and scored at ranks 4, 8 and 16
  if (d->basis_bits != 0 && d->basis_bits != 4 && d->rank != 4 && d->rank != 8 && d->rank != 16)
    return LOCKS_ERR_UNSUPPORTED;
  return LOCKS_OK;
}

// Basis width of the slots (0 means the default int4).
int bits_of(const locks_dims* d) { return d->basis_bits == 0 ? 4 : d->basis_bits; }

// The dims the score, selection and attention launches run on. With
// LOCKS_MERGE_PER_HEAD every query head is a group of its own: the view has
// num_kv_heads x group_size heads of group 1 under the share rule (which, for
// one query head, keys each page by that head's own share), and view head h
// reads the summaries and K/V of KV head h / group_size (hdiv, the kernels'
// head divisor). The build and append launches keep the KV heads.
struct HeadView {
  locks_dims v;
  int hdiv;
};
HeadView view_of(const locks_dims* d) {
  HeadView r{*d, 1};
  if (d->merge_rule == LOCKS_MERGE_PER_HEAD) {
    r.v.num_kv_heads = d->num_kv_heads * d->group_size;
    r.v.group_size = 1;
    r.v.merge_rule = LOCKS_MERGE_SHARE;
    r.hdiv = d->group_size;
  }
  return r;
}

// Score-kernel flags that carry the view's head divisor.
int head_div_flags(const HeadView& hv) {
  return hv.hdiv > 1 ? hv.hdiv << locks::kScoreHeadDivShift : 0;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace regions: page scores [S][H][MP][G] (or, for the fused decode
// step, e_g per page and query); per-page maxima [S][H][MP]; per-tile base-2
// (max, sum) partials [S][H][tiles][G]; selection keys of the separate select kernel
// [S][H][MP]; attention partials of the separate attention kernel
// [S][H][splits][G][kPartStride]; the selection [S][H][KB] and its counts
// [S][H] when locks_decode_step takes the separate launches without caller
// outputs; for the fused decode step, the mailboxes of its workgroups
// [S][H][...] (which also carry its split partials).
struct Workspace {
  size_t scores, pmax, zpart, keys, parts, sel, cnt, mbox, total;
  int nsplit, ntiles;
};

constexpr int kPartStride = locks::kHeadDim + 4;

Workspace carve(const locks_dims* d, int32_t S, int32_t MP, int32_t KB) {
  Workspace w{};
  const size_t sh = (size_t)S * d->num_kv_heads;
  const int per_wg = kAttnWaves * attn_pages_per_wave(KB);
  w.nsplit = (KB + per_wg - 1) / per_wg;
  w.ntiles = (MP + locks::kScorePagesPerWg - 1) / locks::kScorePagesPerWg;
  int per_f, ns_f, slice_f;
  const bool fused = locks::decode_shape(MP, KB, &per_f, &ns_f, &slice_f);
  // (a fused decode step's score outputs have rows of MP rounded up to 32 pages)
  const size_t rowp = fused ? (size_t)locks::step_row_pages(MP) : (size_t)MP;
  size_t off = 0;
  w.scores = off;
  off = align_up(off + sh * rowp * d->group_size * sizeof(float));
  w.pmax = off;
  off = align_up(off + sh * rowp * sizeof(float));
  w.zpart = off;  // (the fused decode step pads it to 64 bytes per tile, tiles rounded up to even,
                  // and may cut the table into smaller tiles)
  const int zt = fused ? std::max(w.ntiles, locks::step_score_tiles(MP, ns_f)) : w.ntiles;
  off = align_up(off + sh * (size_t)((zt + 1) / 2 * 2) * 64);
  w.keys = off;
  off = align_up(off + sh * MP * sizeof(uint32_t));
  w.parts = off;
  off = align_up(off + sh * w.nsplit * d->group_size * kPartStride * sizeof(float));
  w.sel = off;
  off = align_up(off + sh * KB * sizeof(int32_t));
  w.cnt = off;
  off = align_up(off + sh * sizeof(int32_t));
  w.mbox = off;
  off = align_up(off + (fused ? sh * (size_t)locks::decode_mailbox_words(MP, KB, d->group_size) * sizeof(uint32_t)
                              : 0));
  w.total = off;
  return w;
}

locks_status hip_status(hipError_t e) { return e == hipSuccess ? LOCKS_OK : LOCKS_ERR_HIP; }

locks_status check_batch(int32_t S, int32_t MP, int32_t KB, int64_t nb) {
  if (S < 0 || MP < 1 || KB < 2 || nb < 1) return LOCKS_ERR_INVALID_ARG;
  if (MP > kMaxPagesSupported) return LOCKS_ERR_UNSUPPORTED;
  if ((int64_t)MP * locks::kPage > INT32_MAX) return LOCKS_ERR_UNSUPPORTED;
  return LOCKS_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

const char* locks_status_string(int32_t s) {
  switch (s) {
    case LOCKS_OK: return "ok";
    case LOCKS_ERR_INVALID_ARG: return "invalid argument";
    case LOCKS_ERR_UNSUPPORTED: return "unsupported shape";
    case LOCKS_ERR_WORKSPACE: return "workspace missing or too small";
    case LOCKS_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

size_t locks_summary_slot_bytes(const locks_dims* d) {
  if (check_dims(d) != LOCKS_OK) return 0;
  return (size_t)locks::slot_layout(d->rank, bits_of(d)).payload;
}

size_t locks_summary_slot_stride(const locks_dims* d) {
  if (check_dims(d) != LOCKS_OK) return 0;
  return (size_t)locks::slot_layout(d->rank, bits_of(d)).stride;
}

size_t locks_workspace_bytes(const locks_dims* d, int32_t S, int32_t MP, int32_t KB) {
  if (check_dims(d) != LOCKS_OK || check_batch(S, MP, KB, 1) != LOCKS_OK) return 0;
  const HeadView hv = view_of(d);
  return carve(&hv.v, S, MP, KB).total;
}

locks_status locks_build(const locks_dims* d, const void* k_pool, int64_t nb,
                         const int32_t* block_ids, int32_t n, void* summaries, hipStream_t st) {
  locks_status e = check_dims(d);
  if (e != LOCKS_OK) return e;
  if (n < 0 || nb < 1) return LOCKS_ERR_INVALID_ARG;
  if (n == 0) return LOCKS_OK;
  if (!k_pool || !block_ids || !summaries) return LOCKS_ERR_INVALID_ARG;
  if (!aligned16(k_pool) || !aligned16(summaries)) return LOCKS_ERR_INVALID_ARG;
  return hip_status(locks::launch_build(d->rank, k_pool, nb, d->num_kv_heads, block_ids, n,
                                        nullptr, nullptr, 0, summaries, nullptr, nullptr, nullptr,
                                        bits_of(d), st));
}

locks_status locks_build_filled(const locks_dims* d, const void* k_pool, int64_t nb,
                                const int32_t* block_table, const int32_t* seq_lens, int32_t S,
                                int32_t MP, void* summaries, hipStream_t st) {
  locks_status e = check_dims(d);
  if (e != LOCKS_OK) return e;
  if (S < 0 || MP < 1 || nb < 1) return LOCKS_ERR_INVALID_ARG;
  if (S == 0) return LOCKS_OK;
  if (!k_pool || !block_table || !seq_lens || !summaries) return LOCKS_ERR_INVALID_ARG;
  if (!aligned16(k_pool) || !aligned16(summaries)) return LOCKS_ERR_INVALID_ARG;
  return hip_status(locks::launch_build(d->rank, k_pool, nb, d->num_kv_heads, nullptr, S,
                                        block_table, seq_lens, MP, summaries, nullptr, nullptr,
                                        nullptr, bits_of(d), st));
}

locks_status locks_append_kv(const locks_dims* d, const void* k_new, const void* v_new,
                             void* k_pool, void* v_pool, int64_t nb, const int32_t* block_table,
                             const int32_t* seq_lens, int32_t S, int32_t MP, hipStream_t st) {
  locks_status e = check_dims(d);
  if (e != LOCKS_OK) return e;
  if (S < 0 || MP < 1 || nb < 1) return LOCKS_ERR_INVALID_ARG;
  if (S == 0) return LOCKS_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !seq_lens)
    return LOCKS_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return LOCKS_ERR_INVALID_ARG;
  return hip_status(locks::launch_append(k_new, v_new, k_pool, v_pool, nb, block_table, seq_lens,
                                         S, d->num_kv_heads, MP, st));
}

locks_status locks_score_select(const locks_dims* d, const void* q, const void* summaries,
                                int64_t nb, const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* budgets, int32_t S, int32_t MP, int32_t KB,
                                int32_t* sel_pages, int32_t* sel_count, float* scores_out,
                                void* workspace, size_t ws_bytes, hipStream_t st) {
  locks_status e = check_dims(d);
  if (e != LOCKS_OK) return e;
  e = check_batch(S, MP, KB, nb);
  if (e != LOCKS_OK) return e;
  if (S == 0) return LOCKS_OK;
  if (!q || !summaries || !block_table || !seq_lens || !budgets || !sel_pages || !sel_count)
    return LOCKS_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(summaries)) return LOCKS_ERR_INVALID_ARG;
  const HeadView hv = view_of(d);
  const Workspace w = carve(&hv.v, S, MP, KB);
  if (!workspace || ws_bytes < w.total) return LOCKS_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* scores = scores_out ? scores_out : reinterpret_cast<float*>(ws + w.scores);
  const int H = hv.v.num_kv_heads, G = hv.v.group_size;
  hipError_t he = locks::launch_score(d->rank, bits_of(d), G, q, summaries, block_table, seq_lens,
                                      scores, nb, S, H, MP,
                                      (scores_out ? locks::kScoreFillNan : 0) | head_div_flags(hv),
                                      nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                      locks::CoopZero{}, st);
  if (he != hipSuccess) return LOCKS_ERR_HIP;
  he = locks::launch_select(G, scores, seq_lens, budgets, sel_pages, sel_count,
                            reinterpret_cast<float*>(ws + w.keys), S, H, MP, KB, 0, hv.v.merge_rule,
                            st);
  return hip_status(he);
}

locks_status locks_score_pages(const locks_dims* d, const void* q, const void* summaries,
                               int64_t nb, const int32_t* block_table, const int32_t* seq_lens,
                               int32_t S, int32_t MP, float* scores, hipStream_t st) {
  locks_status e = check_dims(d);
  if (e != LOCKS_OK) return e;
  e = check_batch(S, MP, 2, nb);
  if (e != LOCKS_OK) return e;
  if (S == 0) return LOCKS_OK;
  if (!q || !summaries || !block_table || !seq_lens || !scores) return LOCKS_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(summaries)) return LOCKS_ERR_INVALID_ARG;
  const HeadView hv = view_of(d);
  return hip_status(locks::launch_score(d->rank, bits_of(d), hv.v.group_size, q, summaries,
                                        block_table, seq_lens, scores, nb, S, hv.v.num_kv_heads, MP,
                                        head_div_flags(hv), nullptr, nullptr, nullptr, nullptr,
                                        nullptr, nullptr, locks::CoopZero{}, st));
}

locks_status locks_select_pages(const locks_dims* d, const float* scores, const int32_t* seq_lens,
                                const int32_t* budgets, int32_t S, int32_t MP, int32_t KB,
                                int32_t* sel_pages, int32_t* sel_count, void* workspace,
                                size_t ws_bytes, hipStream_t st) {
  locks_status e = check_dims(d);
  if (e != LOCKS_OK) return e;
  e = check_batch(S, MP, KB, 1);
  if (e != LOCKS_OK) return e;
  if (S == 0) return LOCKS_OK;
  if (!scores || !seq_lens || !budgets || !sel_pages || !sel_count) return LOCKS_ERR_INVALID_ARG;
  const HeadView hv = view_of(d);
  const Workspace w = carve(&hv.v, S, MP, KB);
  if (!workspace || ws_bytes < w.total) return LOCKS_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  return hip_status(locks::launch_select(hv.v.group_size, scores, seq_lens, budgets, sel_pages,
                                         sel_count, reinterpret_cast<float*>(ws + w.keys), S,
                                         hv.v.num_kv_heads, MP, KB, 0, hv.v.merge_rule, st));
}

locks_status locks_sparse_attn(const locks_dims* d, const void* q, const void* k_pool,
                               const void* v_pool, int64_t nb, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* sel_pages,
                               const int32_t* sel_count, int32_t S, int32_t MP, int32_t KB,
                               float* out, float* lse_out, void* workspace, size_t ws_bytes,
                               hipStream_t st) {
  locks_status e = check_dims(d);
  if (e != LOCKS_OK) return e;
  e = check_batch(S, MP, KB, nb);
  if (e != LOCKS_OK) return e;
  if (S == 0) return LOCKS_OK;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !sel_pages || !sel_count || !out)
    return LOCKS_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return LOCKS_ERR_INVALID_ARG;
  const HeadView hv = view_of(d);
  const Workspace w = carve(&hv.v, S, MP, KB);
  if (!workspace || ws_bytes < w.total) return LOCKS_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  return hip_status(locks::launch_attn(
      hv.v.group_size, q, k_pool, v_pool, block_table, seq_lens, sel_pages, sel_count,
      reinterpret_cast<float*>(ws + w.parts), out, lse_out, nb, S, hv.v.num_kv_heads, MP, KB,
      w.nsplit, attn_pages_per_wave(KB), hv.hdiv, st));
}

}  // extern "C"

namespace {

// Host checks of locks_decode_step's arguments (everything but the workspace).
locks_status decode_step_check(const locks_dims* d, const void* q, const void* k_new,
                               const void* v_new, const void* k_pool, const void* v_pool,
                               const void* summaries, int64_t nb, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* budgets, int32_t S,
                               int32_t MP, int32_t KB, const float* out, const int32_t* sel_pages,
                               const int32_t* sel_count) {
  locks_status e = check_dims(d);
  if (e != LOCKS_OK) return e;
  e = check_batch(S, MP, KB, nb);
  if (e != LOCKS_OK) return e;
  if (S == 0) return LOCKS_OK;
  if (!q || !k_new || !v_new || !k_pool || !v_pool || !summaries || !block_table || !seq_lens ||
      !budgets || !out)
    return LOCKS_ERR_INVALID_ARG;
  if ((sel_pages == nullptr) != (sel_count == nullptr)) return LOCKS_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) ||
      !aligned16(v_pool) || !aligned16(summaries))
    return LOCKS_ERR_INVALID_ARG;
  return LOCKS_OK;
}

// The launches of one decode step on a checked workspace `ws` laid out as
// `w`. reset_step: first clear the step regions of the mailboxes (epoch,
// poison word, completion flags), for a workspace that persists from call to
// call without the caller zeroing it.
locks_status decode_step_run(const locks_dims* d, const void* q, const void* k_new,
                             const void* v_new, void* k_pool, void* v_pool, void* summaries,
                             int64_t nb, const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* seq_lens_host, const int32_t* budgets, int32_t S,
                             int32_t MP, int32_t KB, float* out, float* lse_out,
                             int32_t* sel_pages, int32_t* sel_count, uint32_t flags,
                             const Workspace& w, uint8_t* ws, bool reset_step, hipStream_t st) {
  // (H, G: the view's heads for the score, selection and attention launches;
  // the build and append launches run on the Hk KV heads)
  const HeadView hv = view_of(d);
  const int H = hv.v.num_kv_heads, G = hv.v.group_size, Hk = d->num_kv_heads, bits = bits_of(d);
  const bool deferred = (flags & LOCKS_STEP_DEFER_BUILD) != 0;
  const int sflags = (deferred ? locks::kScoreDeferred : 0) | head_div_flags(hv);

  // Every decision is taken before the first launch, so that a call that
  // returns an error has enqueued nothing.
  // (i) page build: only when some sequence's new token completes a page, and
  //     never when the caller defers it (the score part then appends)
  bool completes = !deferred;
  if (completes && seq_lens_host) {
    completes = false;
    for (int32_t i = 0; i < S; ++i)
      if (seq_lens_host[i] > 0 && seq_lens_host[i] % locks::kPage == 0) completes = true;
  }
  // (ii) one launch (score + selection + attention) when the table and budget
  //      fit it and the device holds every workgroup of its exchange window at
  //      once; else the separate score, select and attention launches
  int per_wg, nsplit, slice;
  bool fused = locks::decode_shape(MP, KB, &per_wg, &nsplit, &slice);
  // (the matrix-core score part reads int4 bases only)
  const int rfused = (bits == 4 && locks::decode_step_fuses_score(d->rank)) ? d->rank : 0;
  if (fused) {
    const int HL = H < 8 ? H : 8;
    fused = locks::decode_resident_capacity(rfused, G, nsplit) >= HL * nsplit;
  }
  // (iii) where the selection goes: the caller's outputs, else the workspace
  int32_t* sel = sel_pages ? sel_pages : reinterpret_cast<int32_t*>(ws + w.sel);
  int32_t* cnt = sel_count ? sel_count : reinterpret_cast<int32_t*>(ws + w.cnt);

  if (fused && reset_step) {
    hipError_t he = locks::launch_step_reset(reinterpret_cast<uint32_t*>(ws + w.mbox),
                                             (int64_t)S * H, MP, KB, G, st);
    if (he != hipSuccess) return LOCKS_ERR_HIP;
  }
  // 1. append (+ summaries of the pages the new token completes)
  if (completes) {
    hipError_t he = locks::launch_build(d->rank, k_pool, nb, Hk, nullptr, S, block_table, seq_lens,
                                        MP, summaries, k_new, v_new, v_pool, bits, st);
    if (he != hipSuccess) return LOCKS_ERR_HIP;
  }
  // 2. scores of all full pages and Z partials (and the append when no page
  //    completes), 3. selection + attention + merge
  float* scores = reinterpret_cast<float*>(ws + w.scores);
  float2* zpart = reinterpret_cast<float2*>(ws + w.zpart);
  float* pmax = reinterpret_cast<float*>(ws + w.pmax);
  const void* kn = completes ? nullptr : k_new;
  const void* vn = completes ? nullptr : v_new;
  if (fused) {
    const locks::CoopZero coop{reinterpret_cast<uint32_t*>(ws + w.mbox),
                               locks::decode_mailbox_words(MP, KB, G),
                               (int)locks::decode_mailbox_zero_words(MP, KB, G)};
    locks::StepLaunch a{};
    a.escore = scores;
    a.pmax = pmax;
    a.zpart = zpart;
    a.ntiles = w.ntiles;
    a.lens = seq_lens;
    a.budgets = budgets;
    a.q = q;
    a.kpool = k_pool;
    a.vpool = v_pool;
    a.table = block_table;
    a.nb = nb;
    a.S = S;
    a.H = H;
    a.MP = MP;
    a.KB = KB;
    a.nsplit = nsplit;
    a.slice = slice;
    a.per_wg = per_wg;
    a.mbox = reinterpret_cast<uint32_t*>(ws + w.mbox);
    a.out = out;
    a.lse_out = lse_out;
    a.sel = sel_pages;
    a.cnt = sel_count;
    a.summ = summaries;
    a.knew = kn;
    a.vnew = vn;
    a.coop = coop;
    a.r = rfused;
    a.lag = deferred ? 1 : 0;
    a.rule = hv.v.merge_rule;
    a.hdiv = hv.hdiv;
    if (a.r == 0) {
      hipError_t he = locks::launch_score(d->rank, bits, G, q, summaries, block_table, seq_lens,
                                          scores, nb, S, H, MP, sflags, zpart, kn, vn, k_pool,
                                          v_pool, pmax, coop, st);
      if (he != hipSuccess) return LOCKS_ERR_HIP;
    }
    return hip_status(locks::launch_decode(G, a, st));
  }
  hipError_t he = locks::launch_score(d->rank, bits, G, q, summaries, block_table, seq_lens, scores,
                                      nb, S, H, MP, sflags, zpart, kn, vn, k_pool, v_pool, nullptr,
                                      locks::CoopZero{}, st);
  if (he != hipSuccess) return LOCKS_ERR_HIP;
  he = locks::launch_select(G, scores, seq_lens, budgets, sel, cnt,
                            reinterpret_cast<float*>(ws + w.keys), S, H, MP, KB, deferred ? 1 : 0,
                            hv.v.merge_rule, st);
  if (he != hipSuccess) return LOCKS_ERR_HIP;
  return hip_status(locks::launch_attn(G, q, k_pool, v_pool, block_table, seq_lens, sel, cnt,
                                       reinterpret_cast<float*>(ws + w.parts), out, lse_out, nb, S,
                                       H, MP, KB, w.nsplit, attn_pages_per_wave(KB), hv.hdiv, st));
}

// Built-in scratch of locks_decode_step_noalloc, one per device (each GPU the
// library runs on holds its own copy until the process ends). In host code
// `scratch` is a stand-in, not a device address: scratch_ptr() gives the
// address.
constexpr size_t kScratchBytes = LOCKS_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of the current device's scratch, taken once per device with
// that device current; null if a HIP call fails.
void* scratch_ptr() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

locks_status locks_decode_step_noalloc(const locks_dims* d, const void* q, const void* k_new,
                                       const void* v_new, void* k_pool, void* v_pool,
                                       void* summaries, int64_t nb, const int32_t* block_table,
                                       const int32_t* seq_lens, const int32_t* seq_lens_host,
                                       const int32_t* budgets, int32_t S, int32_t MP, int32_t KB,
                                       float* out, float* lse_out, int32_t* sel_pages,
                                       int32_t* sel_count, uint32_t flags, hipStream_t st) {
  locks_status e = decode_step_check(d, q, k_new, v_new, k_pool, v_pool, summaries, nb, block_table,
                                     seq_lens, budgets, S, MP, KB, out, sel_pages, sel_count);
  if (e != LOCKS_OK || S == 0) return e;
  if (flags & ~(uint32_t)LOCKS_STEP_DEFER_BUILD) return LOCKS_ERR_INVALID_ARG;
  const HeadView hv = view_of(d);
  const Workspace w = carve(&hv.v, S, MP, KB);
  if (w.total > kScratchBytes) return LOCKS_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return LOCKS_ERR_HIP;
  return decode_step_run(d, q, k_new, v_new, k_pool, v_pool, summaries, nb, block_table, seq_lens,
                         seq_lens_host, budgets, S, MP, KB, out, lse_out, sel_pages, sel_count,
                         flags, w, static_cast<uint8_t*>(ws), true, st);
}


locks_status locks_decode_step(const locks_dims* d, const void* q, const void* k_new,
                               const void* v_new, void* k_pool, void* v_pool, void* summaries,
                               int64_t nb, const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* seq_lens_host, const int32_t* budgets, int32_t S,
                               int32_t MP, int32_t KB, float* out, float* lse_out,
                               int32_t* sel_pages, int32_t* sel_count, uint32_t flags,
                               void* workspace, size_t ws_bytes, hipStream_t st) {
  locks_status e = decode_step_check(d, q, k_new, v_new, k_pool, v_pool, summaries, nb, block_table,
                                     seq_lens, budgets, S, MP, KB, out, sel_pages, sel_count);
  if (e != LOCKS_OK || S == 0) return e;
  if (flags & ~(uint32_t)LOCKS_STEP_DEFER_BUILD) return LOCKS_ERR_INVALID_ARG;
  const HeadView hv = view_of(d);
  const Workspace w = carve(&hv.v, S, MP, KB);
  if (!workspace || ws_bytes < w.total) return LOCKS_ERR_WORKSPACE;
  return decode_step_run(d, q, k_new, v_new, k_pool, v_pool, summaries, nb, block_table, seq_lens,
                         seq_lens_host, budgets, S, MP, KB, out, lse_out, sel_pages, sel_count,
                         flags, w, static_cast<uint8_t*>(workspace), false, st);
}

locks_status locks_host_pool_alloc(size_t bytes, void** host_ptr, void** device_ptr) {
  if (!host_ptr || !device_ptr || bytes == 0) return LOCKS_ERR_INVALID_ARG;
  *host_ptr = nullptr;
  *device_ptr = nullptr;
  void* h = nullptr;
  if (hipHostMalloc(&h, bytes, hipHostMallocMapped) != hipSuccess || !h) return LOCKS_ERR_HIP;
  void* dp = nullptr;
  if (hipHostGetDevicePointer(&dp, h, 0) != hipSuccess || !dp) {
    (void)hipHostFree(h);
    return LOCKS_ERR_HIP;
  }
  *host_ptr = h;
  *device_ptr = dp;
  return LOCKS_OK;
}

locks_status locks_host_pool_free(void* host_ptr) {
  if (!host_ptr) return LOCKS_OK;
  return hip_status(hipHostFree(host_ptr));
}

}  // extern "C"
