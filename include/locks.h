/*
 * locks.h -- C ABI of the LOCKS decode hot path on AMD Instinct MI355X (gfx950).
 *
 * LOCKS keeps the whole paged KV cache resident and, per decode step and KV
 * head, reads only (a) a small spectral summary of every full page and (b) the
 * full K/V of the pages it selects from those summaries.
 *
 * Pages this interface follows (cited by title and section):
 *   [N] "LOCKS 阅读笔记" (zhongzhuzhou.org reading notes, 2026-07-29) on
 *       "LOCKS: Page-Local Compact Key Summaries for Efficient Long-Context
 *       Decoding", arXiv 2607.24555.
 *   [S] "Resumo Técnico: LOCKS" (gist.science technical summary).
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless stated otherwise. Every call is
 *     asynchronous and ordered on `stream`; none allocates, frees or
 *     synchronises the host.
 *   - The caller owns every buffer (pools, tables, outputs, workspace). The
 *     library's only process-wide state is a per-device table of device
 *     properties it queries once (see locks_decode_step). Calls on different
 *     streams with different output and workspace buffers may run
 *     concurrently, with one caveat for locks_decode_step: its single-launch
 *     form needs the selection workgroups of a (sequence, KV head) running at
 *     the same time (they exchange data); a concurrent kernel that holds the
 *     compute units long enough (for instance another locks_decode_step on
 *     another stream) can make their bounded waits time out, and the step then
 *     writes NaN and poisons its workspace (see there) instead of hanging.
 *   - Errors: arguments known on the host are validated before anything is
 *     enqueued; a call that returns an error has enqueued nothing. A failed
 *     kernel launch returns LOCKS_ERR_HIP.
 *   - Device-resident data (block ids, lengths, budgets, selections) is
 *     trusted in meaning but never dereferenced out of range: a block id
 *     outside [0, num_blocks) is treated as a missing page (not scored, not
 *     attended, its summary not written), lengths are clamped to
 *     [0, max_pages * page_size] and budgets to [2, max_budget].
 *   - Layouts (row-major, innermost last):
 *       K / V pool     bf16 [num_blocks][num_kv_heads][page_size][head_dim]
 *       summaries      uint8 [num_blocks][num_kv_heads][slot_stride]
 *       q              bf16 [num_seqs][num_kv_heads * group_size][head_dim];
 *                      query head h belongs to KV head h / group_size
 *       block_table    int32 [num_seqs][max_pages], logical page -> block id
 *       seq_lens       int32 [num_seqs], tokens cached including the current
 *                      one; the sequence has P = ceil(len / page_size) pages,
 *                      of which F = floor(len / page_size) are full
 *   - Supported shapes: head_dim 128, page_size 16, rank 1..16,
 *     group_size 1, 2 or 4, num_kv_heads >= 1.
 */
#ifndef LOCKS_H
#define LOCKS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version of the summary slot byte layout described below. */
#define LOCKS_SLOT_LAYOUT_VERSION 2  /* 2: stride rounded up to 128 bytes */

typedef struct {
    int32_t head_dim;     /* d: 128 */
    int32_t page_size;    /* B: tokens per page, 16 */
    int32_t rank;         /* r: kept basis vectors per page, 1..16 */
    int32_t num_kv_heads; /* H_kv >= 1 */
    int32_t group_size;   /* G: query heads per KV head (GQA), 1, 2 or 4 */
    int32_t basis_bits;   /* stored basis precision: 0 or 4 (int4, the
                             default), 8 or 2 (the ablation of [N] §6; ranks
                             4, 8 and 16 only) */
    int32_t merge_rule;   /* LOCKS_MERGE_*: how the group's query heads pool
                             their page scores into one key (0: eq. 5) */
} locks_dims;

/* GQA merge rules ([N] §4.2 and the ablation of [N] §6). With m_g(j) =
 * exp(s_jg - Z_g) the share of page j for query head g:
 *   SHARE  key_j = log mean_g m_g(j)                (eq. 5, the default)
 *   MAX    key_j = log max_g m_g(j)                 (group-max)
 *   MASS   key_j = log (sum_g exp(s_jg) / sum_g Z_g) (group-mass: the pooled
 *          unnormalised masses)
 * The selection rule (sink, recent, top-(k-2) keys) is the same for all.
 *   PER_HEAD  no pooling: every query head selects its own sink, recent and
 *          top-(k-2) pages by its own share m_g(j) and attends only those
 *          (the per-head oracle that [N] §4.2 and §6 compare the shared rule
 *          against, G selections per group). Every entry point except
 *          locks_build, locks_build_filled and locks_append_kv then treats
 *          each query head as a KV head of its own: num_kv_heads x group_size
 *          heads of one query head each, head h reading the summaries and
 *          K/V of KV head h / group_size. Arrays with a KV-head axis take
 *          num_kv_heads x group_size rows: sel_pages
 *          [S][H_kv G][max_budget], sel_count [S][H_kv G], page scores
 *          [S][H_kv G][max_pages] (query head h_kv G + g in row h_kv G + g);
 *          the workspace sizes follow (locks_workspace_bytes with the same
 *          dims). q, out and lse_out keep their layouts. Each page summary is
 *          read once per query head, so the score stage reads G times the
 *          bytes of the shared rules. */
#define LOCKS_MERGE_SHARE 0
#define LOCKS_MERGE_MAX 1
#define LOCKS_MERGE_MASS 2
#define LOCKS_MERGE_PER_HEAD 3

typedef enum {
    LOCKS_OK = 0,
    LOCKS_ERR_INVALID_ARG = -1, /* null pointer, negative count, bad shape   */
    LOCKS_ERR_UNSUPPORTED = -2, /* valid but not implemented shape           */
    LOCKS_ERR_WORKSPACE = -3,   /* workspace missing or smaller than needed  */
    LOCKS_ERR_HIP = -4          /* a HIP launch or device query failed       */
} locks_status;

/* Text for a status code; any int32 is accepted ("unknown status" for values
 * that are not a locks_status). */
const char* locks_status_string(int32_t status);

/*
 * Summary slot of one (block, KV head) page -- [N] §4.1 (storage paragraph)
 * and Algorithm 1: an int4 basis with one scale per column, int8 coefficients
 * with one scale per token row, an int8 centroid with one scale; about a
 * tenth of the page's K+V bytes at r = 8, B = 16.
 *
 *   offset 0          Vq   r columns x (d/2) bytes, two's-complement int4.
 *                          Each little-endian 32-bit word of a column covers
 *                          dims 8t..8t+7; its four bytes hold the dim pairs
 *                          (0,1), (4,5), (2,3), (6,7), low nibble first.
 *                          With basis_bits 8: r columns x d bytes, int8 in
 *                          dim order; with 2: r columns x d/4 bytes, four
 *                          dims per byte in dim order, two's-complement
 *                          two-bit fields from the lowest bits (codes -1, 0,
 *                          1). The same quantiser with qmax 127, 7 or 1.
 *   offset r*d*b/8    Cq   page_size x r int8, row-major (row i = c_i)
 *   next              muq  d int8 (centroid codes in dim order)
 *   next              scales, fp16 little-endian: r basis-column scales,
 *                          page_size coefficient-row scales, 1 centroid scale
 *   then zero padding up to slot_stride (a multiple of 128 bytes, so slots
 *   start on cache lines and share none).
 * Decoded values are code * scale. r = 8: 818 payload bytes, stride 896
 * (int8 basis: 1330 and 1408; int2: 562 and 640).
 * The scoring calls take basis-column scales below 8 (the matrix-core path
 * carries V^T q in fp16 parts); locks_build writes at most about 1/7, since
 * its basis columns have unit norm.
 */
size_t locks_summary_slot_bytes(const locks_dims* dims);  /* payload; 0 if dims invalid */
size_t locks_summary_slot_stride(const locks_dims* dims); /* bytes between slots; 0 if invalid */

/*
 * Bytes of device workspace that locks_score_select, locks_select_pages,
 * locks_sparse_attn and locks_decode_step need for up to num_seqs sequences of up to max_pages pages
 * and budgets of up to max_budget pages. One workspace may serve all of them
 * when the calls are ordered on one stream; its contents need no
 * initialisation. Between calls it carries only a per-(sequence, KV head)
 * epoch that locks_decode_step advances (it tells one call's completion
 * flags from another's; no result depends on its value) and the poison word
 * described under locks_decode_step. Returns 0 for invalid arguments.
 */
size_t locks_workspace_bytes(const locks_dims* dims, int32_t num_seqs, int32_t max_pages,
                             int32_t max_budget);

/*
 * locks_build -- [N] §4.1 eq. 2-3 and §4.3 Algorithm 1, for n full pages.
 * For each i < n and each KV head, reads the page_size x head_dim keys of
 * block block_ids[i] (device int32) and writes that (block, head) slot:
 * centroid mu = mean of the keys, deviations D = keys - mu, Gram D D^T,
 * eigendecomposition (Jacobi, descending eigenvalues), basis
 * V = D^T U_r Sigma_r^{-1} and coefficients C = U_r Sigma_r, then int4/int8
 * quantisation. Component k is kept only if lambda_k > 1e-6 trace(D D^T) and
 * lambda_k > 1e-12 sum_i |k_i|^2; otherwise its basis column and
 * coefficients are zero. Each kept basis vector is signed so that its entry of
 * largest magnitude (lowest dim on ties) is positive. Quantiser: scale =
 * fp16(fp32(absmax) / qmax) (qmax 7 for int4, 127 for int8; an overflowing
 * scale saturates at 65504), code = clamp(rint(x / scale), -qmax, qmax) in
 * fp32, all-zero when absmax is 0. Block ids outside [0, num_blocks) are
 * skipped. Errors: INVALID_ARG (null pointers, n < 0, num_blocks < 1, bad
 * dims), UNSUPPORTED (shape), HIP.
 */
locks_status locks_build(const locks_dims* dims, const void* k_pool, int64_t num_blocks,
                         const int32_t* block_ids, int32_t n, void* summaries,
                         hipStream_t stream);

/*
 * locks_build_filled -- the incremental build trigger of [N] §2 and
 * [S] §2: for every sequence whose length is a positive multiple of
 * page_size (its newest page has just filled), builds that page
 * (block_table[s][len/page_size - 1]) for all KV heads exactly as
 * locks_build does. Sequences whose last page is partial are left alone.
 * The decision is taken on the device, so the call can sit in a captured
 * decode step. Errors as for locks_build.
 */
locks_status locks_build_filled(const locks_dims* dims, const void* k_pool, int64_t num_blocks,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int32_t num_seqs, int32_t max_pages, void* summaries,
                                hipStream_t stream);

/*
 * locks_append_kv -- writes one new token per sequence into the paged cache
 * (the decode-step append that precedes scoring, [N] §2 figure 1):
 * k_new / v_new bf16 [num_seqs][num_kv_heads][head_dim] go to position
 * seq_lens[s] - 1 (seq_lens already counts the new token) of block
 * block_table[s][(seq_lens[s]-1) / page_size]. Sequences with length < 1 or
 * an out-of-range block are skipped. Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
locks_status locks_append_kv(const locks_dims* dims, const void* k_new, const void* v_new,
                             void* k_pool, void* v_pool, int64_t num_blocks,
                             const int32_t* block_table, const int32_t* seq_lens,
                             int32_t num_seqs, int32_t max_pages, hipStream_t stream);

/*
 * locks_score_select -- [N] §4.2 eq. 4-5 and §4.4 Algorithm 2 up to the
 * selection; reads summaries only, never K or V.
 *   score: for every full page j < F and query head g of the group,
 *     s_hat_jg = LSE_i ((q_g . mu_j + (V_j^T q_g) . c_i) / sqrt(d))
 *     from the decoded summary (natural-log units).
 *   shares: Z_g = LSE_j s_hat_jg over all F full pages (sink and a full last
 *     page included); key_j = log((1/G) sum_g exp(s_hat_jg - Z_g)).
 *   select: S = {0, P-1} plus the k-2 pages of largest key among pages
 *     1..P-2 (equal keys: lower page first); k = clamp(budgets[s], 2,
 *     max_budget); every page when k >= P; {0} when P == 1; nothing when
 *     P == 0. One S per (sequence, KV head) serves its whole GQA group.
 * Outputs: sel_pages int32 [num_seqs][num_kv_heads][max_budget], the logical
 *   page ids of S in ascending order, padded with -1; sel_count int32
 *   [num_seqs][num_kv_heads] = |S|. scores_out (optional, may be NULL):
 *   float [num_seqs][num_kv_heads][max_pages][group_size] with s_hat for
 *   j < F and NaN elsewhere.
 * Errors: INVALID_ARG (null required pointer, num_seqs < 0, max_pages < 1,
 *   max_budget < 2, num_blocks < 1, bad dims), UNSUPPORTED (shape),
 *   WORKSPACE (workspace NULL or smaller than locks_workspace_bytes), HIP.
 */
locks_status locks_score_select(const locks_dims* dims, const void* q, const void* summaries,
                                int64_t num_blocks, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* budgets,
                                int32_t num_seqs, int32_t max_pages, int32_t max_budget,
                                int32_t* sel_pages, int32_t* sel_count, float* scores_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * locks_score_pages -- the scoring half of locks_score_select ([N] §4.2
 * eq. 4): writes s_hat for every full page j < F of every (sequence, KV head)
 * into scores float [num_seqs][num_kv_heads][max_pages][group_size]
 * (entries j >= F are left untouched; an out-of-range block gives -inf).
 * Needs no workspace. Errors as for locks_score_select.
 */
locks_status locks_score_pages(const locks_dims* dims, const void* q, const void* summaries,
                               int64_t num_blocks, const int32_t* block_table,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t max_pages,
                               float* scores, hipStream_t stream);

/*
 * locks_select_pages -- the selection half of locks_score_select ([N] §4.2
 * eq. 5 and §4.4 Algorithm 2): from scores laid out as locks_score_pages
 * writes them, computes the group-averaged shares and writes sel_pages /
 * sel_count exactly as locks_score_select does. Uses the workspace.
 * Errors as for locks_score_select.
 */
locks_status locks_select_pages(const locks_dims* dims, const float* scores,
                                const int32_t* seq_lens, const int32_t* budgets,
                                int32_t num_seqs, int32_t max_pages, int32_t max_budget,
                                int32_t* sel_pages, int32_t* sel_count, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * locks_sparse_attn -- [N] §4.4 Algorithm 2 last steps and §3.1 eq. 1: for
 * every query head g of KV head h, softmax attention over the tokens of the
 * selected pages only, renormalised over them:
 *   o_g = sum_{t in S} exp(l_t) v_t / sum_{t in S} exp(l_t), l_t = q_g.k_t/sqrt(d),
 * where the last page P-1 contributes its len - (P-1)*page_size valid tokens.
 * The pages are split across workgroups (split-K flash decoding) and a second
 * kernel merges the partial (max, sum, accumulator) triples by log-sum-exp in
 * split order, so results do not depend on scheduling.
 * Outputs: out float [num_seqs][num_kv_heads * group_size][head_dim];
 *   lse_out (optional) float [num_seqs][num_kv_heads * group_size] =
 *   log sum_{t in S} exp(l_t); an empty selection gives out = 0, lse = -inf.
 * Selected ids outside [0, P) or whose block is out of range are ignored.
 * Errors as for locks_score_select.
 */
locks_status locks_sparse_attn(const locks_dims* dims, const void* q, const void* k_pool,
                               const void* v_pool, int64_t num_blocks,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* sel_pages, const int32_t* sel_count,
                               int32_t num_seqs, int32_t max_pages, int32_t max_budget,
                               float* out, float* lse_out, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Flags of locks_decode_step / locks_decode_step_noalloc. */
#define LOCKS_STEP_DEFER_BUILD 1u  /* leave the page the new token completes to locks_build_filled */

/*
 * locks_decode_step -- one whole decode step of one layer, [N] §2 figure 1
 * and §4.4 Algorithm 2 end to end, with the same results as the sequence
 *   locks_append_kv -> locks_build_filled -> locks_score_select ->
 *   locks_sparse_attn
 * (up to floating-point summation order; the probabilities enter the
 * value product in bf16), in one launch, two when a page completes:
 *   1. only when a sequence's new token completes a page: append every new
 *      token and build the summaries of the completed pages (their last key
 *      is taken from k_new);
 *   2. score every full page, keeping per tile of pages (128, or 32 when the
 *      table is short) the (max, sum exp) of the scores for Z_g (and append
 *      the new tokens when step 1 did not run), then select S and attend: the attention workgroups of a
 *      (sequence, KV head) wait for its score workgroups, share the selection
 *      (each selects within its own slice of the pages and they exchange
 *      histograms and candidates through the workspace), attend their own
 *      selected pages, and each merges the splits' shares of 1/nsplit of
 *      the output elements in split order. Ranks other than 4, 8 and 16 score in a launch of
 *      their own before the selection and attention launch.
 * Arguments are those of the calls above; seq_lens counts the new token.
 * seq_lens_host (HOST pointer, optional): a host copy of seq_lens, used only
 *   to skip step 1 when no length is a positive multiple of page_size; with
 *   NULL step 1 always runs. It must equal seq_lens.
 * sel_pages / sel_count (optional, both or neither): the selection, as
 *   locks_score_select writes it.
 * flags: 0, or LOCKS_STEP_DEFER_BUILD for the build outside the decode
 *   critical path ([N] §2): the step then builds nothing; it scores only the
 *   pages that were full before its token, floor((len - 1) / page_size), so a
 *   page its token completes is, for this step, the unsummarised recent page
 *   (selected as always, left out of Z_g). The caller summarises those pages
 *   with locks_build_filled (same block table and lengths) on any stream,
 *   ordered after this call and before the next decode step of the layer.
 *   Other bits: INVALID_ARG.
 * Path: tables of more than 16384 pages, budgets above 2048 pages, and
 *   devices that cannot hold min(H, 8) x nsplit of the kernel's 512-thread
 *   workgroups at once (queried once per device) take separate score, select
 *   and attention launches (the selection then goes through the workspace
 *   when sel_pages is NULL). The choice, and every argument check, is made
 *   before anything is enqueued.
 * Timeouts: the single-launch form waits with a bound (it cannot hang). A
 *   wait that times out (only possible when another kernel holds the compute
 *   units, see the conventions above) makes that step's out and lse NaN and
 *   poisons the workspace: every later locks_decode_step on it writes NaN
 *   until the caller zeroes the whole workspace (e.g. hipMemsetAsync), after
 *   the stream has finished the poisoned call.
 * Errors as for locks_score_select, plus INVALID_ARG for a null k_new, v_new,
 *   k_pool, v_pool or out, or only one of sel_pages / sel_count.
 */
locks_status locks_decode_step(const locks_dims* dims, const void* q, const void* k_new,
                               const void* v_new, void* k_pool, void* v_pool, void* summaries,
                               int64_t num_blocks, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* seq_lens_host,
                               const int32_t* budgets, int32_t num_seqs, int32_t max_pages,
                               int32_t max_budget, float* out, float* lse_out,
                               int32_t* sel_pages, int32_t* sel_count, uint32_t flags,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * locks_decode_step_noalloc -- locks_decode_step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same step, arguments and results
 * (same kernels), without a workspace argument. Its workspace is a built-in
 * scratch array of LOCKS_NOALLOC_SCRATCH_BYTES per device, which the library
 * holds until the process ends; the call itself allocates and frees nothing.
 * A shape whose locks_workspace_bytes exceeds LOCKS_NOALLOC_SCRATCH_BYTES is
 * rejected with LOCKS_ERR_WORKSPACE before anything is enqueued (16 MiB
 * covers, for instance, one sequence of a 65536-page table with budgets up to
 * 2048 pages, or four 8192-page sequences with budgets up to 256, at 8 KV
 * heads and G = 4). Every call on a device shares that device's scratch and
 * each call first clears the parts that must start cleared (one small fill
 * launch), so a timed-out step poisons only itself; calls that overlap on one
 * device (different streams, or different host threads) race and must not
 * be made. Errors as for locks_decode_step; HIP also when the scratch address
 * cannot be obtained.
 */
#define LOCKS_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
locks_status locks_decode_step_noalloc(const locks_dims* dims, const void* q, const void* k_new,
                                       const void* v_new, void* k_pool, void* v_pool,
                                       void* summaries, int64_t num_blocks,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       const int32_t* seq_lens_host, const int32_t* budgets,
                                       int32_t num_seqs, int32_t max_pages, int32_t max_budget,
                                       float* out, float* lse_out, int32_t* sel_pages,
                                       int32_t* sel_count, uint32_t flags, hipStream_t stream);

/*
 * Offload path ([N] §8: the selection never reads keys or values, so the
 * summaries alone can stay on the accelerator while the whole KV cache lives
 * in host memory). K and V pools may be pinned, device-mapped host memory:
 * pass the device pointer that locks_host_pool_alloc returns as k_pool /
 * v_pool to any entry point above, with the same layout. Scoring and
 * selection then read only the summaries in device memory; the attention
 * reads only the selected pages across the host link, the step's append
 * writes one token per (sequence, KV head) there, and a page build reads
 * the completed page's keys once. Results are those of device-memory pools.
 *
 * locks_host_pool_alloc -- bytes of pinned host memory mapped into the
 *   current device's address space (page-aligned). host_ptr: the host
 *   address (fill and read the pool there, ordered with the device work by
 *   stream synchronisation); device_ptr: the address kernels use. The caller
 *   owns the memory and frees it with locks_host_pool_free(host_ptr) once no
 *   enqueued work uses it. Errors: INVALID_ARG (null output, bytes == 0),
 *   HIP (allocation or mapping failed; both outputs are then NULL).
 * locks_host_pool_free -- frees what locks_host_pool_alloc returned (NULL:
 *   no-op). Errors: HIP.
 */
locks_status locks_host_pool_alloc(size_t bytes, void** host_ptr, void** device_ptr);
locks_status locks_host_pool_free(void* host_ptr);

#ifdef __cplusplus
}
#endif

#endif /* LOCKS_H */
