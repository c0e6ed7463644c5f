/*
 * kvsparse: importance-based sparse decode attention over a paged, optionally
 * low-bit KV cache, for AMD Instinct MI355X (gfx950).
 *
 * One decode step for one layer is
 *     kv_page_score  -> kv_page_topk  -> kv_sparse_decode_attn
 * (the last two also fused as kv_topk_sparse_decode_attn)
 * and, when a page is appended, kv_summary_build (and kv_pack_tier for pages
 * stored in a packed low-bit tier).  With shared-basis summaries the score is
 * kv_page_score_basis, the basis comes from kv_basis_build at prefill and the
 * page statistics from kv_summary_build_basis.
 *
 * Method sources (no formulas are published; each call states the reading it
 * implements):
 *   AMASS, decode-time sparse KV-cache attention for vLLM (amass-kv 0.1.1
 *     project page): section "AMASS" (attend only to pages that carry attention
 *     mass; a sparse paged-attention kernel reads just those pages), section
 *     "What is in the box" item 1 (quad, Gaussian-MGF page score from a tiny
 *     per-page summary), section "Quickstart" (fixed budget / per-head
 *     coverage selection), section "Benchmarking" (score, top-B and decode
 *     stages; HBM roofline of the score stage).
 *   ARGUS, virtual memory for transformers (argus_cache 0.1.7.1 project page):
 *     sections "Visual Architecture" and the tier legend (INT8, INT4 2-way,
 *     INT2 4-way, 1-bit 8-way sign-packed tiers) and "Why It Works: Storage
 *     vs. Computation" (packed pages are rebuilt in high precision on chip just
 *     before attention).
 *
 * Conventions for every call
 *   - Plain C.  All array arguments are DEVICE pointers (device memory, or
 *     pinned host memory mapped into the device address space where stated)
 *     unless the name says "host".  The caller owns every buffer; the library
 *     never allocates, frees or synchronises.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Each
 *     call only enqueues work on it and returns.
 *   - Every call validates its host-visible arguments (null pointers, shapes,
 *     supported sizes, alignment, workspace size) BEFORE any HIP call and
 *     returns a negative status without launching anything when they are
 *     wrong.  A failed launch returns KV_ERR_HIP.  No C++ exception crosses
 *     the ABI.
 *   - No global mutable state: calls are thread-safe, and identical inputs give
 *     bit-identical outputs (fixed reduction orders, no floating-point atomics).
 *   - Values read from device memory (seq_lens, block tables, selections) are
 *     not checked on the host; out-of-range values are clamped or skipped as
 *     each call states, never dereferenced out of bounds except that block
 *     table entries and page ids must name existing physical pages.
 *   - Base pointers of 16-bit pools, queries, summaries and packed code pools
 *     must be 16-byte aligned.
 *
 * Layout names: B sequences, Hq query heads, Hkv KV heads, G = Hq / Hkv query
 * heads per KV head, d = head_dim, P = page_size, R = rank, max_pages = the
 * block table's row length.  A "row" is one (sequence b, KV head g) pair,
 * row = b * Hkv + g.  Logical page p of sequence b holds tokens
 * [p*P, min((p+1)*P, seq_lens[b])); Np_b = ceil(seq_lens[b] / P), clamped to
 * max_pages.  block_table[b * max_pages + p] is its physical page.
 */
#ifndef KVSPARSE_H
#define KVSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KV_OK = 0,
  KV_ERR_INVALID_ARG = -1,   /* null pointer, bad shape, misaligned pointer */
  KV_ERR_UNSUPPORTED = -2,   /* valid but not compiled: d, P, R, G, dtype, tier */
  KV_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
  KV_ERR_HIP = -4            /* the HIP runtime reported a launch error */
};

enum { KV_F16 = 0, KV_BF16 = 1 };   /* the cache's native 16-bit dtype (also q's) */

/* Page tiers (ARGUS tier legend).  NATIVE is the cache's own 16-bit dtype;
 * FP8 is the 8-bit float E4M3 (OCP, finite variant). */
enum { KV_TIER_NATIVE = 0, KV_TIER_I8 = 1, KV_TIER_I4 = 2, KV_TIER_I2 = 3, KV_TIER_B1 = 4, KV_TIER_FP8 = 5 };
#define KV_NUM_PACKED_TIERS 5

/* page_entry word: tier in bits 29..31, slot in bits 0..28. */
#define KV_PAGE_ENTRY(tier, slot) ((((uint32_t)(tier)) << 29) | ((uint32_t)(slot) & 0x1FFFFFFFu))

/* One layer's paged cache geometry.
 * Supported: head_dim in {64, 128}; page_size in {16, 32}; rank in {1, 2, 4, 8};
 * num_q_heads a multiple of num_kv_heads with G = Hq / Hkv <= 16 for the
 * summary, score and selection calls, and G <= 8 for every call that runs the
 * attention (kv_sparse_decode_attn, kv_topk_sparse_decode_attn and the
 * whole-step calls kv_sparse_decode_step and kv_sparse_decode_step_noalloc:
 * KV_ERR_UNSUPPORTED above);
 * kv_dtype KV_F16 or KV_BF16.  softmax_scale <= 0 selects 1/sqrt(head_dim). */
typedef struct kv_layout {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t rank;
  int32_t kv_dtype;
  float softmax_scale;
} kv_layout;

/* Physical page pools read by attention.
 *   page_entry == NULL: every physical page is native and lives at
 *     k16/v16[phys] ([n_phys][Hkv][P][d] 16-bit).
 *   page_entry != NULL: page_entry[phys] = KV_PAGE_ENTRY(tier, slot); native
 *     pages live at k16/v16[slot]; a packed tier t (1..5, bits 8/4/2/1/8) keeps
 *     codes at kq[t-1]/vq[t-1][slot] ([slots][Hkv][P][d*bits/8] bytes, codes
 *     LSB-first in head-dim order) and one (scale, zero) float16 pair per
 *     32-element group at ksz[t-1]/vsz[t-1][slot] ([slots][Hkv][P][d/32][2]).
 *     A tier's K and V share the slot.  Decoding: int-b x = c*s + z rounded
 *     once to float32 (fused multiply-add); 1-bit x = z + s if c else z - s;
 *     FP8 x = e4m3(c)*s + z (exact).  Every one of the five tiers' pointers
 *     must be set when page_entry is (a tier with no pages may point to a
 *     one-slot dummy).
 *   v_hot_slot != NULL: the hot buffer, whose unit is one (physical page,
 *     KV head), u = phys * Hkv + g.  Row (b, g)'s V of physical page phys is
 *     read from v_hot[v_hot_slot[u]] ([n_slots][P][d] 16-bit, device memory)
 *     when v_hot_slot[u] >= 0, else from v16[slot]; v16 may then be pinned
 *     host memory mapped into the device address space (zero-copy reads over
 *     the host link).  v_hot_slot holds n_phys * Hkv int32.  AMASS page,
 *     section "What is in the box" item 2 (the DRAM value tier with a bounded
 *     resident hot buffer).
 *   k_hot != NULL (needs v_hot_slot): the mem-kv variant (AMASS page, table
 *     "Two variants, one algorithm": K and V both offloaded).  A hot slot holds
 *     the unit's K as well: K of unit u is read from k_hot[v_hot_slot[u]]
 *     ([n_slots][P][d] 16-bit) when that slot is >= 0, else from k16[slot],
 *     which may then be device-mapped host memory too.  Native pages only: a
 *     packed tier's codes stay where kq/vq point.
 *   kout/vout != NULL (both or neither, with page_entry): the 1-bit tier's
 *     outlier side tables for K and V, uint32 [slots][Hkv][P][d/32] as
 *     kv_pack_tier writes them; a 1-bit group then decodes its kept element
 *     from the table (ARGUS tier legend: 1-bit "with FP16 outlier
 *     preservation"). */
typedef struct kv_pages {
  const void* k16;
  const void* v16;
  const uint8_t* kq[KV_NUM_PACKED_TIERS];
  const uint8_t* vq[KV_NUM_PACKED_TIERS];
  const void* ksz[KV_NUM_PACKED_TIERS];
  const void* vsz[KV_NUM_PACKED_TIERS];
  const uint32_t* page_entry;
  const void* v_hot;
  const int32_t* v_hot_slot;
  const void* k_hot;
  const uint32_t* kout;
  const uint32_t* vout;
} kv_pages;

/* ---------------------------------------------------------------------------
 * kv_summary_build -- per-page key summary for the quad score, run when pages
 * are appended (AMASS page, "What is in the box" item 1; the summary drops the
 * per-key coordinates and keeps r' eigen-quantities of the page).
 *
 * For every entry i in [0, n), (b, p) = (entries[2i], entries[2i+1]), and every
 * KV head g, over the first n_valid[i] tokens of the page's keys in the 16-bit
 * pool k16 ([n_phys][Hkv][P][d], physical page block_table[b * max_pages + p]):
 *   mu = mean key; Xc = keys - mu; Gram = Xc Xc^T / n; (lam_j, v_j) its
 *   eigenpairs, lam descending (cyclic Jacobi in float32);
 *   w_j = Xc^T v_j / sqrt(n) for j = 1..R, set to 0 when j > n - 1 or
 *   lam_j <= 1e-6 lam_1.
 * Summaries are stored in LOGICAL page order per (sequence, KV head), so the
 * scorer streams them without a block-table lookup:
 *   summary: bfloat16 [B][Hkv][max_pages][(1+R)*d], record = [mu, w_1..w_R]
 *            (round to nearest even);
 *   log_n:   float32 [B][max_pages], log(n).
 * Eigenvector signs and rotations inside degenerate eigenspaces are arbitrary.
 * n_valid values are clamped to [0, P]; a page with 0 valid tokens gets a zero
 * record and log_n = -inf.  Entries must be distinct within a call.
 * --------------------------------------------------------------------------- */
int kv_summary_build(const kv_layout* layout, const void* k16, const int32_t* block_table,
                     int32_t max_pages, const int32_t* entries, const int32_t* n_valid, int32_t n,
                     void* summary, float* log_n, void* stream);

/* ---------------------------------------------------------------------------
 * kv_page_score -- quad page score of every logical page for every query head
 * (AMASS page, "What is in the box" item 1: quadratic, Gaussian-MGF score):
 *   s[b][g][h][p] = log_n[b][p] + tau q.mu + (tau^2/2) sum_j (q.w_j)^2
 * with q = q[b][g*G + h] ([B][Hq][d], kv_dtype), record summary[b][g][p]
 * (layout of kv_summary_build), tau = softmax_scale.
 * head_scores: float32 [B][Hkv][G][max_pages]; entries p >= Np_b are -inf.
 * lse_partial: float32 pairs (max, sum exp(s - max)) per (row, 64-page tile,
 *   head) over the tile's valid pages; its size in bytes is
 *   kv_page_score_partial_size().  It feeds kv_page_topk.
 * --------------------------------------------------------------------------- */
int kv_page_score(const kv_layout* layout, const void* q, const void* summary,
                  const float* log_n, const int32_t* seq_lens, int32_t B, int32_t max_pages,
                  float* head_scores, float* lse_partial, void* stream);

size_t kv_page_score_partial_size(const kv_layout* layout, int32_t B, int32_t max_pages);

/* ---------------------------------------------------------------------------
 * Shared-basis summaries (AMASS page, "What is in the box" item 1: the quad
 * summary keeps only r' eigenvalues per page).  The r' directions are shared by
 * every page of a row; a page keeps its mean and the variances of its keys
 * along them.  Record: 2d + 4R + 4 bytes per (page, KV head) against
 * 2(1+R)d + 4 for kv_summary_build's per-page directions.
 *
 * kv_basis_build -- the row basis, at prefill.  For every row, over the keys of
 * its tokens t < seq_lens[b] (clamped to max_pages * P) in k16 through
 * block_table:
 *   C = population covariance of those keys;
 *   basis[row][j] = unit eigenvector of C for its j-th largest eigenvalue
 *   (j < R; cyclic Jacobi in float32), its largest-magnitude entry positive
 *   (the first such entry on ties).
 * basis: float32 [B][Hkv][R][d].  Eigenvectors inside a degenerate eigenspace
 * are arbitrary.  A row with no tokens gets the first R unit vectors.
 * ws/ws_bytes: kv_basis_build_workspace_size() (no state kept between calls).
 * --------------------------------------------------------------------------- * mean (optional, may be NULL): float32 [B][Hkv][d] receives the row mean of
 * the same keys (the r8 low-rank score's centre). */
int kv_basis_build(const kv_layout* layout, const void* k16, const int32_t* block_table,
                   const int32_t* seq_lens, int32_t B, int32_t max_pages, float* basis, float* mean,
                   void* ws, size_t ws_bytes, void* stream);

size_t kv_basis_build_workspace_size(const kv_layout* layout, int32_t B, int32_t max_pages);

/* kv_summary_build_basis -- page statistics in the row basis, when pages are
 * appended.  For every entry i, (b, p) = (entries[2i], entries[2i+1]), and KV
 * head g, over the first n_valid[i] keys of the page (as kv_summary_build):
 *   mu    = mean key (float32), stored bfloat16 (round to nearest even);
 *   lam_j = mean of (u_j . (k - mu))^2 with u_j = basis[b][g][j], float32;
 *   log_n = log(n), float32 [B][max_pages].
 * mu: bfloat16 [B][Hkv][max_pages][d] and lam: float32 [B][Hkv][max_pages][R],
 * both in LOGICAL page order.  A page with 0 valid tokens gets zeros and
 * log_n = -inf.  Entries must be distinct within a call. */
int kv_summary_build_basis(const kv_layout* layout, const void* k16, const int32_t* block_table,
                           int32_t max_pages, const int32_t* entries, const int32_t* n_valid,
                           int32_t n, const float* basis, void* mu, float* lam, float* log_n,
                           void* stream);

/* kv_page_score_basis -- quad page score from shared-basis summaries:
 *   s[b][g][h][p] = log_n[b][p] + tau q.mu + (tau^2/2) sum_j lam_j (q.u_j)^2
 * with the layouts above; outputs exactly as kv_page_score (head_scores,
 * lse_partial of kv_page_score_partial_size()), so kv_page_topk follows
 * unchanged.  basis must be 16-byte aligned. */
int kv_page_score_basis(const kv_layout* layout, const void* q, const void* mu, const float* lam,
                        const float* basis, const float* log_n, const int32_t* seq_lens, int32_t B,
                        int32_t max_pages, float* head_scores, float* lse_partial, void* stream);

/* ---------------------------------------------------------------------------
 * r8 low-rank score (AMASS page, "Quickstart": the r8 low-rank fallback score;
 * "Headline results": r8 keeps per-key low-rank state).  layout->rank is the
 * basis rank r (the pages' r8: 8).  Per (sequence, KV head) row: the basis
 * u_1..u_r and mean m from kv_basis_build (with this rank); per key the
 * coordinates c_tj = bfloat16(u_j . (k_t - m)) (round to nearest even).
 *
 * kv_lowrank_coords -- coordinates of appended pages: for every entry i,
 * (b, p) = (entries[2i], entries[2i+1]), and KV head g, the first n_valid[i]
 * tokens of the page (through block_table, as kv_summary_build); later
 * tokens of the page get 0.  basis float32 [B][Hkv][r][d], mean float32
 * [B][Hkv][d]; coords bfloat16 [B][Hkv][max_pages][P][r] in LOGICAL page
 * order.  Entries must be distinct within a call. */
int kv_lowrank_coords(const kv_layout* layout, const void* k16, const int32_t* block_table, int32_t max_pages,
                      const int32_t* entries, const int32_t* n_valid, int32_t n, const float* basis,
                      const float* mean, void* coords, void* stream);

/* kv_page_score_lowrank -- for every page and query head h of the row's group
 *   s[b][g][h][p] = tau q_h.m + log sum_{t < n_p} exp(tau sum_j (q_h.u_j) c_tj)
 * over the page's n_p valid tokens (-inf for n_p = 0); outputs exactly as
 * kv_page_score, so kv_page_topk follows unchanged.  coords (layout above)
 * and q must be 16-byte aligned. */
int kv_page_score_lowrank(const kv_layout* layout, const void* q, const void* coords, const float* mean,
                          const float* basis, const int32_t* seq_lens, int32_t B, int32_t max_pages,
                          float* head_scores, float* lse_partial, void* stream);

/* ---------------------------------------------------------------------------
 * kv_page_topk -- per row, select k pages (AMASS page, "Quickstart": budget,
 * a fixed selected-page fraction; "Benchmarking": the top-B stage).
 *   L_h  = logsumexp over valid p of s[h][p] (from lse_partial)
 *   S_p  = log( (1/G) sum_h exp(s[h][p] - L_h) )   (group-mean mass fraction)
 *   k    = min(Np_b, k_fixed) if k_fixed > 0, else
 *          min(Np_b, max(1, ceil(keep_frac * Np_b))) (product in double)
 * The first n_force_first and last n_force_last valid pages get S = +inf.
 * Pages are ranked by (S descending, page index ascending), NaN as -inf; the
 * first k are written to sel[row][0..k) in ascending page order, sel entries
 * [k, k_max) are set to -1, sel_count[row] = k.
 * sel: int32 [B][Hkv][k_max]; k_max must be >= the k of a row with max_pages
 * pages.  page_S (optional, may be NULL): float32 [B][Hkv][max_pages], S_p for
 * p < Np_b.  max_pages <= 15360.  ws/ws_bytes: kv_page_topk_workspace_size().
 * --------------------------------------------------------------------------- */
int kv_page_topk(const kv_layout* layout, const float* head_scores, const float* lse_partial,
                 const int32_t* seq_lens, int32_t B, int32_t max_pages, float keep_frac,
                 int32_t k_fixed, int32_t n_force_first, int32_t n_force_last,
                 int32_t* sel, int32_t* sel_count, int32_t k_max, float* page_S,
                 void* ws, size_t ws_bytes, void* stream);

size_t kv_page_topk_workspace_size(const kv_layout* layout, int32_t B, int32_t max_pages);

/* ---------------------------------------------------------------------------
 * kv_page_topk_coverage -- kv_page_topk with k chosen per row by attention-mass
 * coverage (AMASS page, "Quickstart": the `coverage` field, the default
 * selection rule, against the fixed `budget`).  With S_p as in kv_page_topk
 * (sum_p exp(S_p) = 1 over the row's valid pages) and the same order (forced
 * pages first by index, then S descending, page ascending), k is the length of
 * the shortest prefix whose total mass exp(S) reaches `coverage`; forced pages
 * count with their own mass and are always kept, NaN pages have mass 0, and a
 * prefix that never reaches `coverage` keeps every page.  k is then clamped to
 * [max(1, forced pages), min(k_max, Np_b)].  Masses are summed in fixed point
 * with 40 fraction bits (exact integer sums, so the result does not depend on
 * thread timing).  coverage >= 0 (a value above 1 keeps every page); k_max >= 1
 * is the cap and the row length of sel.  Other arguments and outputs as for
 * kv_page_topk.
 * --------------------------------------------------------------------------- */
int kv_page_topk_coverage(const kv_layout* layout, const float* head_scores, const float* lse_partial,
                          const int32_t* seq_lens, int32_t B, int32_t max_pages, float coverage,
                          int32_t n_force_first, int32_t n_force_last, int32_t* sel, int32_t* sel_count,
                          int32_t k_max, float* page_S, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kv_sparse_decode_attn -- softmax attention of every query head over the
 * tokens of its row's selected pages only (AMASS page, "AMASS": a sparse
 * paged-attention kernel reads just the selected pages), renormalised over
 * those tokens, with packed tiers decoded in registers (ARGUS page, "Why It
 * Works"):
 *   z_i = tau q.k_i, out = sum_i softmax(z)_i v_i, lse = log sum_i exp(z_i)
 * over tokens i < seq_lens[b] of logical pages sel[row][0..sel_count[row]).
 * sel entries outside [0, Np_b) are skipped; sel_count is clamped to
 * [0, k_max].  out: float32 [B][Hq][d]; lse: float32 [B][Hq] (natural log);
 * a row with no tokens gives out = 0, lse = -inf.
 * Split-K: num_splits > 0 fixes the number of partial results per row (at
 * most 256); 0 lets the library choose.  Results agree across split counts to
 * float32 rounding.  ws/ws_bytes: kv_sparse_decode_attn_workspace_size() with
 * the same num_splits (or more).  The workspace starts with one uint32 counter
 * per row (B * Hkv of them) that must be zero when a call starts: zero it once
 * after allocating; every completed call leaves the counters at zero.  The
 * split partials follow from the first 256-byte boundary after the counters,
 * so one workspace serves calls over the same B * Hkv rows with any split
 * count up to the one it was sized for, native or packed pages alike; reused
 * for a different number of rows it must be zeroed again.  Calls that share a
 * workspace must not overlap in time.
 * --------------------------------------------------------------------------- */
int kv_sparse_decode_attn(const kv_layout* layout, const void* q, const kv_pages* pages,
                          const int32_t* block_table, const int32_t* seq_lens, int32_t B,
                          int32_t max_pages, const int32_t* sel, const int32_t* sel_count,
                          int32_t k_max, int32_t num_splits, float* out, float* lse,
                          void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace for num_splits partials per row; num_splits = 0 gives
 * enough for the automatic count of either page kind. */
size_t kv_sparse_decode_attn_workspace_size(const kv_layout* layout, int32_t B, int32_t k_max,
                                            int32_t num_splits);

/* The split count kv_sparse_decode_attn uses for num_splits = 0: tiered != 0
 * for a pool with packed tiers (pages->page_entry set), 0 for native pages. */
int32_t kv_sparse_decode_attn_num_splits(const kv_layout* layout, int32_t B, int32_t k_max,
                                         int32_t tiered);

/* ---------------------------------------------------------------------------
 * kv_topk_sparse_decode_attn -- the selector and the sparse attention of one
 * step in one launch (AMASS page, "Benchmarking": the top-B and decode stages
 * of a step, here without the selection's round trip through memory).  With
 * coverage < 0 the selection is kv_page_topk's (keep_frac, k_fixed); with
 * coverage >= 0 it is kv_page_topk_coverage's (keep_frac and k_fixed ignored,
 * k_max the cap).  Every block of a row selects the row's pages itself and
 * attends over its split's share of them; sel, sel_count and page_S
 * (optional, may be NULL) are written exactly as the selector call writes
 * them, and out and lse are bit-identical to kv_sparse_decode_attn over that
 * selection with the same num_splits (0 picks the same automatic count).
 * Arguments and their rules are the union of the two calls'; ws/ws_bytes:
 * kv_sparse_decode_attn_workspace_size() for the split count, with the same
 * zeroed counters and the same rule against overlapping calls.  Returns
 * KV_ERR_UNSUPPORTED when the row's keys and a split's share of the selection
 * do not fit one block's LDS (max_pages 2048 at d = 128 always fits); then the
 * two calls do the same work.  coverage may not be NaN or infinite.
 * --------------------------------------------------------------------------- */
int kv_topk_sparse_decode_attn(const kv_layout* layout, const void* q, const kv_pages* pages,
                               const int32_t* block_table, const int32_t* seq_lens, int32_t B,
                               int32_t max_pages, const float* head_scores, const float* lse_partial,
                               float keep_frac, int32_t k_fixed, float coverage, int32_t n_force_first,
                               int32_t n_force_last, int32_t* sel, int32_t* sel_count, int32_t k_max,
                               float* page_S, int32_t num_splits, float* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream);

/* 1 when kv_topk_sparse_decode_attn supports this shape with num_splits (> 0,
 * the count it will use) splits per row, else 0. */
int32_t kv_topk_sparse_decode_attn_supported(const kv_layout* layout, int32_t max_pages, int32_t k_max,
                                             int32_t num_splits);

/* ---------------------------------------------------------------------------
 * kv_sparse_decode_step -- a whole decode step of one layer in one call
 * (AMASS page, "Benchmarking": the score, top-B and decode stages of a step):
 * kv_page_score, then either kv_topk_sparse_decode_attn (one launch) or
 * kv_page_topk / kv_page_topk_coverage followed by kv_sparse_decode_attn,
 * whichever is the faster schedule for the shape on MI355X (the fused launch
 * for native pages, at most four query heads per KV head and rows under 4096
 * pages; kv_sparse_decode_step_fused says which a call will use).  All
 * launches go to `stream`.  Outputs are bit-identical to kv_page_score
 * followed by kv_topk_sparse_decode_attn with the same arguments (which equal
 * the separate selector and attention calls'): head_scores and lse_partial
 * (shapes and sizes as kv_page_score's), sel, sel_count, page_S (optional,
 * may be NULL), out, lse.  coverage < 0 selects by keep_frac / k_fixed,
 * coverage >= 0 by mass coverage with k_max as the cap (as
 * kv_topk_sparse_decode_attn).  Every argument follows those calls' rules; in
 * addition 1 <= max_pages <= 15360.  ws/ws_bytes:
 * kv_sparse_decode_step_workspace_size(), which is kv_sparse_decode_attn's
 * workspace for the split count, with the same zeroed counters and the same
 * rule against overlapping calls.
 * --------------------------------------------------------------------------- */
int kv_sparse_decode_step(const kv_layout* layout, const void* q, const void* summary, const float* log_n,
                          const kv_pages* pages, const int32_t* block_table, const int32_t* seq_lens,
                          int32_t B, int32_t max_pages, float keep_frac, int32_t k_fixed, float coverage,
                          int32_t n_force_first, int32_t n_force_last, float* head_scores, float* lse_partial,
                          int32_t* sel, int32_t* sel_count, int32_t k_max, float* page_S, int32_t num_splits,
                          float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kv_sparse_decode_step_noalloc -- kv_sparse_decode_step without a workspace,
 * for callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments (minus ws / ws_bytes), same launches, and
 * outputs bit-identical to kv_sparse_decode_step with the same num_splits.
 * The attention's split counters and partials live in a 32 MiB array of
 * device memory inside the library (one copy per GPU, kept until the process
 * ends): 256 KiB of counters for up to 65535 rows, then room for
 * B * Hkv * splits * G * (head_dim + 2) float32 partials, at most
 * 33292288 bytes; a larger call returns KV_ERR_WORKSPACE without launching.
 * The first call on a device looks the array up and clears its counters with
 * a kernel on `stream`; every completed call leaves them at zero.  The call
 * allocates nothing.  All calls on one GPU share the array, so calls that
 * overlap in time on one GPU (on different streams or from different host
 * threads) race and must be serialised by the caller.
 * --------------------------------------------------------------------------- */
int kv_sparse_decode_step_noalloc(const kv_layout* layout, const void* q, const void* summary, const float* log_n,
                                  const kv_pages* pages, const int32_t* block_table, const int32_t* seq_lens,
                                  int32_t B, int32_t max_pages, float keep_frac, int32_t k_fixed, float coverage,
                                  int32_t n_force_first, int32_t n_force_last, float* head_scores,
                                  float* lse_partial, int32_t* sel, int32_t* sel_count, int32_t k_max,
                                  float* page_S, int32_t num_splits, float* out, float* lse, void* stream);

/* Bytes of workspace for kv_sparse_decode_step: kv_sparse_decode_attn's for
 * the same arguments; 0 for invalid arguments. */
size_t kv_sparse_decode_step_workspace_size(const kv_layout* layout, int32_t B, int32_t k_max,
                                            int32_t num_splits);

/* 1 when kv_sparse_decode_step supports this layout and shape, else 0. */
int32_t kv_sparse_decode_step_supported(const kv_layout* layout, int32_t B, int32_t max_pages, int32_t k_max,
                                        int32_t num_splits);

/* 1 when kv_sparse_decode_step uses the fused selector + attention launch
 * for these arguments, 0 when it uses the separate selector and attention
 * launches (or the shape is not supported). */
int32_t kv_sparse_decode_step_fused(const kv_layout* layout, const kv_pages* pages, int32_t B, int32_t max_pages,
                                    int32_t k_max, int32_t num_splits);

/* ---------------------------------------------------------------------------
 * kv_hot_admit -- hot-buffer admission for a host-resident V pool (AMASS page,
 * "What is in the box" item 2 and the AMASS-mem variant: V in pinned,
 * device-mapped host memory, a bounded resident hot buffer plus a staging
 * pool).  The buffer's unit is one (physical page, KV head), u = phys * Hkv
 * + g: the P x d values one row's attention reads of a page.  Run once per
 * step after its selection and before its attention, on the attention's
 * stream: the attention then reads every admitted unit from device memory.
 * With U = the units of the step's selection (entries i < sel_count of row
 * (b, g), clamped to [0, k_max], of pages 0 <= p < Np_b, through block_table,
 * as block_table[b][p] * Hkv + g; duplicates removed):
 *   1. a unit of U already hot (v_hot_slot[u] = s >= 0) stamps its slot:
 *      slot_stamp[s] = step;
 *   2. the units of U that are not hot, ascending by unit id, are admitted
 *      into the slots least recently used before this step -- the smallest
 *      (slot_stamp, slot index) among slots with slot_stamp < step -- one unit
 *      per slot, paired in ascending slot order; with fewer such slots than
 *      units the lowest unit ids are admitted;
 *   3. an admitted slot s drops its old unit (v_hot_slot[old] = -1), takes u
 *      (slot_page[s] = u, v_hot_slot[u] = s, slot_stamp[s] = step) and u's V,
 *      [P][d] 16-bit at v16 + u * P * d (the pool [n_phys][Hkv][P][d],
 *      device-mapped host memory or device memory), is copied to
 *      v_hot + s * P * d ([n_slots][P][d]); with k16 and k_hot given (the
 *      mem-kv variant, both or neither) u's K is copied from k16 into k_hot the
 *      same way.
 * State, device memory owned by the caller: v_hot_slot int32 [n_units] with
 * n_units = n_phys * Hkv, slot_page int32 [n_slots], slot_stamp uint32
 * [n_slots] (0 = never used).  Initialise them consistently (all -1 / 0 for an
 * empty buffer).  step >= 1 and increasing across calls.  n_units <= 2^24 and
 * a multiple of Hkv, n_slots <= 2^22 (else KV_ERR_UNSUPPORTED).
 * ws/ws_bytes: kv_hot_admit_workspace_size(n_slots, n_units) bytes of device
 * memory, 4-byte aligned; no contents carry over between calls.  After the
 * call ws[0] (int32) is the number of units copied and ws[1 + 2i], ws[2 + 2i]
 * the i-th (unit, slot) pair, ascending by slot.
 * --------------------------------------------------------------------------- */
int kv_hot_admit(const kv_layout* layout, const void* v16, void* v_hot, const void* k16, void* k_hot,
                 int32_t* v_hot_slot, int32_t n_units, int32_t* slot_page, uint32_t* slot_stamp, int32_t n_slots,
                 const int32_t* block_table, const int32_t* seq_lens, int32_t B, int32_t max_pages,
                 const int32_t* sel, const int32_t* sel_count, int32_t k_max, uint32_t step,
                 void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of kv_hot_admit (0 for sizes it does not support). */
size_t kv_hot_admit_workspace_size(int32_t n_slots, int32_t n_units);

/* ---------------------------------------------------------------------------
 * kv_dequant_tier -- the attention kernel's in-register tier decoding as a
 * standalone call (for tests and tier migration): K and V of physical pages
 * pages[0..n) decoded through `pages_desc` (page_entry, tiers, hot buffer) into
 * out, float32 [n][2][Hkv][P][d] (index 0 = K, 1 = V).  ARGUS page, "Why It
 * Works: Storage vs. Computation".
 * --------------------------------------------------------------------------- */
int kv_dequant_tier(const kv_layout* layout, const kv_pages* pages_desc, const int32_t* pages,
                    int32_t n, float* out, void* stream);

/* ---------------------------------------------------------------------------
 * kv_pack_tier -- encode 16-bit pages into packed tier `tier` (1..5; ARGUS tier
 * legend and "Visual Architecture": INT8, INT4 2-way, INT2 4-way, 1-bit 8-way
 * sign-packed, FP8).
 * Per token vector, per group of 32 consecutive head-dim elements, x the
 * float32 value of the 16-bit input, every step an IEEE float32 operation
 * rounded to nearest even, no fused multiply-add:
 *   int-b: s = f16(f32(max - min) / (2^b - 1)), z = f16(min),
 *          c = 0 if s == 0 else clamp(rint(f32(x - z) / s), 0, 2^b - 1)
 *   1-bit: z = f16(T(x) / 32), s = f16(T(|x - z|) / 32), c = (x >= z),
 *          T the pairwise tree sum (level by level, pairs (2i, 2i+1))
 *   FP8:   s = f16(f32(max |x|) / 448), z = 0,
 *          c = 0 if s == 0 else E4M3(f32(x / s)), one code per byte, where
 *          E4M3(y) is the nearest finite E4M3 value (ties to the even code,
 *          |y| >= 448 saturating to 448, sign bit copied from y)
 *   f16() rounds to nearest even and saturates at +-65504.
 * Source page src_pages[i] of src16 ([*][Hkv][P][d]) goes to slot dst_slots[i]
 * of codes ([slots][Hkv][P][d*bits/8]) and scale_zero ([slots][Hkv][P][d/32][2]
 * float16, scale first).  NULL src_pages / dst_slots mean i.
 * outliers (1-bit tier only, may be NULL): uint32 [slots][Hkv][P][d/32]; per
 * group, the element e* farthest from z (fp32 |x - z|, lowest index on ties)
 * is kept: word = e* | (float16 bits of x_e*, round to nearest even,
 * saturating) << 16.  Must be NULL for the other tiers.
 * --------------------------------------------------------------------------- */
int kv_pack_tier(const kv_layout* layout, const void* src16, const int32_t* src_pages, int32_t n,
                 int32_t tier, uint8_t* codes, void* scale_zero, uint32_t* outliers, const int32_t* dst_slots,
                 void* stream);

/* ---------------------------------------------------------------------------
 * kv_tier_plan -- which pages move one step down the compression cascade
 * (ARGUS page, "The One-Minute Explanation" and "Visual Architecture": 16-bit
 * for critical and recent pages, then FP8 -> int8 -> int4 -> int2 -> 1-bit as
 * pages cool; per-tier page budgets from its configuration).  Levels: 0
 * native, 1 FP8, 2 int8, 3 int4, 4 int2, 5 1-bit.  For every sequence b, over
 * its valid pages p < Np_b:
 *   importance i_p = max over KV heads g of page_S[b][g][p] (the group-mean
 *   page mass kv_page_topk writes; NaN counts as -inf);
 *   rank: the first n_force_first and last n_force_last pages first (by
 *   index), then i descending, page index ascending;
 *   desired level d_p = the smallest l <= 4 with rank < caps[0] + .. + caps[l],
 *   else 5 (caps: host array of 5 page budgets, >= 0);
 *   a page with d_p above its current level (from page_entry through
 *   block_table) moves down one level; no page moves up.
 * page_S float32 [B][Hkv][max_pages]; moves int32 [B][max_pages][2] receives
 * per sequence, in page order, (physical page, new tier id); move_count int32
 * [B].  max_pages <= 15360.
 * --------------------------------------------------------------------------- */
int kv_tier_plan(const kv_layout* layout, const float* page_S, const int32_t* seq_lens, int32_t B,
                 int32_t max_pages, const int32_t* block_table, const uint32_t* page_entry, const int32_t* caps,
                 int32_t n_force_first, int32_t n_force_last, int32_t* moves, int32_t* move_count, void* stream);

/* ---------------------------------------------------------------------------
 * kv_tier_demote -- carry out a tier plan: every listed page's K and V (all KV
 * heads and tokens) is decoded from its current tier (the attention kernel's
 * decoding) and encoded into the new tier with kv_pack_tier's encoder, applied
 * to the decoded float32 values; the codes and (scale, zero) pairs go to slot
 * `phys` of the new tier's pools, which must therefore hold at least n_phys
 * slots, and page_entry[phys] becomes KV_PAGE_ENTRY(new tier, phys).  With
 * kout/vout set, pages entering the 1-bit tier get their outlier words too.
 * pages_desc: the pools (written: the tier pools named by the moves) with
 * pages_desc->page_entry == page_entry.  moves / move_count as kv_tier_plan
 * leaves them (device memory).  Pages of a move list are distinct.
 * --------------------------------------------------------------------------- */
int kv_tier_demote(const kv_layout* layout, const kv_pages* pages_desc, uint32_t* page_entry, int32_t B,
                   int32_t max_pages, const int32_t* moves, const int32_t* move_count, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* kv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVSPARSE_H */
