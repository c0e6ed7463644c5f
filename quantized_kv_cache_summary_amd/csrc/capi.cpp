// C ABI of libkvsparse: argument validation (before any HIP call), workspace
// sizing, launch-shape choice and status codes.  Declared in include/kvsparse.h.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/kvsparse.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_layout(const kv_layout* L) {
  if (!L) return KV_ERR_INVALID_ARG;
  if (L->num_q_heads <= 0 || L->num_kv_heads <= 0) return KV_ERR_INVALID_ARG;
  if (L->num_q_heads % L->num_kv_heads != 0) return KV_ERR_INVALID_ARG;
  if (L->head_dim <= 0 || L->page_size <= 0 || L->rank <= 0) return KV_ERR_INVALID_ARG;
  if (L->kv_dtype != KV_F16 && L->kv_dtype != KV_BF16) return KV_ERR_UNSUPPORTED;
  if (L->head_dim != 64 && L->head_dim != 128) return KV_ERR_UNSUPPORTED;
  if (L->page_size != 16 && L->page_size != 32) return KV_ERR_UNSUPPORTED;
  if (L->rank != 1 && L->rank != 2 && L->rank != 4 && L->rank != 8) return KV_ERR_UNSUPPORTED;
  if (L->num_q_heads / L->num_kv_heads > 16) return KV_ERR_UNSUPPORTED;
  if (!(L->softmax_scale == L->softmax_scale)) return KV_ERR_INVALID_ARG;
  return KV_OK;
}

// Attention (and every call that runs it) takes at most eight query heads per
// KV head; scoring and selection take up to sixteen.
constexpr int kMaxAttnGroup = 8;
int check_attn_group(const kv_layout* L) {
  return L->num_q_heads / L->num_kv_heads > kMaxAttnGroup ? KV_ERR_UNSUPPORTED : KV_OK;
}

float scale_of(const kv_layout* L) {
  return L->softmax_scale > 0.f ? L->softmax_scale : 1.0f / std::sqrt((float)L->head_dim);
}

int from_hip(hipError_t e) { return e == hipSuccess ? KV_OK : KV_ERR_HIP; }

int topk_bound(int max_pages, float keep, int k_fixed) {
  if (max_pages <= 0) return 0;
  if (k_fixed > 0) return k_fixed < max_pages ? k_fixed : max_pages;
  int k = (int)std::ceil((double)keep * (double)max_pages);
  k = k < 1 ? 1 : k;
  return k > max_pages ? max_pages : k;
}

// Splits per row.  A native-page block streams K/V at the gather rate with one
// wave per SIMD, and every further split only lengthens the latency-bound head
// (page list) and tail (merge) of the kernel, so native pages get about one
// 4-wave block per CU (256 blocks).  Packed tiers spend VALU time decoding, so
// they get as many blocks as stay resident (three 4-wave blocks per CU).  At
// least two pages per wave either way.
int auto_splits(int rows, int k_max, bool tiered) {
  if (rows <= 0) return 1;
  const int waves = 4;
  const int target = tiered ? 512 : 256;
  int s = (target + rows - 1) / rows;
  int cap = k_max / (2 * waves);
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s > kvs::kMaxSplits) s = kvs::kMaxSplits;
  return s < 1 ? 1 : s;
}

// Workspace for num_splits = 0 covers whichever automatic count the pages need.
int auto_splits_any(int rows, int k_max) {
  const int a = auto_splits(rows, k_max, false), b = auto_splits(rows, k_max, true);
  return a > b ? a : b;
}

int check_pages(const kv_layout* L, const kv_pages* pg) {
  if (!pg) return KV_ERR_INVALID_ARG;
  if (!pg->k16 || !pg->v16) return KV_ERR_INVALID_ARG;
  if (!aligned16(pg->k16) || !aligned16(pg->v16)) return KV_ERR_INVALID_ARG;
  if (pg->page_entry) {
    for (int t = 0; t < KV_NUM_PACKED_TIERS; ++t) {
      if (!pg->kq[t] || !pg->vq[t] || !pg->ksz[t] || !pg->vsz[t]) return KV_ERR_INVALID_ARG;
      if (!aligned16(pg->kq[t]) || !aligned16(pg->vq[t])) return KV_ERR_INVALID_ARG;
      if ((reinterpret_cast<uintptr_t>(pg->ksz[t]) & 3u) || (reinterpret_cast<uintptr_t>(pg->vsz[t]) & 3u))
        return KV_ERR_INVALID_ARG;
    }
  }
  if (pg->v_hot_slot && (!pg->v_hot || !aligned16(pg->v_hot))) return KV_ERR_INVALID_ARG;
  if (pg->k_hot && (!pg->v_hot_slot || !aligned16(pg->k_hot))) return KV_ERR_INVALID_ARG;
  if (!pg->kout != !pg->vout) return KV_ERR_INVALID_ARG;
  if (pg->kout && !pg->page_entry) return KV_ERR_INVALID_ARG;
  (void)L;
  return KV_OK;
}

}  // namespace

extern "C" {

const char* kv_status_string(int status) {
  switch (status) {
    case KV_OK: return "ok";
    case KV_ERR_INVALID_ARG: return "invalid argument";
    case KV_ERR_UNSUPPORTED: return "unsupported configuration";
    case KV_ERR_WORKSPACE: return "workspace missing or too small";
    case KV_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int kv_summary_build(const kv_layout* L, const void* k16, const int32_t* block_table, int32_t max_pages,
                     const int32_t* entries, const int32_t* n_valid, int32_t n, void* summary,
                     float* log_n, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (n < 0 || max_pages < 0) return KV_ERR_INVALID_ARG;
  if (n == 0) return KV_OK;
  if (max_pages == 0) return KV_ERR_INVALID_ARG;
  if (!k16 || !block_table || !entries || !n_valid || !summary || !log_n) return KV_ERR_INVALID_ARG;
  if (!aligned16(k16) || !aligned16(summary)) return KV_ERR_INVALID_ARG;
  if ((int64_t)n * L->num_kv_heads > 0x7FFFFFFF) return KV_ERR_UNSUPPORTED;
  return from_hip(kvs::launch_summary_build(*L, k16, block_table, max_pages, entries, n_valid, n,
                                            summary, log_n, (hipStream_t)stream));
}

size_t kv_page_score_partial_size(const kv_layout* L, int32_t B, int32_t max_pages) {
  if (check_layout(L) || B <= 0 || max_pages <= 0) return 0;
  const size_t G = (size_t)(L->num_q_heads / L->num_kv_heads);
  return (size_t)B * L->num_kv_heads * kvs::score_tiles(max_pages) * G * 2 * sizeof(float);
}

int kv_page_score(const kv_layout* L, const void* q, const void* summary, const float* log_n,
                  const int32_t* seq_lens, int32_t B, int32_t max_pages, float* head_scores,
                  float* lse_partial, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (B < 0 || max_pages < 0) return KV_ERR_INVALID_ARG;
  if (B == 0 || max_pages == 0) return KV_OK;
  if (!q || !summary || !log_n || !seq_lens || !head_scores || !lse_partial) return KV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(summary)) return KV_ERR_INVALID_ARG;
  if ((int64_t)B * L->num_kv_heads > 65535) return KV_ERR_UNSUPPORTED;
  return from_hip(kvs::launch_page_score(*L, q, summary, log_n, seq_lens, B, max_pages, scale_of(L),
                                         head_scores, lse_partial, (hipStream_t)stream));
}

size_t kv_basis_build_workspace_size(const kv_layout* L, int32_t B, int32_t max_pages) {
  if (check_layout(L) || B <= 0 || max_pages <= 0) return 0;
  return kvs::basis_workspace_bytes(B * L->num_kv_heads, max_pages, L->head_dim);
}

int kv_basis_build(const kv_layout* L, const void* k16, const int32_t* block_table, const int32_t* seq_lens,
                   int32_t B, int32_t max_pages, float* basis, float* mean, void* ws, size_t ws_bytes,
                   void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (B < 0 || max_pages < 0) return KV_ERR_INVALID_ARG;
  if (B == 0) return KV_OK;
  if (max_pages == 0 || !k16 || !block_table || !seq_lens || !basis) return KV_ERR_INVALID_ARG;
  if (!aligned16(k16)) return KV_ERR_INVALID_ARG;
  if ((int64_t)B * L->num_kv_heads > 65535) return KV_ERR_UNSUPPORTED;
  if ((int64_t)max_pages * L->page_size > 0x3FFFFFFF) return KV_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < kv_basis_build_workspace_size(L, B, max_pages)) return KV_ERR_WORKSPACE;
  return from_hip(kvs::launch_basis_build(*L, k16, block_table, seq_lens, B, max_pages, basis, mean, (float*)ws,
                                          (hipStream_t)stream));
}

int kv_summary_build_basis(const kv_layout* L, const void* k16, const int32_t* block_table, int32_t max_pages,
                           const int32_t* entries, const int32_t* n_valid, int32_t n, const float* basis,
                           void* mu, float* lam, float* log_n, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (n < 0 || max_pages < 0) return KV_ERR_INVALID_ARG;
  if (n == 0) return KV_OK;
  if (max_pages == 0) return KV_ERR_INVALID_ARG;
  if (!k16 || !block_table || !entries || !n_valid || !basis || !mu || !lam || !log_n) return KV_ERR_INVALID_ARG;
  if (!aligned16(k16)) return KV_ERR_INVALID_ARG;
  if ((int64_t)n * L->num_kv_heads > 0x7FFFFFFF) return KV_ERR_UNSUPPORTED;
  return from_hip(kvs::launch_summary_build_basis(*L, k16, block_table, max_pages, entries, n_valid, n, basis,
                                                  mu, lam, log_n, (hipStream_t)stream));
}

int kv_page_score_basis(const kv_layout* L, const void* q, const void* mu, const float* lam, const float* basis,
                        const float* log_n, const int32_t* seq_lens, int32_t B, int32_t max_pages,
                        float* head_scores, float* lse_partial, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (B < 0 || max_pages < 0) return KV_ERR_INVALID_ARG;
  if (B == 0 || max_pages == 0) return KV_OK;
  if (!q || !mu || !lam || !basis || !log_n || !seq_lens || !head_scores || !lse_partial)
    return KV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(mu) || !aligned16(basis)) return KV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(lam) & 3u) || (reinterpret_cast<uintptr_t>(log_n) & 3u))
    return KV_ERR_INVALID_ARG;
  if ((int64_t)B * L->num_kv_heads > 65535) return KV_ERR_UNSUPPORTED;
  return from_hip(kvs::launch_page_score_basis(*L, q, mu, lam, basis, log_n, seq_lens, B, max_pages,
                                               scale_of(L), head_scores, lse_partial, (hipStream_t)stream));
}

int kv_lowrank_coords(const kv_layout* L, const void* k16, const int32_t* block_table, int32_t max_pages,
                      const int32_t* entries, const int32_t* n_valid, int32_t n, const float* basis,
                      const float* mean, void* coords, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (n < 0 || max_pages < 0) return KV_ERR_INVALID_ARG;
  if (n == 0) return KV_OK;
  if (max_pages == 0 || !k16 || !block_table || !entries || !n_valid || !basis || !mean || !coords)
    return KV_ERR_INVALID_ARG;
  if (!aligned16(k16)) return KV_ERR_INVALID_ARG;
  if (n > 0x7FFFFFFF / 2) return KV_ERR_UNSUPPORTED;
  return from_hip(kvs::launch_lowrank_coords(*L, k16, block_table, max_pages, entries, n_valid, n, basis, mean,
                                             coords, (hipStream_t)stream));
}

int kv_page_score_lowrank(const kv_layout* L, const void* q, const void* coords, const float* mean,
                          const float* basis, const int32_t* seq_lens, int32_t B, int32_t max_pages,
                          float* head_scores, float* lse_partial, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (B < 0 || max_pages < 0) return KV_ERR_INVALID_ARG;
  if (B == 0 || max_pages == 0) return KV_OK;
  if (!q || !coords || !mean || !basis || !seq_lens || !head_scores || !lse_partial) return KV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(coords)) return KV_ERR_INVALID_ARG;
  if ((int64_t)B * L->num_kv_heads > 65535) return KV_ERR_UNSUPPORTED;
  return from_hip(kvs::launch_page_score_lowrank(*L, q, coords, mean, basis, seq_lens, B, max_pages, scale_of(L),
                                                 head_scores, lse_partial, (hipStream_t)stream));
}

size_t kv_page_topk_workspace_size(const kv_layout* L, int32_t B, int32_t max_pages) {
  (void)L; (void)B; (void)max_pages;
  return 0;
}

int kv_page_topk(const kv_layout* L, const float* head_scores, const float* lse_partial,
                 const int32_t* seq_lens, int32_t B, int32_t max_pages, float keep_frac,
                 int32_t k_fixed, int32_t n_force_first, int32_t n_force_last, int32_t* sel,
                 int32_t* sel_count, int32_t k_max, float* page_S, void* ws, size_t ws_bytes,
                 void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  (void)ws; (void)ws_bytes;
  if (B < 0 || max_pages < 0 || k_max < 0 || k_fixed < 0 || n_force_first < 0 || n_force_last < 0)
    return KV_ERR_INVALID_ARG;
  if (!(keep_frac >= 0.f) || !std::isfinite(keep_frac)) return KV_ERR_INVALID_ARG;
  if (B == 0) return KV_OK;
  if (max_pages > kvs::kMaxTopkPages) return KV_ERR_UNSUPPORTED;
  if (!seq_lens || !sel_count) return KV_ERR_INVALID_ARG;
  if (max_pages > 0 && (!head_scores || !lse_partial)) return KV_ERR_INVALID_ARG;
  if (k_max > 0 && !sel) return KV_ERR_INVALID_ARG;
  if (k_max < topk_bound(max_pages, keep_frac, k_fixed)) return KV_ERR_INVALID_ARG;
  if ((int64_t)B * L->num_kv_heads > 0x7FFFFFFF) return KV_ERR_UNSUPPORTED;
  return from_hip(kvs::launch_page_topk(*L, head_scores, lse_partial, seq_lens, B, max_pages,
                                        keep_frac, k_fixed, -1.f, n_force_first, n_force_last, sel,
                                        sel_count, k_max, page_S, (hipStream_t)stream));
}

int32_t kv_sparse_decode_attn_num_splits(const kv_layout* L, int32_t B, int32_t k_max, int32_t tiered) {
  if (check_layout(L) || B <= 0) return 1;
  return auto_splits(B * L->num_kv_heads, k_max, tiered != 0);
}

int kv_page_topk_coverage(const kv_layout* L, const float* head_scores, const float* lse_partial,
                          const int32_t* seq_lens, int32_t B, int32_t max_pages, float coverage,
                          int32_t n_force_first, int32_t n_force_last, int32_t* sel, int32_t* sel_count,
                          int32_t k_max, float* page_S, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  (void)ws; (void)ws_bytes;
  if (B < 0 || max_pages < 0 || k_max < 1 || n_force_first < 0 || n_force_last < 0) return KV_ERR_INVALID_ARG;
  if (!(coverage >= 0.f) || !std::isfinite(coverage)) return KV_ERR_INVALID_ARG;
  if (B == 0) return KV_OK;
  if (max_pages > kvs::kMaxTopkPages) return KV_ERR_UNSUPPORTED;
  if (!seq_lens || !sel_count || !sel) return KV_ERR_INVALID_ARG;
  if (max_pages > 0 && (!head_scores || !lse_partial)) return KV_ERR_INVALID_ARG;
  if ((int64_t)B * L->num_kv_heads > 0x7FFFFFFF) return KV_ERR_UNSUPPORTED;
  return from_hip(kvs::launch_page_topk(*L, head_scores, lse_partial, seq_lens, B, max_pages, 0.f, 0,
                                        coverage, n_force_first, n_force_last, sel, sel_count, k_max,
                                        page_S, (hipStream_t)stream));
}

size_t kv_sparse_decode_attn_workspace_size(const kv_layout* L, int32_t B, int32_t k_max,
                                            int32_t num_splits) {
  if (check_layout(L) || B <= 0 || num_splits < 0) return 0;
  const int rows = B * L->num_kv_heads;
  const int s = num_splits > 0 ? num_splits : auto_splits_any(rows, k_max);
  return kvs::attn_workspace_bytes(rows, s, L->num_q_heads / L->num_kv_heads, L->head_dim);
}

int kv_sparse_decode_attn(const kv_layout* L, const void* q, const kv_pages* pg,
                          const int32_t* block_table, const int32_t* seq_lens, int32_t B,
                          int32_t max_pages, const int32_t* sel, const int32_t* sel_count,
                          int32_t k_max, int32_t num_splits, float* out, float* lse, void* ws,
                          size_t ws_bytes, void* stream) {
  int rc = check_layout(L);
  if (!rc) rc = check_attn_group(L);
  if (rc) return rc;
  if (B < 0 || max_pages < 0 || k_max < 0 || num_splits < 0) return KV_ERR_INVALID_ARG;
  if (num_splits > kvs::kMaxSplits) return KV_ERR_UNSUPPORTED;
  if (B == 0) return KV_OK;
  if (!q || !block_table || !seq_lens || !sel_count || !out || !lse) return KV_ERR_INVALID_ARG;
  if (k_max > 0 && !sel) return KV_ERR_INVALID_ARG;
  if (!aligned16(q)) return KV_ERR_INVALID_ARG;
  rc = check_pages(L, pg);
  if (rc) return rc;
  const int rows = B * L->num_kv_heads;
  if ((int64_t)rows > 65535) return KV_ERR_UNSUPPORTED;
  const int s = num_splits > 0 ? num_splits : auto_splits(rows, k_max, pg->page_entry != nullptr);
  const size_t need = kv_sparse_decode_attn_workspace_size(L, B, k_max, s);
  if (!ws || ws_bytes < need) return KV_ERR_WORKSPACE;
  return from_hip(kvs::launch_sparse_attn(*L, q, *pg, block_table, seq_lens, B, max_pages, sel,
                                          sel_count, k_max, s, scale_of(L), out, lse,
                                          kvs::attn_scratch_in(ws, rows), (hipStream_t)stream));
}

int32_t kv_topk_sparse_decode_attn_supported(const kv_layout* L, int32_t max_pages, int32_t k_max,
                                             int32_t num_splits) {
  if (check_layout(L) || check_attn_group(L) || max_pages < 0 || k_max < 0 || num_splits <= 0 || num_splits > kvs::kMaxSplits) return 0;
  if (max_pages > kvs::kMaxTopkPages) return 0;
  return kvs::topk_attn_dyn_lds_bytes(*L, max_pages, k_max, num_splits) <= kvs::kTopkAttnMaxLds ? 1 : 0;
}

int kv_topk_sparse_decode_attn(const kv_layout* L, const void* q, const kv_pages* pg,
                               const int32_t* block_table, const int32_t* seq_lens, int32_t B,
                               int32_t max_pages, const float* head_scores, const float* lse_partial,
                               float keep_frac, int32_t k_fixed, float coverage, int32_t n_force_first,
                               int32_t n_force_last, int32_t* sel, int32_t* sel_count, int32_t k_max,
                               float* page_S, int32_t num_splits, float* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream) {
  int rc = check_layout(L);
  if (!rc) rc = check_attn_group(L);
  if (rc) return rc;
  if (B < 0 || max_pages < 0 || k_max < 0 || k_fixed < 0 || n_force_first < 0 || n_force_last < 0 ||
      num_splits < 0)
    return KV_ERR_INVALID_ARG;
  if (coverage != coverage || std::isinf(coverage)) return KV_ERR_INVALID_ARG;
  const bool cov = coverage >= 0.f;
  if (!cov && (!(keep_frac >= 0.f) || !std::isfinite(keep_frac))) return KV_ERR_INVALID_ARG;
  if (cov && k_max < 1) return KV_ERR_INVALID_ARG;
  if (num_splits > kvs::kMaxSplits) return KV_ERR_UNSUPPORTED;
  if (B == 0) return KV_OK;
  if (max_pages > kvs::kMaxTopkPages) return KV_ERR_UNSUPPORTED;
  if (!q || !block_table || !seq_lens || !sel_count || !out || !lse) return KV_ERR_INVALID_ARG;
  if (k_max > 0 && !sel) return KV_ERR_INVALID_ARG;
  if (max_pages > 0 && (!head_scores || !lse_partial)) return KV_ERR_INVALID_ARG;
  if (!cov && k_max < topk_bound(max_pages, keep_frac, k_fixed)) return KV_ERR_INVALID_ARG;
  if (!aligned16(q)) return KV_ERR_INVALID_ARG;
  rc = check_pages(L, pg);
  if (rc) return rc;
  const int rows = B * L->num_kv_heads;
  if ((int64_t)rows > 65535) return KV_ERR_UNSUPPORTED;
  const int s = num_splits > 0 ? num_splits : auto_splits(rows, k_max, pg->page_entry != nullptr);
  if (kvs::topk_attn_dyn_lds_bytes(*L, max_pages, k_max, s) > kvs::kTopkAttnMaxLds) return KV_ERR_UNSUPPORTED;
  const size_t need = kv_sparse_decode_attn_workspace_size(L, B, k_max, s);
  if (!ws || ws_bytes < need) return KV_ERR_WORKSPACE;
  return from_hip(kvs::launch_topk_sparse_attn(*L, q, *pg, block_table, seq_lens, B, max_pages, head_scores,
                                               lse_partial, cov ? 0.f : keep_frac, cov ? 0 : k_fixed,
                                               cov ? coverage : -1.f, n_force_first, n_force_last, sel,
                                               sel_count, k_max, page_S, s, scale_of(L), out, lse,
                                               kvs::attn_scratch_in(ws, rows), (hipStream_t)stream));
}

size_t kv_sparse_decode_step_workspace_size(const kv_layout* L, int32_t B, int32_t k_max, int32_t num_splits) {
  return kv_sparse_decode_attn_workspace_size(L, B, k_max, num_splits);
}

int32_t kv_sparse_decode_step_supported(const kv_layout* L, int32_t B, int32_t max_pages, int32_t k_max,
                                        int32_t num_splits) {
  if (check_layout(L) || check_attn_group(L) || B < 0 || max_pages < 1 || k_max < 0 || num_splits < 0 ||
      num_splits > kvs::kMaxSplits)
    return 0;
  return max_pages <= kvs::kMaxTopkPages ? 1 : 0;
}

int32_t kv_sparse_decode_step_fused(const kv_layout* L, const kv_pages* pages, int32_t B, int32_t max_pages,
                                    int32_t k_max, int32_t num_splits) {
  if (!kv_sparse_decode_step_supported(L, B, max_pages, k_max, num_splits) || !pages) return 0;
  // measured: the fused selector + attention wins for native pages, up to four
  // query heads per KV head (eight-wave blocks) and rows under 4096 pages;
  // packed tiers want two attention blocks per CU, and longer rows or wider
  // groups select too slowly inside one block
  if (pages->page_entry || L->num_q_heads / L->num_kv_heads > 4 || max_pages >= kvs::kTopkWideFrom) return 0;
  const int s = num_splits > 0 ? num_splits : auto_splits(B * L->num_kv_heads, k_max, false);
  return kvs::topk_attn_dyn_lds_bytes(*L, max_pages, k_max, s) <= kvs::kTopkAttnMaxLds ? 1 : 0;
}

}  // extern "C"

namespace {

// Validation of kv_sparse_decode_step's arguments other than its workspace;
// sets the split count the call uses.
int check_step(const kv_layout* L, const void* q, const void* summary, const float* log_n, const kv_pages* pg,
               const int32_t* block_table, const int32_t* seq_lens, int32_t B, int32_t max_pages, float keep_frac,
               int32_t k_fixed, float coverage, int32_t n_force_first, int32_t n_force_last,
               const float* head_scores, const float* lse_partial, const int32_t* sel, const int32_t* sel_count,
               int32_t k_max, int32_t num_splits, const float* out, const float* lse, int* splits) {
  int rc = check_layout(L);
  if (!rc) rc = check_attn_group(L);
  if (rc) return rc;
  if (B < 0 || max_pages < 0 || k_max < 0 || k_fixed < 0 || n_force_first < 0 || n_force_last < 0 ||
      num_splits < 0)
    return KV_ERR_INVALID_ARG;
  if (coverage != coverage || std::isinf(coverage)) return KV_ERR_INVALID_ARG;
  const bool cov = coverage >= 0.f;
  if (!cov && (!(keep_frac >= 0.f) || !std::isfinite(keep_frac))) return KV_ERR_INVALID_ARG;
  if (cov && k_max < 1) return KV_ERR_INVALID_ARG;
  if (num_splits > kvs::kMaxSplits) return KV_ERR_UNSUPPORTED;
  *splits = 1;
  if (B == 0) return KV_OK;
  if (max_pages == 0) return KV_ERR_INVALID_ARG;
  if (max_pages > kvs::kMaxTopkPages) return KV_ERR_UNSUPPORTED;
  if (!q || !summary || !log_n || !block_table || !seq_lens || !head_scores || !lse_partial || !sel_count ||
      !out || !lse)
    return KV_ERR_INVALID_ARG;
  if (k_max > 0 && !sel) return KV_ERR_INVALID_ARG;
  if (!cov && k_max < topk_bound(max_pages, keep_frac, k_fixed)) return KV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(summary)) return KV_ERR_INVALID_ARG;
  rc = check_pages(L, pg);
  if (rc) return rc;
  const int rows = B * L->num_kv_heads;
  if ((int64_t)rows > 65535) return KV_ERR_UNSUPPORTED;
  *splits = num_splits > 0 ? num_splits : auto_splits(rows, k_max, pg->page_entry != nullptr);
  return KV_OK;
}

// The whole step's launches (arguments already validated).
int enqueue_step(const kv_layout* L, const void* q, const void* summary, const float* log_n, const kv_pages* pg,
                 const int32_t* block_table, const int32_t* seq_lens, int32_t B, int32_t max_pages, float keep_frac,
                 int32_t k_fixed, float coverage, int32_t n_force_first, int32_t n_force_last, float* head_scores,
                 float* lse_partial, int32_t* sel, int32_t* sel_count, int32_t k_max, float* page_S, int s,
                 float* out, float* lse, kvs::AttnScratch sc, hipStream_t st);

}  // namespace

extern "C" {

int kv_sparse_decode_step(const kv_layout* L, const void* q, const void* summary, const float* log_n,
                          const kv_pages* pg, const int32_t* block_table, const int32_t* seq_lens, int32_t B,
                          int32_t max_pages, float keep_frac, int32_t k_fixed, float coverage,
                          int32_t n_force_first, int32_t n_force_last, float* head_scores, float* lse_partial,
                          int32_t* sel, int32_t* sel_count, int32_t k_max, float* page_S, int32_t num_splits,
                          float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  int s = 1;
  const int rc = check_step(L, q, summary, log_n, pg, block_table, seq_lens, B, max_pages, keep_frac, k_fixed,
                            coverage, n_force_first, n_force_last, head_scores, lse_partial, sel, sel_count, k_max,
                            num_splits, out, lse, &s);
  if (rc || B == 0) return rc;
  if (!ws || ws_bytes < kv_sparse_decode_attn_workspace_size(L, B, k_max, s)) return KV_ERR_WORKSPACE;
  return enqueue_step(L, q, summary, log_n, pg, block_table, seq_lens, B, max_pages, keep_frac, k_fixed, coverage,
                      n_force_first, n_force_last, head_scores, lse_partial, sel, sel_count, k_max, page_S, s, out,
                      lse, kvs::attn_scratch_in(ws, B * L->num_kv_heads), (hipStream_t)stream);
}

}  // extern "C"

namespace {

int enqueue_step(const kv_layout* L, const void* q, const void* summary, const float* log_n, const kv_pages* pg,
                 const int32_t* block_table, const int32_t* seq_lens, int32_t B, int32_t max_pages, float keep_frac,
                 int32_t k_fixed, float coverage, int32_t n_force_first, int32_t n_force_last, float* head_scores,
                 float* lse_partial, int32_t* sel, int32_t* sel_count, int32_t k_max, float* page_S, int s,
                 float* out, float* lse, kvs::AttnScratch sc, hipStream_t st) {
  const bool cov = coverage >= 0.f;
  const float tau = scale_of(L);
  const float kf = cov ? 0.f : keep_frac, cv = cov ? coverage : -1.f;
  const int kx = cov ? 0 : k_fixed;
  int rc = from_hip(kvs::launch_page_score(*L, q, summary, log_n, seq_lens, B, max_pages, tau, head_scores,
                                           lse_partial, st));
  if (rc) return rc;
  if (kv_sparse_decode_step_fused(L, pg, B, max_pages, k_max, s))
    return from_hip(kvs::launch_topk_sparse_attn(*L, q, *pg, block_table, seq_lens, B, max_pages, head_scores,
                                                 lse_partial, kf, kx, cv, n_force_first, n_force_last, sel,
                                                 sel_count, k_max, page_S, s, tau, out, lse, sc, st));
  rc = from_hip(kvs::launch_page_topk(*L, head_scores, lse_partial, seq_lens, B, max_pages, kf, kx, cv,
                                      n_force_first, n_force_last, sel, sel_count, k_max, page_S, st));
  if (rc) return rc;
  return from_hip(kvs::launch_sparse_attn(*L, q, *pg, block_table, seq_lens, B, max_pages, sel, sel_count, k_max,
                                          s, tau, out, lse, sc, st));
}

}  // namespace

extern "C" {

}  // extern "C"

// ---------------------------------------------------------------- whole step without a workspace
//
// For callers that cannot allocate: the attention's cross-block state lives
// in this file-scope device array instead of a caller workspace.  Counters
// for up to 65535 rows sit at a fixed offset in front (so calls over
// different numbers of rows never overwrite each other's counters), the split
// partials after them.  Every GPU the library runs on holds its own copy until
// the process ends; its device address is looked up once per device.

namespace {
constexpr size_t kNoAllocBytes = (size_t)32 << 20;
constexpr size_t kNoAllocCounterBytes = (size_t)65536 * sizeof(unsigned);
constexpr size_t kNoAllocPartialBytes = kNoAllocBytes - kNoAllocCounterBytes;
constexpr int kNoAllocMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices];

__global__ void clear_words_kernel(unsigned* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The current device's copy of `scratch` (looked up on its first use, with its
// counters then cleared on `st` by a fill kernel).  KV_ERR_HIP on failure.
int scratch_on_current_device(hipStream_t st, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return KV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KV_ERR_HIP;
    const int n = (int)(kNoAllocCounterBytes / sizeof(unsigned));
    hipLaunchKernelGGL(clear_words_kernel, dim3(64), dim3(256), 0, st, reinterpret_cast<unsigned*>(ptr), n);
    if (hipGetLastError() != hipSuccess) return KV_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = reinterpret_cast<char*>(g_scratch_ptr[dev]);
  return KV_OK;
}

}  // namespace

extern "C" {

int kv_sparse_decode_step_noalloc(const kv_layout* L, const void* q, const void* summary, const float* log_n,
                                  const kv_pages* pg, const int32_t* block_table, const int32_t* seq_lens,
                                  int32_t B, int32_t max_pages, float keep_frac, int32_t k_fixed, float coverage,
                                  int32_t n_force_first, int32_t n_force_last, float* head_scores,
                                  float* lse_partial, int32_t* sel, int32_t* sel_count, int32_t k_max,
                                  float* page_S, int32_t num_splits, float* out, float* lse, void* stream) {
  int s = 1;
  int rc = check_step(L, q, summary, log_n, pg, block_table, seq_lens, B, max_pages, keep_frac, k_fixed, coverage,
                      n_force_first, n_force_last, head_scores, lse_partial, sel, sel_count, k_max, num_splits, out,
                      lse, &s);
  if (rc || B == 0) return rc;
  const int rows = B * L->num_kv_heads;
  if (kvs::attn_partial_bytes(rows, s, L->num_q_heads / L->num_kv_heads, L->head_dim) > kNoAllocPartialBytes)
    return KV_ERR_WORKSPACE;
  char* base = nullptr;
  rc = scratch_on_current_device((hipStream_t)stream, &base);
  if (rc) return rc;
  const kvs::AttnScratch sc{reinterpret_cast<unsigned*>(base),
                            reinterpret_cast<float*>(base + kNoAllocCounterBytes)};
  return enqueue_step(L, q, summary, log_n, pg, block_table, seq_lens, B, max_pages, keep_frac, k_fixed, coverage,
                      n_force_first, n_force_last, head_scores, lse_partial, sel, sel_count, k_max, page_S, s, out,
                      lse, sc, (hipStream_t)stream);
}

size_t kv_hot_admit_workspace_size(int32_t n_slots, int32_t n_units) {
  if (n_slots < 1 || n_units < 1 || n_units > kvs::kAdmitMaxUnits || n_slots > kvs::kAdmitMaxSlots) return 0;
  return kvs::hot_admit_workspace_bytes(n_slots, n_units);
}

int kv_hot_admit(const kv_layout* L, const void* v16, void* v_hot, const void* k16, void* k_hot,
                 int32_t* v_hot_slot, int32_t n_units,
                 int32_t* slot_page, uint32_t* slot_stamp, int32_t n_slots, const int32_t* block_table,
                 const int32_t* seq_lens, int32_t B, int32_t max_pages, const int32_t* sel,
                 const int32_t* sel_count, int32_t k_max, uint32_t step, void* ws, size_t ws_bytes,
                 void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (B < 0 || max_pages < 0 || k_max < 0 || n_units < 1 || n_slots < 1 || step == 0) return KV_ERR_INVALID_ARG;
  if (n_units % L->num_kv_heads != 0) return KV_ERR_INVALID_ARG;
  if (n_units > kvs::kAdmitMaxUnits || n_slots > kvs::kAdmitMaxSlots) return KV_ERR_UNSUPPORTED;
  if (!v16 || !v_hot || !v_hot_slot || !slot_page || !slot_stamp) return KV_ERR_INVALID_ARG;
  if (!aligned16(v16) || !aligned16(v_hot)) return KV_ERR_INVALID_ARG;
  if (!k16 != !k_hot || (k16 && (!aligned16(k16) || !aligned16(k_hot)))) return KV_ERR_INVALID_ARG;
  if (B > 0 && k_max > 0 && (!block_table || !seq_lens || !sel || !sel_count)) return KV_ERR_INVALID_ARG;
  if ((int64_t)B * L->num_kv_heads * k_max > 0x7FFFFFFF) return KV_ERR_UNSUPPORTED;
  if (!ws || ((uintptr_t)ws & 3u) || ws_bytes < kv_hot_admit_workspace_size(n_slots, n_units)) return KV_ERR_WORKSPACE;
  return from_hip(kvs::launch_hot_admit(*L, v16, v_hot, k16, k_hot, v_hot_slot, n_units, slot_page, slot_stamp,
                                        n_slots, block_table, seq_lens, B, max_pages, sel, sel_count, k_max, step,
                                        (int32_t*)ws, (hipStream_t)stream));
}

int kv_dequant_tier(const kv_layout* L, const kv_pages* pg, const int32_t* pages, int32_t n,
                    float* out, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (n < 0) return KV_ERR_INVALID_ARG;
  if (n == 0) return KV_OK;
  if (!pages || !out) return KV_ERR_INVALID_ARG;
  rc = check_pages(L, pg);
  if (rc) return rc;
  return from_hip(kvs::launch_dequant_tier(*L, *pg, pages, n, out, (hipStream_t)stream));
}

int kv_tier_plan(const kv_layout* L, const float* page_S, const int32_t* seq_lens, int32_t B, int32_t max_pages,
                 const int32_t* block_table, const uint32_t* page_entry, const int32_t* caps,
                 int32_t n_force_first, int32_t n_force_last, int32_t* moves, int32_t* move_count, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (B < 0 || max_pages < 0 || n_force_first < 0 || n_force_last < 0 || !caps) return KV_ERR_INVALID_ARG;
  if (max_pages > kvs::kMaxTopkPages) return KV_ERR_UNSUPPORTED;
  if (B == 0 || max_pages == 0) return KV_OK;
  if (!page_S || !seq_lens || !block_table || !page_entry || !moves || !move_count) return KV_ERR_INVALID_ARG;
  int32_t c[5];
  for (int l = 0; l < 5; ++l) {
    if (caps[l] < 0) return KV_ERR_INVALID_ARG;
    c[l] = caps[l] < max_pages ? caps[l] : max_pages;
  }
  return from_hip(kvs::launch_tier_plan(*L, page_S, seq_lens, B, max_pages, block_table, page_entry, c,
                                        n_force_first, n_force_last, moves, move_count, (hipStream_t)stream));
}

int kv_tier_demote(const kv_layout* L, const kv_pages* pg, uint32_t* page_entry, int32_t B, int32_t max_pages,
                   const int32_t* moves, const int32_t* move_count, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (B < 0 || max_pages < 0) return KV_ERR_INVALID_ARG;
  if (B == 0 || max_pages == 0) return KV_OK;
  rc = check_pages(L, pg);
  if (rc) return rc;
  if (!page_entry || pg->page_entry != page_entry || !moves || !move_count) return KV_ERR_INVALID_ARG;
  return from_hip(kvs::launch_tier_demote(*L, *pg, page_entry, B, max_pages, moves, move_count,
                                          (hipStream_t)stream));
}

int kv_pack_tier(const kv_layout* L, const void* src16, const int32_t* src_pages, int32_t n,
                 int32_t tier, uint8_t* codes, void* scale_zero, uint32_t* outliers, const int32_t* dst_slots,
                 void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (tier < KV_TIER_I8 || tier > KV_TIER_FP8) return KV_ERR_UNSUPPORTED;
  if (outliers && tier != KV_TIER_B1) return KV_ERR_INVALID_ARG;
  if (n < 0) return KV_ERR_INVALID_ARG;
  if (n == 0) return KV_OK;
  if (!src16 || !codes || !scale_zero) return KV_ERR_INVALID_ARG;
  if (!aligned16(src16) || (reinterpret_cast<uintptr_t>(codes) & 3u) ||
      (reinterpret_cast<uintptr_t>(scale_zero) & 3u))
    return KV_ERR_INVALID_ARG;
  return from_hip(kvs::launch_pack_tier(*L, src16, src_pages, n, tier, codes, scale_zero, outliers, dst_slots,
                                        (hipStream_t)stream));
}

}  // extern "C"
