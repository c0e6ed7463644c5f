// Internal launchers: the C ABI (capi.cpp) validates arguments, then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kvsparse.h"

namespace kvs {

// Pages of 16 logical pages per MFMA tile; a score block covers this many pages.
constexpr int kScorePagesPerBlock = 64;
constexpr int kTopkThreads = 512;        // selector block; rows of kTopkWideFrom pages or more get twice this
constexpr int kTopkWideFrom = 4096;
constexpr int kMaxTopkPages = 15360;   // keys in LDS stay under 64 KB
constexpr int kMaxSplits = 256;

inline int score_tiles(int max_pages) { return (max_pages + kScorePagesPerBlock - 1) / kScorePagesPerBlock; }

// Attention workspace: one uint32 counter per row first (zero between calls),
// then per (row, split, head) partials [d + 2] floats from a 256-byte boundary.
// The counters sit at a fixed offset whatever the split count or page kind, so
// one workspace serves calls with different split counts over the same rows.
inline size_t attn_counter_bytes(int rows) { return ((size_t)rows * sizeof(unsigned) + 255) & ~(size_t)255; }
inline size_t attn_partial_bytes(int rows, int splits, int G, int d) {
  return (size_t)rows * splits * G * (d + 2) * sizeof(float);
}
inline size_t attn_workspace_bytes(int rows, int splits, int G, int d) {
  return attn_counter_bytes(rows) + attn_partial_bytes(rows, splits, G, d);
}

// Where the attention keeps its cross-block state: one counter per row (zero
// between calls) and the split partials.
struct AttnScratch {
  unsigned* counters;
  float* partials;
};
inline AttnScratch attn_scratch_in(void* ws, int rows) {
  return AttnScratch{reinterpret_cast<unsigned*>(ws),
                     reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + attn_counter_bytes(rows))};
}

// Shared-basis build: covariance statistics per (row, chunk of pages), then
// one merge + eigen block per row.  Workspace: [rows][chunks][1 + d + d*d] floats.
constexpr int kBasisChunkPages = 256;
inline int basis_chunks(int max_pages) { return (max_pages + kBasisChunkPages - 1) / kBasisChunkPages; }
inline size_t basis_workspace_bytes(int rows, int max_pages, int d) {
  return (size_t)rows * basis_chunks(max_pages) * (size_t)(1 + d + d * d) * sizeof(float);
}

hipError_t launch_basis_build(const kv_layout& L, const void* k16, const int32_t* block_table,
                              const int32_t* seq_lens, int B, int max_pages, float* basis, float* mean,
                              float* part, hipStream_t st);

hipError_t launch_lowrank_coords(const kv_layout& L, const void* k16, const int32_t* block_table, int max_pages,
                                 const int32_t* entries, const int32_t* n_valid, int n, const float* basis,
                                 const float* mean, void* coords, hipStream_t st);

hipError_t launch_page_score_lowrank(const kv_layout& L, const void* q, const void* coords, const float* mean,
                                     const float* basis, const int32_t* seq_lens, int B, int max_pages,
                                     float tau, float* head_scores, float* lse_partial, hipStream_t st);

hipError_t launch_summary_build_basis(const kv_layout& L, const void* k16, const int32_t* block_table,
                                      int max_pages, const int32_t* entries, const int32_t* n_valid, int n,
                                      const float* basis, void* mu, float* lam, float* log_n,
                                      hipStream_t st);

hipError_t launch_page_score_basis(const kv_layout& L, const void* q, const void* mu, const float* lam,
                                   const float* basis, const float* log_n, const int32_t* seq_lens, int B,
                                   int max_pages, float tau, float* head_scores, float* lse_partial,
                                   hipStream_t st);

// Hot-buffer admission: units u = phys * Hkv + g, limits, and the workspace
// (int32 words): count, (unit, slot) pairs, miss list, then at 64-word
// boundaries the unit bitmap, the slot keys, the per-block miss counts, the
// per-block victim counts and three scalars.
constexpr int kAdmitMaxUnits = 1 << 24;
constexpr int kAdmitMaxSlots = 1 << 22;
struct HotAdmitWs { size_t bits, keys, wcnt, vcnt, scal, words; };
inline HotAdmitWs hot_admit_ws_layout(int n_slots, int n_units) {
  auto up64 = [](size_t x) { return (x + 63) & ~(size_t)63; };
  const size_t n_words = ((size_t)n_units + 31) >> 5;
  const size_t n_wblocks = (n_words + 255) / 256, n_sblocks = ((size_t)n_slots + 255) / 256;
  HotAdmitWs l;
  l.bits = up64(1 + 3 * (size_t)n_slots);
  l.keys = up64(l.bits + n_words);
  l.wcnt = up64(l.keys + (size_t)n_slots);
  l.vcnt = up64(l.wcnt + n_wblocks);
  l.scal = up64(l.vcnt + 2 * n_sblocks);
  l.words = l.scal + 4;
  return l;
}
inline size_t hot_admit_workspace_bytes(int n_slots, int n_units) {
  return hot_admit_ws_layout(n_slots, n_units).words * sizeof(int32_t);
}

hipError_t launch_hot_admit(const kv_layout& L, const void* v16, void* v_hot, const void* k16, void* k_hot,
                            int32_t* hot, int n_units,
                            int32_t* slot_page, uint32_t* slot_stamp, int n_slots, const int32_t* block_table,
                            const int32_t* seq_lens, int B, int max_pages, const int32_t* sel,
                            const int32_t* sel_count, int k_max, uint32_t step, int32_t* ws, hipStream_t st);

hipError_t launch_summary_build(const kv_layout& L, const void* k16, const int32_t* block_table,
                                int max_pages, const int32_t* entries, const int32_t* n_valid, int n,
                                void* summary, float* log_n, hipStream_t st);

hipError_t launch_page_score(const kv_layout& L, const void* q, const void* summary,
                             const float* log_n, const int32_t* seq_lens, int B, int max_pages,
                             float tau, float* head_scores, float* lse_partial, hipStream_t st);

// coverage < 0: budget mode (keep / k_fixed); coverage >= 0: coverage mode.
hipError_t launch_page_topk(const kv_layout& L, const float* head_scores, const float* lse_partial,
                            const int32_t* seq_lens, int B, int max_pages, float keep, int k_fixed,
                            float coverage, int n_force_first, int n_force_last, int32_t* sel,
                            int32_t* sel_count, int k_max, float* page_S, hipStream_t st);

hipError_t launch_sparse_attn(const kv_layout& L, const void* q, const kv_pages& pg,
                              const int32_t* block_table, const int32_t* seq_lens, int B,
                              int max_pages, const int32_t* sel, const int32_t* sel_count, int k_max,
                              int n_splits, float tau, float* out, float* lse, AttnScratch sc,
                              hipStream_t st);

// Fused selector + attention: every block of a row selects the row's pages
// (as launch_page_topk) and attends over its split's slice of them.  Dynamic
// LDS: the slice, then the selector's state and the row's keys, reused by the
// attention afterwards.  Kept under 64 KB (the fused call refuses larger).
size_t topk_attn_dyn_lds_bytes(const kv_layout& L, int max_pages, int k_max, int n_splits);
constexpr size_t kTopkAttnMaxLds = 64 * 1024 - 64;

hipError_t launch_topk_sparse_attn(const kv_layout& L, const void* q, const kv_pages& pg,
                                   const int32_t* block_table, const int32_t* seq_lens, int B, int max_pages,
                                   const float* head_scores, const float* lse_partial, float keep, int k_fixed,
                                   float coverage, int n_force_first, int n_force_last, int32_t* sel,
                                   int32_t* sel_count, int k_max, float* page_S, int n_splits, float tau,
                                   float* out, float* lse, AttnScratch sc, hipStream_t st);

hipError_t launch_dequant_tier(const kv_layout& L, const kv_pages& pg, const int32_t* pages, int n,
                               float* out, hipStream_t st);

hipError_t launch_tier_plan(const kv_layout& L, const float* page_S, const int32_t* seq_lens, int B,
                            int max_pages, const int32_t* block_table, const uint32_t* page_entry,
                            const int32_t* caps, int n_force_first, int n_force_last, int32_t* moves,
                            int32_t* move_count, hipStream_t st);

hipError_t launch_tier_demote(const kv_layout& L, const kv_pages& pg, uint32_t* page_entry, int B, int max_pages,
                              const int32_t* moves, const int32_t* move_count, hipStream_t st);

hipError_t launch_pack_tier(const kv_layout& L, const void* src16, const int32_t* src_pages, int n,
                            int tier, uint8_t* codes, void* scale_zero, uint32_t* outliers,
                            const int32_t* dst_slots, hipStream_t st);

}  // namespace kvs
