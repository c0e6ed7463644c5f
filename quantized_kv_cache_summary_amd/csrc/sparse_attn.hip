// Sparse paged decode attention over the selected pages only, split-K with a
// log-sum-exp merge.  AMASS (amass-kv 0.1.1 project page), "AMASS": each decode
// step attends only to the pages that carry attention mass, read by a sparse
// paged-attention kernel.  Packed tiers are rebuilt in registers just before
// use (ARGUS, argus_cache 0.1.7.1 project page, "Why It Works: Storage vs.
// Computation"); the arithmetic stays float32.
//
// gfx950 design.  One block of 4 waves per (row, split); the split's selected
// pages are dealt round-robin to the waves; a wave handles 16 tokens at a time.
//   QK^T: the G query heads of the group are the 16 B columns of a 16x16x32
//     MFMA, the 16 tokens its A rows.  Each lane loads d/4 contiguous elements
//     (64 bytes) of one token's key.  A packed page is decoded to float32 and
//     fed as an exact bf16 (or f16) hi + lo pair, two MFMAs per step.
//   softmax: the MFMA leaves head h / tokens 4g'+i in lane h + 16g'.  The
//     running max is shared by the four lane groups and only raised when a
//     chunk exceeds it by more than 2^8 (the stale max cancels exactly in
//     out = acc / l), so rescaling is rare.
//   PV: lane (token slot ts, element chunk ec) loads d/16 values of token
//     4j + ts, so the V page is read with 16-byte coalesced loads; the
//     probabilities reach it through a 1 KB per-wave LDS tile; acc[head][d/16]
//     accumulates in float32 FMAs.
// The four waves merge in LDS; the last block of a row to finish (a counter per
// row in the workspace) merges the row's splits into out and lse.
// With SEL the kernel also selects the pages: every block of a row runs the
// row's exact top-k (select.h) on the head scores in LDS and keeps the slice of
// the ascending page list its split owns, so the list never makes a round trip
// through memory and no selector launch sits between score and attention.  The
// selection is the separate selector's bit for bit, and the pages are dealt to
// the waves as in the plain kernel, so out and lse are too.  Partials
// cross blocks through device-coherent stores and loads: a release fence
// would write back the whole L2 and costs far more than the merge.

#include "attn_split.h"
#include "select.h"

namespace kvs {

template <int D, int GM, bool F16, bool TIERED, bool SEL>
__global__ __launch_bounds__((64 * attn_waves<GM, SEL>()))
__attribute__((amdgpu_waves_per_eu(attn_min_waves_per_simd<GM, TIERED, SEL>()))) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, PagesDev pg, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int Hkv, int G, int P, int max_pages,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int k_max, int n_splits,
    float scale_log2, float* __restrict__ partials, unsigned* __restrict__ counters,
    float* __restrict__ out, float* __restrict__ lse, SelArgs sa) {
  constexpr int KS = D / 32;     // MFMA k-steps
  constexpr int kAttnWaves = attn_waves<GM, SEL>();
  constexpr int kThreads = 64 * kAttnWaves;
  using ALds = AttnLds<kStreamWaves, GM, D>;
  using SLds = SelectLds<kThreads>;

  __shared__ typename std::conditional<SEL, char, ALds>::type al_static;
  extern __shared__ __align__(16) uint32_t sel_lds[];   // SEL only
  ALds* al;
  SLds* sshp = nullptr;
  uint32_t* keys = nullptr;
  int32_t* mine = nullptr;
  if constexpr (SEL) {
    const int off = sel_slice_words(k_max, n_splits);
    mine = reinterpret_cast<int32_t*>(sel_lds);
    al = reinterpret_cast<ALds*>(sel_lds + off);
    sshp = reinterpret_cast<SLds*>(sel_lds + off);
    keys = sel_lds + off + sizeof(SLds) / sizeof(uint32_t);
  } else {
    al = &al_static;
  }

  const int row = blockIdx.y, split = blockIdx.x;
  const int b = row / Hkv, g = row - b * Hkv;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;

  const int L = seq_lens[b];
  int Np = L > 0 ? (L + P - 1) / P : 0;
  Np = Np < max_pages ? Np : max_pages;
  int cnt;
  const float* hs_row = nullptr;
  SelectLoads<kThreads, GM> sld;
  if constexpr (SEL) {
    // head scores in flight before anything else is known
    hs_row = sa.head_scores + (size_t)row * G * max_pages;
    if (max_pages > 0)
      select_issue<kThreads, GM>(sld, hs_row, sa.lse_partial + (size_t)row * sa.n_tiles * G * 2, G, max_pages,
                                 sa.n_tiles);
    cnt = sa.coverage >= 0.f ? (Np > 0 ? 1 : 0) : selection_count(Np, sa.keep, sa.k_fixed);
  } else {
    cnt = sel_count[row];
    cnt = cnt < 0 ? 0 : (cnt > k_max ? k_max : cnt);
  }

  // B operand: query head `col`, at k-step s the elements [32s + 8grp, +8)
  // (the same assignment as the key rows); heads past G are zero.
  u32x4_t qop[KS];
  {
    const int Hq = Hkv * G;
    const uint32_t keep = col < G ? 0xFFFFFFFFu : 0u;
    const uint16_t* qp = q + ((size_t)b * Hq + (size_t)g * G + (col < G ? col : 0)) * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qop[s] = ld16(qp + 32 * s);
#pragma unroll
      for (int w = 0; w < 4; ++w) qop[s][w] &= keep;
    }
  }

  // SEL: the row's selection (identical in every block of the row); split 0
  // publishes it, every block keeps its own slice in LDS
  if constexpr (SEL) {
    SLds& ssh = *sshp;
    const bool writer = split == 0;
    const bool cov = sa.coverage >= 0.f;
    SelectStats sst{};
    if (cnt > 0) {
      sst = select_keys<kThreads, GM>(ssh, keys, sld, hs_row, G, max_pages, sa.n_tiles, Np, sa.n_force_first,
                                      sa.n_force_last,
                                      writer && sa.page_S ? sa.page_S + (size_t)row * max_pages : nullptr, cov);
      if (cov) {
        cnt = select_coverage_k<kThreads>(ssh, keys, Np, sst, sa.coverage, k_max);
        __syncthreads();             // every wave is done with the histograms
        if (threadIdx.x < 256) ssh.hist[0][threadIdx.x] = 0;
        __syncthreads();
      }
    }
    int32_t* sout = sa.sel + (size_t)row * k_max;
    if (writer) {
      for (int i = cnt + (int)threadIdx.x; i < k_max; i += kThreads) sout[i] = -1;
      if (threadIdx.x == 0) sa.sel_count[row] = cnt;
    }
    if (cnt > 0) {
      const int lo = (int)(((long long)split * cnt) / n_splits);
      const int hi = (int)(((long long)(split + 1) * cnt) / n_splits);
      uint32_t T;
      int take;
      select_kth<kThreads>(ssh, keys, Np, sst, cnt, T, take);
      select_compact<kThreads>(ssh, keys, Np, T, take, [&](int p, int pos) {
        if (writer && pos < cnt) sout[pos] = p;
        if (pos >= lo && pos < hi) mine[pos - lo] = p;
      });
    }
    __syncthreads();
  }
  attend_split<D, GM, F16, TIERED, SEL, kThreads>(pg, block_table, Hkv, G, P, max_pages, row, split, n_splits, cnt,
                                                 SEL ? mine : sel + (size_t)row * k_max, L, Np, qop,
                                                 scale_log2, partials, counters, nullptr, out, lse, al);
}

// Arguments shared by every instantiation's launch.
struct AttnLaunch {
  const void* q;
  PagesDev pd;
  const int32_t* bt;
  const int32_t* sl;
  int B, max_pages;
  const int32_t* sel;
  const int32_t* cnt;
  int k_max, n_splits;
  float tau;
  float* out;
  float* lse;
  AttnScratch sc;
  SelArgs sa;
  size_t dyn_lds;
};

template <int D, int GM, bool F16, bool TIERED, bool SEL>
static hipError_t launch_attn_t(const kv_layout& L, const AttnLaunch& a, hipStream_t st) {
  const int G = L.num_q_heads / L.num_kv_heads;
  const int rows = a.B * L.num_kv_heads;
  hipLaunchKernelGGL((sparse_attn_kernel<D, GM, F16, TIERED, SEL>), dim3(a.n_splits, rows),
                     dim3(64 * attn_waves<GM, SEL>()), a.dyn_lds, st, (const uint16_t*)a.q, a.pd, a.bt, a.sl,
                     L.num_kv_heads, G, L.page_size, a.max_pages, a.sel, a.cnt, a.k_max, a.n_splits,
                     a.tau * kLog2e, a.sc.partials, a.sc.counters, a.out, a.lse, a.sa);
  return hipGetLastError();
}

template <int D, bool F16, bool TIERED, bool SEL>
static hipError_t launch_attn_g(const kv_layout& L, const AttnLaunch& a, hipStream_t st) {
  const int G = L.num_q_heads / L.num_kv_heads;
  // the C ABI refuses groups wider than eight query heads for attention
  if (G <= 4) return launch_attn_t<D, 4, F16, TIERED, SEL>(L, a, st);
  return launch_attn_t<D, 8, F16, TIERED, SEL>(L, a, st);
}

template <bool SEL>
static hipError_t launch_attn_any(const kv_layout& L, const AttnLaunch& a, bool tiered, hipStream_t st) {
  const bool f16 = L.kv_dtype == KV_F16;
#define KVS_ATTN(D_, F16_)                                                              \
  return tiered ? launch_attn_g<D_, F16_, true, SEL>(L, a, st) : launch_attn_g<D_, F16_, false, SEL>(L, a, st)
  if (L.head_dim == 64) {
    if (f16) KVS_ATTN(64, true);
    KVS_ATTN(64, false);
  }
  if (f16) KVS_ATTN(128, true);
  KVS_ATTN(128, false);
#undef KVS_ATTN
}

hipError_t launch_sparse_attn(const kv_layout& L, const void* q, const kv_pages& pg,
                              const int32_t* block_table, const int32_t* seq_lens, int B,
                              int max_pages, const int32_t* sel, const int32_t* sel_count, int k_max,
                              int n_splits, float tau, float* out, float* lse, AttnScratch sc,
                              hipStream_t st) {
  AttnLaunch a{q, to_dev(pg), block_table, seq_lens, B, max_pages, sel, sel_count, k_max, n_splits,
               tau, out, lse, sc, SelArgs{}, 0};
  return launch_attn_any<false>(L, a, pg.page_entry != nullptr, st);
}

template <int D, int GM>
static size_t sel_dyn_bytes(int max_pages, int k_max, int n_splits) {
  constexpr int W = attn_waves<GM, true>();
  const size_t sel = sizeof(SelectLds<64 * W>) + (size_t)(max_pages > 0 ? max_pages : 1) * sizeof(uint32_t);
  const size_t att = sizeof(AttnLds<kStreamWaves, GM, D>);
  return (size_t)sel_slice_words(k_max, n_splits) * sizeof(uint32_t) + (sel > att ? sel : att);
}

size_t topk_attn_dyn_lds_bytes(const kv_layout& L, int max_pages, int k_max, int n_splits) {
  const int G = L.num_q_heads / L.num_kv_heads;
  if (L.head_dim == 64)
    return G <= 4 ? sel_dyn_bytes<64, 4>(max_pages, k_max, n_splits) : sel_dyn_bytes<64, 8>(max_pages, k_max, n_splits);
  return G <= 4 ? sel_dyn_bytes<128, 4>(max_pages, k_max, n_splits) : sel_dyn_bytes<128, 8>(max_pages, k_max, n_splits);
}

hipError_t launch_topk_sparse_attn(const kv_layout& L, const void* q, const kv_pages& pg,
                                   const int32_t* block_table, const int32_t* seq_lens, int B, int max_pages,
                                   const float* head_scores, const float* lse_partial, float keep, int k_fixed,
                                   float coverage, int n_force_first, int n_force_last, int32_t* sel,
                                   int32_t* sel_count, int k_max, float* page_S, int n_splits, float tau,
                                   float* out, float* lse, AttnScratch sc, hipStream_t st) {
  SelArgs sa{head_scores, lse_partial, keep, k_fixed, coverage, n_force_first, n_force_last,
             score_tiles(max_pages), sel, sel_count, page_S};
  AttnLaunch a{q, to_dev(pg), block_table, seq_lens, B, max_pages, nullptr, nullptr, k_max, n_splits,
               tau, out, lse, sc, sa, topk_attn_dyn_lds_bytes(L, max_pages, k_max, n_splits)};
  return launch_attn_any<true>(L, a, pg.page_entry != nullptr, st);
}

// ---------------------------------------------------------------- standalone decode

template <int D, bool F16>
__global__ __launch_bounds__(256) void dequant_kernel(PagesDev pg, const int32_t* __restrict__ pages,
                                                      int n, int Hkv, int P, float* __restrict__ out) {
  // one thread per (page i, K/V, head, token, 8-element run)
  constexpr int RUN = 8;
  const size_t total = (size_t)n * 2 * Hkv * P * (D / RUN);
  for (size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x; id < total;
       id += (size_t)gridDim.x * blockDim.x) {
    size_t r = id;
    const int run = (int)(r % (D / RUN)); r /= (D / RUN);
    const int tk = (int)(r % P); r /= P;
    const int g = (int)(r % Hkv); r /= Hkv;
    const int kv = (int)(r % 2); r /= 2;
    const int i = (int)r;
    const int phys = pages[i];
    uint32_t tier = 0, slot = (uint32_t)phys;
    if (pg.page_entry) {
      const uint32_t e = pg.page_entry[phys];
      tier = e >> 29;
      slot = e & 0x1FFFFFFFu;
    }
    const size_t prow = ((size_t)slot * Hkv + g) * P + tk;
    float x[RUN];
    if (tier == KV_TIER_NATIVE) {
      const uint16_t* src = (kv == 0 ? pg.k16 : pg.v16) + prow * D;
      if (pg.v_hot_slot && (kv == 1 || pg.k_hot)) {
        const int hs = pg.v_hot_slot[(size_t)phys * Hkv + g];
        if (hs >= 0) src = (kv == 0 ? pg.k_hot : pg.v_hot) + ((size_t)hs * P + tk) * D;
      }
      const u32x4_t w = ld16(src + run * RUN);
#pragma unroll
      for (int j = 0; j < 4; ++j) { x[2 * j] = lo16<F16>(w[j]); x[2 * j + 1] = hi16<F16>(w[j]); }
    } else {
      const int t = (int)tier - 1;
      const uint8_t* codes = kv == 0 ? pg.kq[t] : pg.vq[t];
      const uint16_t* sz = kv == 0 ? pg.ksz[t] : pg.vsz[t];
      switch (tier) {
        case KV_TIER_I8: decode_run<D, RUN, 8>(codes, sz, prow, run * RUN, x); break;
        case KV_TIER_I4: decode_run<D, RUN, 4>(codes, sz, prow, run * RUN, x); break;
        case KV_TIER_I2: decode_run<D, RUN, 2>(codes, sz, prow, run * RUN, x); break;
        case KV_TIER_FP8: decode_fp8<D, RUN>(codes, sz, prow, run * RUN, x); break;
        default:
          decode_run<D, RUN, 1>(codes, sz, prow, run * RUN, x);
          if (pg.kout) apply_outlier<RUN>(x, run * RUN, (kv == 0 ? pg.kout : pg.vout)[prow * (D / 32) + run * RUN / 32]);
          break;
      }
    }
    float* dst = out + ((((size_t)i * 2 + kv) * Hkv + g) * P + tk) * D + run * RUN;
#pragma unroll
    for (int j = 0; j < RUN; ++j) dst[j] = x[j];
  }
}

hipError_t launch_dequant_tier(const kv_layout& L, const kv_pages& pg, const int32_t* pages, int n,
                               float* out, hipStream_t st) {
  const PagesDev pd = to_dev(pg);
  const size_t total = (size_t)n * 2 * L.num_kv_heads * L.page_size * (L.head_dim / 8);
  const int blocks = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  const bool f16 = L.kv_dtype == KV_F16;
  if (L.head_dim == 64) {
    if (f16) hipLaunchKernelGGL((dequant_kernel<64, true>), dim3(blocks), dim3(256), 0, st, pd, pages, n, L.num_kv_heads, L.page_size, out);
    else hipLaunchKernelGGL((dequant_kernel<64, false>), dim3(blocks), dim3(256), 0, st, pd, pages, n, L.num_kv_heads, L.page_size, out);
  } else {
    if (f16) hipLaunchKernelGGL((dequant_kernel<128, true>), dim3(blocks), dim3(256), 0, st, pd, pages, n, L.num_kv_heads, L.page_size, out);
    else hipLaunchKernelGGL((dequant_kernel<128, false>), dim3(blocks), dim3(256), 0, st, pd, pages, n, L.num_kv_heads, L.page_size, out);
  }
  return hipGetLastError();
}

}  // namespace kvs
