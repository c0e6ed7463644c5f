"""CPU oracle for importance-based sparse decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
numpy implementation of what the GPU path computes.  Only the tests, the
``smoke()`` check of ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (the HIP library and its Python
binding) never imports, calls or links anything here, and this package never
imports the product path.

Precision: float64 everywhere, except the packed-tier encoder, which is a
bit-level codec definition and is therefore specified step by step in IEEE
float32 (see ``oracle.codec``).

Sources (the method has no published formulas; every exact definition below is
a stated reading of the prose, listed in the design notes):

* AMASS, "decode-time sparse KV-cache attention for vLLM" (amass-kv 0.1.1
  project page): the decode step (section "AMASS"), the quad page score from a
  tiny per-page summary (section "What is in the box", item 1), the fixed
  budget / per-head coverage selection rule (section "Quickstart", the
  AmassConfig fields) and the top-B stage (section "Benchmarking").
* ARGUS, "Virtual Memory for Transformers" (argus_cache 0.1.7.1 project page):
  the packed low-bit tiers (sections "The One-Minute Explanation", "Visual
  Architecture" and the tier legend) and reconstruction of packed pages just
  before attention (section "Why It Works: Storage vs. Computation").

Parity status per function is stated in each module's header.
"""

from .rounding import round_bf16, round_fp16_sat, as_float32
from .paging import page_token_counts, num_pages, logical_page_tokens
from .summary import summarize_page, store_summary, summarize_and_store
from .score import page_score, exact_page_logmass
from .basis import (row_basis, row_covariance, store_basis, basis_page_stats, store_basis_summary,
                    page_score_basis)
from .select import group_aggregate, selection_count, select_pages, coverage_count
from .attention import sparse_attention, dense_attention
from .codec import (
    BITS_OF_TIER, TIER_NATIVE, TIER_I8, TIER_I4, TIER_I2, TIER_B1, TIER_FP8, FP8_MAX,
    encode_group_int, encode_group_1bit, encode_group_fp8, e4m3_magnitudes, e4m3_value, round_e4m3,
    encode_vector, decode_vector, outlier_words, apply_outliers,
    pack_codes, unpack_codes,
)
from .hotbuffer import HotBuffer, selected_physical_pages, selected_units
from .lowrank import row_mean, store_mean, key_coords, row_lowrank, page_score_lowrank
from .cascade import (TIER_OF_LEVEL, LEVEL_OF_TIER, page_importance, rank_pages, desired_levels, plan_row,
                      retier_vectors)
from .pipeline import decode_row

__all__ = [
    "round_bf16", "round_fp16_sat", "as_float32",
    "page_token_counts", "num_pages", "logical_page_tokens",
    "summarize_page", "store_summary", "summarize_and_store",
    "page_score", "exact_page_logmass",
    "row_basis", "row_covariance", "store_basis", "basis_page_stats", "store_basis_summary",
    "page_score_basis",
    "group_aggregate", "selection_count", "select_pages", "coverage_count",
    "sparse_attention", "dense_attention",
    "BITS_OF_TIER", "TIER_NATIVE", "TIER_I8", "TIER_I4", "TIER_I2", "TIER_B1", "TIER_FP8", "FP8_MAX",
    "encode_group_int", "encode_group_1bit", "encode_group_fp8", "e4m3_magnitudes", "e4m3_value",
    "round_e4m3", "encode_vector", "decode_vector", "outlier_words", "apply_outliers",
    "pack_codes", "unpack_codes",
    "HotBuffer", "selected_physical_pages", "selected_units",
    "row_mean", "store_mean", "key_coords", "row_lowrank", "page_score_lowrank",
    "TIER_OF_LEVEL", "LEVEL_OF_TIER", "page_importance", "rank_pages", "desired_levels", "plan_row",
    "retier_vectors",
    "decode_row",
]
