"""Pins for the oracle's rounding helpers and paging (CPU only).

Rounding is checked against independent IEEE implementations (numpy's float16
cast, torch's bfloat16 cast) and against hand-computed boundary values; paging
against a token-by-token enumeration.
"""

import numpy as np
import torch

from oracle.rounding import round_bf16, round_fp16_sat
from oracle.paging import num_pages, page_token_counts, logical_page_tokens


def test_fp16_matches_numpy_cast_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000),
                        rng.uniform(-65504, 65504, 2000)])
    x = x[np.abs(x) <= 65504]
    ref = x.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(round_fp16_sat(x), ref)


def test_fp16_boundaries_and_saturation():
    assert round_fp16_sat(65504.0) == 65504.0
    assert round_fp16_sat(70000.0) == 65504.0
    assert round_fp16_sat(-1e9) == -65504.0
    assert round_fp16_sat(2.0 ** -24) == 2.0 ** -24          # smallest subnormal
    assert round_fp16_sat(2.0 ** -25) == 0.0                  # tie to even (zero)
    assert round_fp16_sat(1.5 * 2.0 ** -25) == 2.0 ** -24
    assert round_fp16_sat(1.0 + 2.0 ** -11) == 1.0            # tie -> even
    assert round_fp16_sat(1.0 + 3 * 2.0 ** -11) == 1.0 + 2.0 ** -9
    assert round_fp16_sat(31.0 / 15.0) == 2.06640625


def test_bf16_matches_torch_cast_for_float32_inputs():
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x32.astype(np.float64)), ref)


def test_bf16_rounds_directly_from_float64():
    # just above the midpoint between 1 and 1 + 2^-7: a detour through float32
    # would drop the 2^-40 and tie to 1.0
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert round_bf16(x) == 1.0 + 2.0 ** -7
    assert round_bf16(1.0 + 2.0 ** -8) == 1.0                 # exact tie -> even
    assert round_bf16(float.fromhex("0x1.ffp127")) == np.inf  # overflow
    assert np.isnan(round_bf16(np.nan))


def test_paging_matches_enumeration():
    for L in [0, 1, 15, 16, 17, 31, 32, 33, 1000, 1024]:
        for P in [16, 32]:
            owner = [t // P for t in range(L)]
            npg = num_pages(L, P)
            assert npg == (max(owner) + 1 if L else 0)
            counts = page_token_counts(L, P)
            for p in range(npg):
                toks = [t for t in range(L) if owner[t] == p]
                assert counts[p] == len(toks)
                assert list(logical_page_tokens(p, L, P)) == toks
