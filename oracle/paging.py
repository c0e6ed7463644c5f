"""Paging of one sequence's KV cache (test infrastructure only).

AMASS (amass-kv 0.1.1 project page), section "AMASS": the cache is paged and
each decode step reads only selected pages; ARGUS (argus_cache 0.1.7.1 project
page), section "The One-Minute Explanation": pages are the unit that moves
between tiers.  Reading: a sequence of L tokens with page size P has
ceil(L / P) logical pages; page p holds tokens [p*P, min((p+1)*P, L)); a block
table maps each logical page to a physical page of the pool.

Pinned by brute force (enumerating every token) in tests/test_oracle_paging.py.
"""

import numpy as np


def num_pages(seq_len, page_size):
    """Number of logical pages, ceil(L / P)."""
    return -(-int(seq_len) // int(page_size))


def page_token_counts(seq_len, page_size):
    """n_p, the number of valid tokens of every logical page (int64 array)."""
    npg = num_pages(seq_len, page_size)
    starts = np.arange(npg, dtype=np.int64) * page_size
    return np.minimum(page_size, seq_len - starts)


def logical_page_tokens(page, seq_len, page_size):
    """Token indices held by logical page ``page``."""
    lo = page * page_size
    return np.arange(lo, min(lo + page_size, seq_len), dtype=np.int64)
