"""Sparse paged decode attention (test infrastructure only).

AMASS (amass-kv 0.1.1 project page), section "AMASS": each decode step attends
only to the selected pages, read by a sparse paged-attention kernel.  Reading:
softmax attention of each query head over the tokens of the selected pages
(renormalised over those tokens, no correction for the dropped mass), with
the natural-log log-sum-exp of the logits returned beside the output.

  z_i = tau q . k_i,   m = max z,   l = sum exp(z_i - m)
  o   = sum exp(z_i - m) v_i / l,   lse = m + log l
An empty token set gives o = 0 and lse = -inf.

Pinned in tests/test_oracle_attention.py against torch's
scaled_dot_product_attention in float64 on the CPU (selecting all pages equals
dense attention), one-token and equal-logit closed forms.
"""

import numpy as np


def dense_attention(q, keys, values, tau):
    """q (G, d), keys (T, d), values (T, dv) -> (out (G, dv), lse (G,)) in float64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(keys, dtype=np.float64)
    V = np.asarray(values, dtype=np.float64)
    G = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((G, V.shape[1])), np.full(G, -np.inf)
    z = tau * (q @ K.T)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ V) / l, (m + np.log(l))[:, 0]


def sparse_attention(q, keys, values, seq_len, page_size, selected, tau):
    """Attention over the tokens of the selected logical pages.

    keys, values: (L, d) logical token order of one (sequence, KV head).
    selected: logical page indices.  Tokens at or beyond seq_len are excluded.
    """
    tok = []
    for p in selected:
        lo = int(p) * page_size
        tok.extend(range(lo, min(lo + page_size, seq_len)))
    tok = np.asarray(tok, dtype=np.int64)
    K = np.asarray(keys)[tok] if tok.size else np.zeros((0, np.asarray(keys).shape[1]))
    V = np.asarray(values)[tok] if tok.size else np.zeros((0, np.asarray(values).shape[1]))
    return dense_attention(q, K, V, tau)
