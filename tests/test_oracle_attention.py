"""Pins for sparse attention (CPU only): torch's SDPA in float64 and closed forms."""

import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle.attention import dense_attention, sparse_attention
from oracle.pipeline import decode_row


def test_dense_matches_torch_sdpa_float64():
    rng = np.random.default_rng(0)
    for G, T, d in [(4, 37, 64), (8, 300, 128), (1, 1, 16)]:
        q = rng.standard_normal((G, d))
        K = rng.standard_normal((T, d))
        V = rng.standard_normal((T, d))
        tau = 1 / math.sqrt(d)
        out, lse = dense_attention(q, K, V, tau)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None, None], torch.from_numpy(K)[None, None],
                                             torch.from_numpy(V)[None, None], scale=tau)[0, 0].numpy()
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
        ref_lse = torch.logsumexp(torch.from_numpy(tau * q @ K.T), dim=1).numpy()
        np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 8))
    v = rng.standard_normal((1, 8))
    k = rng.standard_normal((1, 8))
    out, lse = dense_attention(q, k, v, 0.5)
    np.testing.assert_allclose(out, np.repeat(v, 3, 0), atol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * (q @ k.T)[:, 0], atol=1e-15)
    K = np.zeros((5, 8))
    V = rng.standard_normal((5, 8))
    out, lse = dense_attention(q, K, V, 0.5)
    np.testing.assert_allclose(out, np.repeat(V.mean(0, keepdims=True), 3, 0), atol=1e-15)
    np.testing.assert_allclose(lse, np.full(3, math.log(5)), atol=1e-15)
    out, lse = dense_attention(q, np.zeros((0, 8)), np.zeros((0, 8)), 0.5)
    assert not out.any() and np.all(lse == -np.inf)


def test_sparse_selects_tokens_of_pages_and_respects_seq_len():
    rng = np.random.default_rng(2)
    L, P, d = 45, 16, 8                    # three pages, the last one partial (13 tokens)
    K = rng.standard_normal((48, d))
    V = rng.standard_normal((48, d))
    q = rng.standard_normal((2, d))
    out, lse = sparse_attention(q, K, V, L, P, [0, 2], 0.3)
    toks = list(range(0, 16)) + list(range(32, 45))
    ref, ref_lse = dense_attention(q, K[toks], V[toks], 0.3)
    np.testing.assert_allclose(out, ref, atol=1e-15)
    np.testing.assert_allclose(lse, ref_lse, atol=1e-15)


def test_all_pages_selected_equals_dense():
    rng = np.random.default_rng(3)
    L, P, d, G = 100, 16, 32, 4
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    q = rng.standard_normal((G, d))
    tau = 1 / math.sqrt(d)
    r = decode_row(q, K, V, L, P, rank=2, tau=tau, k_fixed=100)
    assert list(r["sel"]) == list(range(7))
    ref, ref_lse = dense_attention(q, K, V, tau)
    np.testing.assert_allclose(r["out"], ref, atol=1e-12)
    np.testing.assert_allclose(r["lse"], ref_lse, atol=1e-12)
