"""Pins of the oracle's importance estimate against facts outside itself.

* the page's reshape listing (token order of each reshaped slice);
* stride 1: the estimate reduces to block sums of exact causal attention
  probabilities, obtained from torch's scaled_dot_product_attention with
  identity values (a library routine, not the oracle's formula);
* stride > 1: each reshaped score equals the antidiagonal sum of the
  token-level score tile, computed by brute-force loops;
* invariants: each query block's scores sum to block/stride (rows are
  probability distributions), blocks right of the diagonal are zero, the
  streaming three-stage form equals the one-shot form, and a chunk's rows
  equal the matching rows of a one-shot estimate over the whole sequence.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import xattn_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa_probs(q, k, q_start_pos):
    """Exact attention probabilities [Lq, Lk] of one head via torch SDPA with V = I."""
    Lq, d = q.shape
    Lk = k.shape[0]
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(k)[None, None]
    eye = torch.eye(Lk, dtype=torch.float64)[None, None]
    vis = (torch.arange(Lk)[None, :] <= (q_start_pos + torch.arange(Lq))[:, None])
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, eye, attn_mask=vis)
    return out[0, 0].numpy()


def test_reshape_order_matches_page_listing():
    gold = json.load(open(os.path.join(GOLD, "reshape_order_stride8.json")))
    S = gold["stride"]
    L = 64
    pos = np.arange(L, dtype=np.float64)[:, None]          # feature = token position
    qr = O.reshape_q_inverse(pos, S)                        # [L/S, S]
    kr = O.reshape_k_forward(pos, S)
    assert qr.shape == (L // S, S) and kr.shape == (L // S, S)
    # slice t of the concatenation is column t (feature width 1)
    for t, start in enumerate(gold["k_slice_starts"]):
        assert kr[0, t] == start
        np.testing.assert_array_equal(kr[:, t], np.arange(start, L, S))
    for t, start in enumerate(gold["q_slice_starts"]):
        assert qr[0, t] == start
        np.testing.assert_array_equal(qr[:, t], np.arange(start, L, S))
    np.testing.assert_array_equal(kr[:3, 0], gold["k_first_positions_of_slice0"])
    np.testing.assert_array_equal(kr[:3, S - 1], gold["k_first_positions_of_slice7"])
    np.testing.assert_array_equal(qr[:3, 0], gold["q_first_positions_of_slice0"])
    np.testing.assert_array_equal(qr[:3, S - 1], gold["q_first_positions_of_slice7"])


@pytest.mark.parametrize("q_start_pos", [0, 256])
def test_stride1_equals_exact_attention_block_sums(q_start_pos):
    rng = np.random.default_rng(1)
    d, B, Lq = 16, 32, 128
    Lk = q_start_pos + Lq
    q = rng.standard_normal((Lq, d))
    k = rng.standard_normal((Lk, d))
    A = O.estimate_head(q, k, q_start_pos, stride=1, block=B)
    P = _sdpa_probs(q, k, q_start_pos)
    ref = P.reshape(Lq // B, B, Lk // B, B).sum(axis=(1, 3))
    np.testing.assert_allclose(A, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("S", [2, 4, 8])
def test_reshaped_score_is_antidiagonal_tile_sum(S):
    rng = np.random.default_rng(2)
    d, L = 8, 48
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    z = O.reshaped_logits(q, k, S)
    for r in range(L // S):
        for c in range(L // S):
            acc = 0.0
            for t in range(S):                    # query token r*S+S-1-t meets key token c*S+t
                qi = r * S + S - 1 - t
                kj = c * S + t
                acc += sum(q[qi, e] * k[kj, e] for e in range(d))
            assert abs(z[r, c] - acc / (S * math.sqrt(d))) < 1e-12


@pytest.mark.parametrize("S,p", [(8, 0), (8, 512), (16, 256), (4, 128)])
def test_row_sums_and_causal_zero(S, p):
    rng = np.random.default_rng(3)
    Lq, d, B = 256, 16, 128
    q = rng.standard_normal((Lq, 2, d))
    k = rng.standard_normal((p + Lq, 1, d))
    A = O.estimate_scores(q, k, p, S, B)
    nQB = Lq // B
    np.testing.assert_allclose(A.sum(axis=2), np.full((2, nQB), B // S), rtol=1e-12)
    cur = p // B
    for qb in range(nQB):
        assert np.all(A[:, qb, cur + qb + 1:] == 0.0)
        assert np.all(A[:, qb, :cur + qb + 1] > 0.0)


@pytest.mark.parametrize("S", [8, 16])
def test_streaming_three_stage_form_equals_one_shot(S):
    rng = np.random.default_rng(4)
    Lq, d, B, p = 256, 16, 128, 512
    q = rng.standard_normal((Lq, 2, d))
    k = rng.standard_normal((p + Lq, 1, d))
    one = O.estimate_scores(q, k, p, S, B)
    for kv_chunk in (128, 256, 384):
        st = O.estimate_scores_kv_chunked(q, k, p, S, B, kv_chunk)
        np.testing.assert_allclose(st, one, rtol=1e-12, atol=1e-15)


def test_chunk_rows_equal_one_shot_rows():
    rng = np.random.default_rng(5)
    L, d, B, S, C = 768, 16, 128, 8, 256
    q = rng.standard_normal((L, 2, d))
    k = rng.standard_normal((L, 2, d))
    full = O.estimate_scores(q, k, 0, S, B)
    for p in range(0, L, C):
        part = O.estimate_scores(q[p:p + C], k[:p + C], p, S, B)
        np.testing.assert_allclose(part, full[:, p // B:(p + C) // B, :(p + C) // B],
                                   rtol=1e-12, atol=1e-15)


def test_gqa_heads_read_their_group():
    rng = np.random.default_rng(6)
    L, d, B, S = 256, 16, 128, 8
    q = rng.standard_normal((L, 4, d))
    k = rng.standard_normal((L, 2, d))
    A = O.estimate_scores(q, k, 0, S, B)
    for h in range(4):
        np.testing.assert_array_equal(A[h], O.estimate_head(q[:, h], k[:, h // 2], 0, S, B))
    # heads 0/1 differ from what kv head 1 would give
    assert not np.allclose(A[0], O.estimate_head(q[:, 0], k[:, 1], 0, S, B))
