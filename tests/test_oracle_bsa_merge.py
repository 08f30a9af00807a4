"""Pins of the oracle's block-sparse attention, LSE merge and chunked prefill.

* all-ones masks with causality equal torch's scaled_dot_product_attention
  (float64, explicit causal mask at the chunk's global offset);
* random block masks equal SDPA with the block mask expanded to tokens;
* LSE is pinned through SDPA too: append one extra key with score 0 whose
  value is an indicator column; the output in that column is
  1 / (exp(lse) + 1);
* tiny cases by pure-Python brute force;
* merge: an empty partial (lse -inf) is the identity, the merge is
  symmetric, and attention over two disjoint key sets merged by LSE equals
  attention over their union;
* chunked prefill at threshold 1 equals one-shot causal SDPA over the whole
  sequence.
"""
import math

import numpy as np
import pytest
import torch

from oracle import xattn_oracle as O

F = torch.nn.functional


def _sdpa(q, k, v, allowed):
    """q [Lq,d], k/v [Lk,d], allowed bool [Lq,Lk] -> out [Lq,d] (float64)."""
    return F.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], attn_mask=torch.from_numpy(allowed))[0, 0].numpy()


def _sdpa_lse(q, k, allowed):
    """Natural-log LSE per row via SDPA with an extra zero-score key."""
    Lq, d = q.shape
    Lk = k.shape[0]
    k2 = np.concatenate([k, np.zeros((1, d))], axis=0)
    v2 = np.zeros((Lk + 1, 1))
    v2[Lk, 0] = 1.0
    a2 = np.concatenate([allowed, np.ones((Lq, 1), dtype=bool)], axis=1)
    o = _sdpa(q, k2, v2, a2)[:, 0]
    return np.log(1.0 / o - 1.0)


def _token_allowed(mask_h, Lq, kv_len, p, kv_start, causal, B):
    qi = np.arange(Lq)[:, None]
    kj = np.arange(kv_len)[None, :]
    allowed = mask_h[qi // B, (kv_start + kj) // B].astype(bool)
    if causal:
        allowed &= (kv_start + kj) <= (p + qi)
    return allowed


@pytest.mark.parametrize("p,kv_start,kv_len,causal", [
    (0, 0, 256, True), (256, 0, 256, False), (256, 256, 256, True), (384, 0, 640, True)])
def test_bsa_all_ones_equals_sdpa(p, kv_start, kv_len, causal):
    rng = np.random.default_rng(10)
    B, d, Lq = 128, 32, 256
    q = rng.standard_normal((Lq, 2, d))
    k = rng.standard_normal((kv_len, 1, d))
    v = rng.standard_normal((kv_len, 1, d))
    nCols = (kv_start + kv_len) // B
    mask = np.ones((2, Lq // B, nCols), dtype=np.uint8)
    out, lse = O.bsa(q, k, v, p, kv_start, mask, 0, causal, None, B)
    for h in range(2):
        allowed = _token_allowed(mask[h], Lq, kv_len, p, kv_start, causal, B)
        np.testing.assert_allclose(out[:, h], _sdpa(q[:, h], k[:, 0], v[:, 0], allowed),
                                   rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[h], _sdpa_lse(q[:, h], k[:, 0], allowed),
                                   rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("seed", range(4))
def test_bsa_random_mask_equals_sdpa(seed):
    rng = np.random.default_rng(20 + seed)
    B, d, Lq, p = 128, 16, 384, 256
    kv_len = p + Lq
    q = rng.standard_normal((Lq, 4, d))
    k = rng.standard_normal((kv_len, 2, d))
    v = rng.standard_normal((kv_len, 2, d))
    nQB, nKB = Lq // B, kv_len // B
    mask = (rng.random((4, nQB, nKB)) < 0.5).astype(np.uint8)
    mask[:, :, 0] = 1                              # keep every row non-empty for SDPA
    out, lse = O.bsa(q, k, v, p, 0, mask, 0, True, None, B)
    for h in range(4):
        allowed = _token_allowed(mask[h], Lq, kv_len, p, 0, True, B)
        np.testing.assert_allclose(out[:, h], _sdpa(q[:, h], k[:, h // 2], v[:, h // 2], allowed),
                                   rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[h], _sdpa_lse(q[:, h], k[:, h // 2], allowed),
                                   rtol=1e-9, atol=1e-9)


def test_bsa_mask_offset_and_history_segment():
    rng = np.random.default_rng(30)
    B, d, Lq, p = 128, 16, 128, 384
    k = rng.standard_normal((p + Lq, 1, d))
    v = rng.standard_normal((p + Lq, 1, d))
    q = rng.standard_normal((Lq, 1, d))
    full_mask = np.array([[[1, 0, 1, 1]]], dtype=np.uint8)
    # history [128, 384) passed as its own segment with a mask that starts at block 1
    o1, l1 = O.bsa(q, k[B:p], v[B:p], p, B, full_mask[:, :, 1:], 1, False, None, B)
    o2, l2 = O.bsa(q, k[:p], v[:p], p, 0, np.array([[[0, 0, 1, 1]]], dtype=np.uint8), 0,
                   False, None, B)
    np.testing.assert_allclose(o1, o2, rtol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)


def test_bsa_empty_row_and_brute_force_tiny():
    B, d = 128, 4
    rng = np.random.default_rng(31)
    q = rng.standard_normal((B, 1, d))
    k = rng.standard_normal((2 * B, 1, d))
    v = rng.standard_normal((2 * B, 1, d))
    out, lse = O.bsa(q, k, v, 2 * B, 0, np.zeros((1, 1, 2), np.uint8), 0, False, None, B)
    assert np.all(out == 0.0) and np.all(lse == -np.inf)
    mask = np.array([[[0, 1]]], dtype=np.uint8)
    out, lse = O.bsa(q, k, v, 2 * B, 0, mask, 0, False, None, B)
    for i in (0, 5, 127):
        ws = [math.exp(sum(q[i, 0, e] * k[j, 0, e] for e in range(d)) / math.sqrt(d))
              for j in range(B, 2 * B)]
        tot = sum(ws)
        assert abs(lse[0, i] - math.log(tot)) < 1e-12
        for e in range(d):
            ref = sum(w * v[B + jj, 0, e] for jj, w in enumerate(ws)) / tot
            assert abs(out[i, 0, e] - ref) < 1e-12


def test_merge_identity_symmetry_and_union():
    rng = np.random.default_rng(40)
    B, d, Lq = 128, 16, 256
    q = rng.standard_normal((Lq, 2, d))
    k = rng.standard_normal((512, 1, d))
    v = rng.standard_normal((512, 1, d))
    mA = (rng.random((2, 2, 4)) < 0.5).astype(np.uint8)
    mA[:, :, 0] = 1
    mB = (1 - mA).astype(np.uint8)
    oa, la = O.bsa(q, k, v, 512, 0, mA, 0, False, None, B)
    ob, lb = O.bsa(q, k, v, 512, 0, mB, 0, False, None, B)
    ou, lu = O.bsa(q, k, v, 512, 0, np.ones_like(mA), 0, False, None, B)
    om, lm = O.merge(oa, la, ob, lb)
    np.testing.assert_allclose(om, ou, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lm, lu, rtol=1e-12)
    om2, lm2 = O.merge(ob, lb, oa, la)
    np.testing.assert_allclose(om2, om, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(lm2, lm)
    empty_o = np.zeros_like(oa)
    empty_l = np.full_like(la, -np.inf)
    o, l = O.merge(oa, la, empty_o, empty_l)
    np.testing.assert_array_equal(o, oa)
    np.testing.assert_array_equal(l, la)
    o, l = O.merge(empty_o, empty_l, empty_o, empty_l)
    assert np.all(o == 0.0) and np.all(l == -np.inf)


def test_chunked_prefill_threshold_one_equals_one_shot():
    rng = np.random.default_rng(50)
    B, d, L, C, S = 128, 16, 768, 256, 8
    q = rng.standard_normal((L, 2, d))
    k = rng.standard_normal((L, 1, d))
    v = rng.standard_normal((L, 1, d))
    r = O.chunked_prefill(q, k, v, C, S, 1.0, B)
    allowed = np.tril(np.ones((L, L), dtype=bool))
    for h in range(2):
        np.testing.assert_allclose(r["out"][:, h], _sdpa(q[:, h], k[:, 0], v[:, 0], allowed),
                                   rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(r["lse"][h], _sdpa_lse(q[:, h], k[:, 0], allowed),
                                   rtol=1e-9, atol=1e-9)
    for i, m in enumerate(r["masks"]):
        assert O.density(m, i * C, B) == 1.0
