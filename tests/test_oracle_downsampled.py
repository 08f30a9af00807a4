"""Pins of the oracle's estimate against downsampled history keys.

* downsampling keeps key tokens 0, S, 2S, ... (index arithmetic, not slicing);
* the block scores are block sums of exact (non-causal) attention
  probabilities of the query tokens over the downsampled keys, obtained from
  torch's scaled_dot_product_attention with block-indicator values (a library
  routine, not the oracle's formula), at strides 1, 4 and 8;
* invariants: each query block's scores sum to its block/stride rows;
  block 0 is kept even when it carries no mass; threshold 1 keeps every
  block; threshold 0 keeps block 0 only; the kept set is the smallest set
  holding block 0 that reaches the threshold mass (brute force);
* the cache-block union is the OR over heads, query blocks and the eight
  128-token blocks of each cache block (brute-force loops).
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import xattn_oracle as O


def _sdpa_block_sums(q, k_ds, b):
    """[Hq, Lq/b, n_ds/b] block sums of softmax(q k^T / sqrt(d)) via SDPA."""
    Lq, Hq, d = q.shape
    n_ds, Hkv, _ = k_ds.shape
    g = Hq // Hkv
    ind = torch.zeros(n_ds, n_ds // b, dtype=torch.float64)
    ind[torch.arange(n_ds), torch.arange(n_ds) // b] = 1.0
    out = []
    for h in range(Hq):
        qt = torch.from_numpy(q[:, h])[None, None]
        kt = torch.from_numpy(k_ds[:, h // g])[None, None]
        p = torch.nn.functional.scaled_dot_product_attention(qt, kt, ind[None, None])[0, 0].numpy()
        out.append(p.reshape(Lq // b, b, n_ds // b).sum(axis=1))
    return np.stack(out)


def test_downsample_keeps_every_stride_th_token():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((100, 2, 8))
    for S in (1, 3, 8):
        ds = O.downsample_keys(k, S)
        idx = [t for t in range(100) if t % S == 0]
        assert ds.shape[0] == len(idx)
        for j, t in enumerate(idx):
            np.testing.assert_array_equal(ds[j], k[t])


@pytest.mark.parametrize("S", [1, 4, 8])
def test_scores_are_block_sums_of_exact_attention(S):
    rng = np.random.default_rng(S)
    b = 128 // S
    q = rng.standard_normal((2 * b, 4, 32))
    k = rng.standard_normal((3 * 128, 2, 32))   # three 128-token history blocks
    k_ds = O.downsample_keys(k, S)
    scores, mask = O.estimate_history_downsampled(q, k_ds, S, 0.9)
    ref = _sdpa_block_sums(q, k_ds, b)
    assert scores.shape == (4, 2, 3)
    np.testing.assert_allclose(scores, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(scores.sum(axis=2), np.full((4, 2), b), rtol=1e-12)


def test_sink_forced_and_threshold_extremes():
    rng = np.random.default_rng(3)
    u = np.zeros(16)
    u[0] = 1.0
    q = 8.0 * u + 0.1 * rng.standard_normal((16, 2, 16))    # every query along u
    k_ds = rng.standard_normal((64, 1, 16))
    k_ds[:16] = -8.0 * u                                    # block 0: keys opposite to every query
    s, m = O.estimate_history_downsampled(q, k_ds, 8, 0.5)
    assert (s[:, :, 0] < 1e-3 * s.sum(axis=2)).all()
    assert m[:, :, 0].all()
    _, m1 = O.estimate_history_downsampled(q, k_ds, 8, 1.0)
    assert m1.all()
    _, m0 = O.estimate_history_downsampled(q, k_ds, 8, 0.0)
    assert m0[:, :, 0].all() and not m0[:, :, 1:].any()


def test_selection_is_minimal_cover_with_block_zero():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((16, 1, 16)) * 2.0
    k_ds = rng.standard_normal((112, 1, 16)) * 2.0   # 7 blocks of 16 downsampled keys
    for tau in (0.3, 0.6, 0.9):
        s, m = O.estimate_history_downsampled(q, k_ds, 8, tau)
        row, keep = s[0, 0], m[0, 0].astype(bool)
        need = tau * row.sum()
        best = None
        for r in range(0, 7):
            for sub in itertools.combinations(range(1, 7), r):
                if row[0] + row[list(sub)].sum() >= need:
                    best = r + 1
                    break
            if best is not None:
                break
        assert keep[0] and keep.sum() == best


def test_cache_block_union_brute_force():
    rng = np.random.default_rng(5)
    mask = (rng.random((3, 4, 20)) < 0.08).astype(np.uint8)
    keep = O.history_cache_blocks_downsampled(mask, 3)
    for cb in range(3):
        want = any(mask[h, qb, c] for h in range(3) for qb in range(4) for c in range(8 * cb, min(8 * cb + 8, 20)))
        assert bool(keep[cb]) == want
