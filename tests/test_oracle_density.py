"""Pins of the density counts (compute density and comm density).

XAttentionBSAPolicy ``select_blocks`` step 5 (selected ∩ causal over the
causal count) and the comm density recorded after step 6 (kept cache blocks
over the history's cache blocks).  Pinned by brute-force loops over every
(head, query block, key block), by threshold 1 (every causal block kept, so
selected == total) and by the monotone growth of density with the threshold.
"""
import numpy as np
import pytest

from oracle import xattn_oracle as O


@pytest.mark.parametrize("seed,H,nQB,nKB", [(0, 2, 4, 4), (1, 3, 4, 9), (2, 1, 1, 1), (3, 4, 8, 40)])
def test_density_counts_brute_force(seed, H, nQB, nKB):
    rng = np.random.default_rng(seed)
    mask = (rng.random((H, nQB, nKB)) < 0.4).astype(np.uint8)
    sel = tot = 0
    for h in range(H):
        for qb in range(nQB):
            # the chunk's queries are the last nQB blocks: query block qb sits at global block nKB - nQB + qb
            last = nKB - nQB + qb
            for kb in range(nKB):
                if kb <= last:
                    tot += 1
                    sel += int(mask[h, qb, kb] != 0)
    assert O.density_counts(mask) == (sel, tot)
    s, t = O.density_counts(mask)
    assert O.density(mask, (nKB - nQB) * 128) == s / t


def test_density_counts_threshold_one_and_monotone():
    rng = np.random.default_rng(7)
    H, nQB, nKB = 3, 4, 12
    p = (nKB - nQB) * 128
    raw = rng.random((H, nQB, nKB)) ** 4
    scores = raw / raw.sum(axis=2, keepdims=True)
    prev = -1
    for tau in (0.0, 0.5, 0.8, 0.9, 0.95, 0.99, 1.0):
        m = O.select_blocks(scores, p, tau)
        s, t = O.density_counts(m)
        assert t == H * sum(nKB - nQB + qb + 1 for qb in range(nQB))
        assert s >= prev
        prev = s
        if tau >= 1.0:
            assert s == t
        if tau == 0.0:
            # only block 0 and the diagonal survive (2 per row; one where they coincide)
            assert s == H * sum(len({0, nKB - nQB + qb}) for qb in range(nQB))


def test_comm_density_counts():
    keep = np.array([1, 0, 0, 1, 1, 0, 1], dtype=np.uint8)
    assert O.comm_density_counts(keep) == (4, 7)
    mask = np.zeros((2, 3, 24), dtype=np.uint8)
    mask[1, 2, 9] = 1                      # one 128-token block in cache block 1
    _, anyk = O.mask_to_cache_blocks(mask, 0, 3, 8, True)
    assert O.comm_density_counts(anyk) == (3, 3)   # first and last forced, block 1 selected
    _, anyk = O.mask_to_cache_blocks(mask, 0, 3, 8, False)
    assert O.comm_density_counts(anyk) == (1, 3)
    assert O.comm_density_counts(np.zeros(0, dtype=np.uint8)) == (0, 0)
