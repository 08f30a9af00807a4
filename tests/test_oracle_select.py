"""Pins of the oracle's cumulative-threshold selection.

* the page's worked example (tests/golden/worked_example_selection.json);
* brute force: the greedy rule keeps a smallest set that contains the
  always-kept blocks and holds at least threshold * total mass, and that set
  is those blocks plus the highest-scoring others;
* invariants: block 0 and the diagonal are always kept, nothing right of
  the diagonal is kept, density never falls as the threshold rises, and
  threshold 1 keeps every causal block.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import xattn_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example():
    g = json.load(open(os.path.join(GOLD, "worked_example_selection.json")))
    row = np.array(g["row"])
    keep = O.select_row(row, forced=[], threshold=g["threshold"])
    assert sorted(np.nonzero(keep)[0].tolist()) == sorted(g["selected_indices_in_order"])
    # the order the page lists them in is descending score order
    order = sorted(np.nonzero(keep)[0].tolist(), key=lambda i: -row[i])
    assert order == g["selected_indices_in_order"]
    np.testing.assert_allclose(np.cumsum(np.sort(row)[::-1]), g["running_sums"], atol=1e-12)


def test_literal_pseudocode_differs_on_worked_example():
    # The printed pseudo-code compares the inclusive running sum with '<',
    # which would stop one block earlier than the page's own example.
    g = json.load(open(os.path.join(GOLD, "worked_example_selection.json")))
    keep = O.select_row(np.array(g["row"]), forced=[], threshold=g["threshold"], rule="literal")
    assert sorted(np.nonzero(keep)[0].tolist()) == [1, 2, 3]


def _brute_min_sets(row, forced, tau):
    n = len(row)
    need = tau * row.sum()
    others = [i for i in range(n) if i not in forced]
    for extra in range(len(others) + 1):
        sets = [set(forced) | set(c) for c in itertools.combinations(others, extra)
                if row[list(set(forced) | set(c))].sum() >= need - 1e-15]
        if sets:
            return extra, sets
    raise AssertionError


@pytest.mark.parametrize("seed", range(40))
def test_greedy_is_minimal_cover(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 10))
    row = rng.exponential(size=n) ** 2
    if seed % 5 == 0:                       # include exact ties
        row[: n // 2] = row[0]
    diag = n - 1
    forced = sorted({0, diag})
    tau = float(rng.choice([0.5, 0.8, 0.9, 0.95, 0.99]))
    keep = O.select_row(row, forced, tau)
    extra, sets = _brute_min_sets(row, forced, tau)
    assert keep.sum() == len(forced) + extra or (keep.sum() == len(forced) and extra == 0)
    assert set(np.nonzero(keep)[0].tolist()) in [set(s) for s in sets]
    assert row[keep].sum() >= tau * row.sum() - 1e-12
    # kept non-forced blocks are the top-scoring ones (ties by lower index)
    others = [i for i in range(n) if i not in forced]
    ranked = sorted(others, key=lambda i: (-row[i], i))
    kept_others = [i for i in ranked if keep[i]]
    assert kept_others == ranked[:len(kept_others)]


def test_forced_mass_alone_can_satisfy():
    row = np.array([0.72, 0.03, 0.05, 0.2])      # forced {0, 3} already hold 0.92
    keep = O.select_row(row, [0, 3], 0.9)
    assert keep.tolist() == [True, False, False, True]


def _scores(seed, H=2, nQB=4, cur=3):
    rng = np.random.default_rng(seed)
    A = rng.exponential(size=(H, nQB, cur + nQB))
    for qb in range(nQB):
        A[:, qb, cur + qb + 1:] = 0.0
    return A


@pytest.mark.parametrize("seed", range(5))
def test_mask_invariants_and_monotone_density(seed):
    B = 128
    A = _scores(seed)
    p = 3 * B
    prev = None
    for tau in (0.0, 0.3, 0.5, 0.8, 0.9, 0.95, 0.99, 1.0):
        m = O.select_blocks(A, p, tau, B)
        H, nQB, nKB = m.shape
        for qb in range(nQB):
            diag = 3 + qb
            assert np.all(m[:, qb, 0] == 1) and np.all(m[:, qb, diag] == 1)
            assert np.all(m[:, qb, diag + 1:] == 0)
        if prev is not None:
            assert np.all(m >= prev)             # kept sets only grow with the threshold
        prev = m
    causal = np.arange(prev.shape[2])[None, :] <= (3 + np.arange(prev.shape[1]))[:, None]
    assert np.array_equal(prev.astype(bool), np.broadcast_to(causal, prev.shape))
    assert O.density(prev, p, B) == 1.0
