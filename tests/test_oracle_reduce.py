"""Pin of the 128-token -> cache-block reducer by brute-force loops."""
import numpy as np
import pytest

from oracle import xattn_oracle as O


@pytest.mark.parametrize("seed,nCols,kb_begin,sub,force", [
    (0, 32, 0, 8, True), (1, 31, 0, 8, True), (2, 40, 4, 8, False), (3, 17, 1, 4, True),
    (4, 8, 0, 8, False)])
def test_reducer_brute_force(seed, nCols, kb_begin, sub, force):
    rng = np.random.default_rng(seed)
    H, nQB = 3, 5
    mask = (rng.random((H, nQB, nCols)) < 0.08).astype(np.uint8)
    nCB = (nCols - kb_begin + sub - 1) // sub
    per, anyk = O.mask_to_cache_blocks(mask, kb_begin, nCB, sub, force)
    for h in range(H):
        for qb in range(nQB):
            for cb in range(nCB):
                hit = 0
                for s in range(sub):
                    col = kb_begin + cb * sub + s
                    if col < nCols and mask[h, qb, col]:
                        hit = 1
                assert per[h, qb, cb] == hit
    for cb in range(nCB):
        hit = 0
        for h in range(H):
            for qb in range(nQB):
                hit |= int(per[h, qb, cb])
        if force and cb in (0, nCB - 1):
            hit = 1
        assert anyk[cb] == hit
    exp = O.expand_cache_keep(anyk, sub, nCB * sub)
    for kb in range(nCB * sub):
        assert exp[kb] == anyk[kb // sub]
