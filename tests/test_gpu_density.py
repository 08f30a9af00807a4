"""GPU density counts (xattn_density_counts) against the oracle.

XAttentionBSAPolicy.select_blocks step 5 (compute density: kept causal
(head, query block, key block) pairs over causal pairs) and the comm density
after step 6 (kept cache blocks over the history's cache blocks).  Integer
counts, compared exactly.
"""
import numpy as np
import pytest
import torch

from oracle import xattn_oracle as O
from tests import parity as PAR

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return t.detach().float().cpu().double().numpy()


def test_density_small_chunked_prefill_vs_oracle():
    """8K tokens in chunks of 2048 (8 query / 2 kv heads): the accumulated counts equal the oracle's counts of
    the GPU masks exactly, and the oracle's counts of its own masks up to the bounded exempt flips."""
    from block_sparse_attention_xattn_amd import synthetic
    from block_sparse_attention_xattn_amd.prefill import ChunkedPrefill
    q, k, v = synthetic.long_context(8192, 8, 2, 128, n_needles=4, seed=21)
    run = ChunkedPrefill(q.to(DEV), k.to(DEV), v.to(DEV), chunk=2048, stride=8, threshold=0.9)
    run.track_density = True
    run.run()
    torch.cuda.synchronize()
    got = run.density()
    sel = tot = kept = avail = 0
    ref_sel = 0
    n_exempt = 0
    qn, kn = _np(q), _np(k)
    for b in run.bufs:
        m = b.mask.cpu().numpy()
        s, t = O.density_counts(m)
        sel, tot = sel + s, tot + t
        ncb = b.p // 1024
        if ncb:
            _, anyk = O.mask_to_cache_blocks(m, 0, ncb, 8, True)
            k_, a_ = O.comm_density_counts(anyk)
            kept, avail = kept + k_, avail + a_
        rs, rm = O.estimate(qn[b.p:b.p + 2048], kn[:b.p + 2048], b.p, 8, 0.9)
        _, ne = PAR.check_mask(m, rs, rm, b.p, 0.9, label=f"chunk at {b.p}")
        n_exempt += ne
        ref_sel += O.density_counts(rm)[0]
    assert (got["selected"], got["causal"]) == (sel, tot)
    assert (got["kept_cache_blocks"], got["cache_blocks"]) == (kept, avail)
    assert avail == sum(p // 1024 for p in run.starts)
    assert abs(got["selected"] - ref_sel) <= n_exempt
    assert 0.0 < got["density"] <= 1.0


@pytest.mark.parametrize("diag0,keep,shape", [(5, True, (3, 6, 13)), (0, False, (3, 6, 13)),
                                              (-3, True, (3, 6, 13)), (40, True, (3, 6, 13)),
                                              (7, None, (3, 6, 13)), (250, True, (40, 64, 300))])
def test_density_counts_abi_edges(diag0, keep, shape):
    """Strided mask views, diagonals before / past the mask, no keep list, accumulation over two calls, and
    more rows than the grid holds waves (each wave takes several rows, each lane several columns)."""
    from block_sparse_attention_xattn_amd import binding as B
    rng = np.random.default_rng(diag0 + 10)
    H, nqb, ncols = shape
    full = (rng.random((H, nqb, ncols + 4)) < 0.5).astype(np.uint8)
    view = torch.from_numpy(full).to(DEV)[:, :, 2:2 + ncols]      # row stride ncols + 4, column offset 2
    m = full[:, :, 2:2 + ncols]
    kany = None if keep is None else (rng.random(9) < (0.5 if keep else 0.0)).astype(np.uint8)
    counts = torch.zeros(4, dtype=torch.int64, device=DEV)
    for _ in range(2):
        B.xattn_density_counts(counts, view, diag0, None if kany is None else torch.from_numpy(kany).to(DEV))
    torch.cuda.synchronize()
    # closed forms: row qb's causal columns are 0 .. min(diag0 + qb, ncols - 1)
    last = np.minimum(diag0 + np.arange(nqb), ncols - 1)
    sel = sum(int(m[h, qb, :last[qb] + 1].sum()) for h in range(H) for qb in range(nqb) if last[qb] >= 0)
    tot = H * int(sum(max(x + 1, 0) for x in last))
    want = [2 * sel, 2 * tot, 0 if kany is None else 2 * int(kany.sum()), 0 if kany is None else 2 * kany.size]
    assert counts.cpu().tolist() == want
    if diag0 == ncols - nqb:
        assert O.density_counts(m) == (sel, tot)


def test_density_counts_keep_only_and_errors():
    from block_sparse_attention_xattn_amd import binding as B
    counts = torch.zeros(4, dtype=torch.int64, device=DEV)
    kany = torch.tensor([1, 0, 1, 1, 0], dtype=torch.uint8, device=DEV)
    B.xattn_density_counts(counts, None, 0, kany)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0, 0, 3, 5]
    with pytest.raises(B.XattnError):
        B.xattn_density_counts(counts.to(torch.int32), None, 0, kany)
    with pytest.raises(B.XattnError):
        B.xattn_density_counts(counts[1:], None, 0, kany)
