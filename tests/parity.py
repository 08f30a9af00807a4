"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerances (fixed by the requirements of the path, stated once here):
  * block scores: |gpu - oracle| <= 1e-3 * |oracle| + 1e-6 * row_total;
  * block masks: identical, except blocks whose oracle running mass before
    them (always-kept mass first, then the others in descending score
    order) lies within 1e-4 of threshold * row_total ("mass" exemptions), or
    whose oracle score ties with the block at the cut-off within twice the
    score tolerance, so that the two may swap places in the ranking ("tie"
    exemptions); every comparison reports both counts, and together they may
    cover at most 1e-3 of the causal blocks compared (at least 2 allowed);
  * attention out: max |gpu - oracle| <= 2e-2 (bf16 inputs), 2e-3 (fp32 inputs);
  * lse: max |gpu - oracle| <= 1e-3.
"""
from __future__ import annotations

import numpy as np

SCORE_RTOL = 1e-3
SCORE_ATOL_ROW = 1e-6
MASK_MASS_TOL = 1e-4
MASK_TIE_RTOL = 2 * SCORE_RTOL
MASK_EXEMPT_FRAC = 1e-3
OUT_ATOL_BF16 = 2e-2
OUT_ATOL_F32 = 2e-3
LSE_ATOL = 1e-3


def check_scores(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    row_total = ref.sum(axis=-1, keepdims=True)
    err = np.abs(gpu - ref)
    bound = SCORE_RTOL * np.abs(ref) + SCORE_ATOL_ROW * row_total
    bad = err > bound
    assert not bad.any(), (f"{int(bad.sum())} block scores outside tolerance; worst rel "
                           f"{float((err / (np.abs(ref) + 1e-30)).max()):.3e}")


def mask_exemptions(gpu_mask, ref_scores, ref_mask, q_start_pos, threshold, block=128, hist_only=False):
    """Return (n_diff, n_exempt, list of unexplained (h, qb, kb), counts by kind) for a mask comparison.

    hist_only: the keys are history only (every block visible, block 0 the only forced block).
    """
    gpu_mask = np.asarray(gpu_mask).astype(bool)
    ref_mask = np.asarray(ref_mask).astype(bool)
    H, nQB, nKB = ref_mask.shape
    diff = np.argwhere(gpu_mask != ref_mask)
    cur = q_start_pos // block
    bad = []
    n_exempt = 0
    kinds = {"mass": 0, "tie": 0}
    rows = {}
    for h, qb, kb in diff:
        rows.setdefault((h, qb), []).append(kb)
    for (h, qb), kbs in rows.items():
        diag = nKB - 1 if hist_only else cur + qb
        a = ref_scores[h, qb, :diag + 1].astype(np.float64)
        total = a.sum()
        forced = {0} if hist_only else {0, diag}
        others = sorted((i for i in range(diag + 1) if i not in forced), key=lambda i: (-a[i], i))
        run = sum(a[i] for i in forced)
        excl = {}
        for i in others:
            excl[i] = run
            run += a[i]
        kept = [i for i in others if ref_mask[h, qb, i]]
        cut = []
        if kept:
            cut.append(a[kept[-1]])
        nxt = [i for i in others if not ref_mask[h, qb, i]]
        if nxt:
            cut.append(a[nxt[0]])
        for kb in kbs:
            kind = None
            if kb in excl and abs(excl[kb] / total - threshold) <= MASK_MASS_TOL:
                kind = "mass"
            elif kb in excl and any(abs(a[kb] - c) <= MASK_TIE_RTOL * abs(c) + 2 * SCORE_ATOL_ROW * total
                                    for c in cut):
                kind = "tie"
            if kind:
                n_exempt += 1
                kinds[kind] += 1
            else:
                bad.append((int(h), int(qb), int(kb)))
    return len(diff), n_exempt, bad, kinds


def _causal_blocks(shape, q_start_pos, block, hist_only):
    H, nQB, nKB = shape
    if hist_only:
        return H * nQB * nKB
    cur = q_start_pos // block
    return H * sum(min(cur + qb, nKB - 1) + 1 for qb in range(nQB))


def check_mask(gpu_mask, ref_scores, ref_mask, q_start_pos, threshold, block=128, hist_only=False, label=""):
    """Assert the mask comparison and print its exemption counts.  Returns (n_diff, n_exempt)."""
    n_diff, n_exempt, bad, kinds = mask_exemptions(gpu_mask, ref_scores, ref_mask, q_start_pos, threshold, block,
                                                   hist_only)
    assert not bad, f"{len(bad)} unexplained mask differences (of {n_diff}), first {bad[:5]}"
    n_blocks = _causal_blocks(np.asarray(ref_mask).shape, q_start_pos, block, hist_only)
    print(f"[mask{(' ' + label) if label else ''}] {n_blocks} causal blocks, {n_diff} differ: "
          f"{kinds['mass']} mass exemptions, {kinds['tie']} tie exemptions", flush=True)
    limit = max(2, int(MASK_EXEMPT_FRAC * n_blocks))
    assert n_exempt <= limit, f"{n_exempt} exempt mask differences exceed the bound {limit} of {n_blocks} blocks"
    return n_diff, n_exempt


def oracle_chunk_attention(O, q, k, v, q_start, hist_end, mask, cur_mask="mask"):
    """The oracle's attention of query rows at global positions q_start .. q_start + len(q) - 1 (whole query
    blocks of one chunk, all of q's heads) with a GIVEN block mask [H, rows/128, nKB] (columns = key blocks from
    0): the history keys [0, hist_end) without the causal rule and the chunk's own keys [hist_end, len(k)) with
    it, merged by LSE (XAttentionBSAPolicy.compute_chunked_prefill).  cur_mask="dense" attends the chunk's own
    keys densely (the cache-block form; mask then covers the history columns only).  Arrays float64; k / v hold
    the query heads' kv heads [keys, Hkv, d]."""
    o_c, l_c = O.bsa(q, k[hist_end:], v[hist_end:], q_start, hist_end, None if cur_mask == "dense" else mask, 0,
                     True)
    if hist_end == 0:
        return o_c, l_c
    o_h, l_h = O.bsa(q, k[:hist_end], v[:hist_end], q_start, 0, mask, 0, False)
    return O.merge(o_h, l_h, o_c, l_c)


def check_out_lse(out_gpu, lse_gpu, out_ref, lse_ref, atol_out):
    out_gpu = np.asarray(out_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), "empty-row pattern differs"
    if fin.any():
        dl = np.abs(lse_gpu[fin] - lse_ref[fin]).max()
        assert dl <= LSE_ATOL, f"lse max abs err {dl:.3e}"
    do = np.abs(out_gpu - out_ref).max() if out_ref.size else 0.0
    assert do <= atol_out, f"out max abs err {do:.3e}"
    return float(do)
