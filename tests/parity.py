"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerances (fixed by the requirements of the path, stated once here):
  * block scores: |gpu - oracle| <= 1e-3 * |oracle| + 1e-6 * row_total;
  * block masks: identical, except blocks whose oracle running mass before
    them (always-kept mass first, then the others in descending score
    order) lies within 1e-4 of threshold * row_total, or whose oracle score
    ties (1e-3 relative) with the block at the cut-off;
  * attention out: max |gpu - oracle| <= 2e-2 (bf16 inputs), 2e-3 (fp32 inputs);
  * lse: max |gpu - oracle| <= 1e-3.
"""
from __future__ import annotations

import numpy as np

SCORE_RTOL = 1e-3
SCORE_ATOL_ROW = 1e-6
MASK_MASS_TOL = 1e-4
MASK_TIE_RTOL = 1e-3
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
    """Return (n_diff, n_exempt, list of unexplained (h, qb, kb)) for a mask comparison.

    hist_only: the keys are history only (every block visible, block 0 the only forced block).
    """
    gpu_mask = np.asarray(gpu_mask).astype(bool)
    ref_mask = np.asarray(ref_mask).astype(bool)
    H, nQB, nKB = ref_mask.shape
    diff = np.argwhere(gpu_mask != ref_mask)
    cur = q_start_pos // block
    bad = []
    n_exempt = 0
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
            ok = False
            if kb in excl and abs(excl[kb] / total - threshold) <= MASK_MASS_TOL:
                ok = True
            if kb in excl and any(abs(a[kb] - c) <= MASK_TIE_RTOL * max(abs(c), 1e-30) for c in cut):
                ok = True
            if ok:
                n_exempt += 1
            else:
                bad.append((int(h), int(qb), int(kb)))
    return len(diff), n_exempt, bad


def check_mask(gpu_mask, ref_scores, ref_mask, q_start_pos, threshold, block=128, hist_only=False):
    n_diff, n_exempt, bad = mask_exemptions(gpu_mask, ref_scores, ref_mask, q_start_pos, threshold, block,
                                            hist_only)
    assert not bad, f"{len(bad)} unexplained mask differences (of {n_diff}), first {bad[:5]}"
    return n_diff, n_exempt


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
