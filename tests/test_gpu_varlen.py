"""GPU parity of the packed-batch (varlen) estimate and attention.

* xattn_estimate_varlen: each sequence's scores and mask equal the
  single-sequence xattn_estimate of that sequence bit for bit, and the
  oracle's estimate / selection to the score and mask tolerances;
* bsa_prefill_varlen: each sequence's output and LSE match the oracle's
  causal block-sparse attention with the GPU mask (and, with no mask, dense
  causal attention); the batch includes a sequence with no queries, a
  one-block sequence, chunk-shaped sequences (queries at the end of longer
  keys) whose long rows take the split path, and ragged lengths;
* the 8-sequence workload the benchmark times: sampled (head, query block)
  rows of every sequence against the oracle (its own masks), plus any-size
  properties on every row (block 0 and the diagonal kept, nothing right of
  the diagonal, row sums = block/stride, finite outputs).
"""
import numpy as np
import pytest
import torch

from oracle import xattn_oracle as O
from tests import parity as PAR

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LENS = [(256, 512), (128, 128), (0, 256), (384, 896), (512, 1536), (1024, 8192)]   # (q_len, k_len)


def _np(t):
    return t.detach().float().cpu().double().numpy()


def _batch(lens, seed, hq=4, hkv=2, d=128):
    g = torch.Generator().manual_seed(seed)
    cq = np.cumsum([0] + [a for a, _ in lens]).tolist()
    ck = np.cumsum([0] + [b for _, b in lens]).tolist()
    q = torch.randn(cq[-1], hq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(ck[-1], hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(ck[-1], hkv, d, generator=g).to(torch.bfloat16)
    return q, k, v, cq, ck


# 4 query heads on 2 kv heads (attention in head pairs) and 3 on 1 (one query head per workgroup)
@pytest.fixture(scope="module", params=[(4, 2), (3, 1)], ids=["pairs", "single"])
def small(request):
    from block_sparse_attention_xattn_amd.varlen import VarlenPrefill
    hq, hkv = request.param
    q, k, v, cq, ck = _batch(LENS, 30, hq=hq, hkv=hkv)
    run = VarlenPrefill(q.to(DEV), k.to(DEV), v.to(DEV), cq, ck, 8, 0.9)
    run.run()
    torch.cuda.synchronize()
    return q, k, v, cq, ck, run


def test_estimate_varlen_equals_single_and_oracle(small):
    from block_sparse_attention_xattn_amd import binding as B
    q, k, v, cq, ck, run = small
    for b, (sc, m) in enumerate(zip(run.block_scores(), run.masks())):
        ql, kl = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        if ql == 0:
            assert sc.shape == (q.shape[1], 0, kl // 128)
            continue
        p = kl - ql
        rs, rm = B.xattn_estimate(q[cq[b]:cq[b + 1]].to(DEV), k[ck[b]:ck[b + 1]].to(DEV), p, 8, 0.9)
        assert torch.equal(sc, rs) and torch.equal(m, rm), f"sequence {b}"
        ref_s, ref_m = O.estimate(_np(q[cq[b]:cq[b + 1]]), _np(k[ck[b]:ck[b + 1]]), p, 8, 0.9)
        PAR.check_scores(_np(sc), ref_s)
        PAR.check_mask(m.cpu().numpy(), ref_s, ref_m, p, 0.9)


def test_bsa_varlen_sparse_vs_oracle(small):
    q, k, v, cq, ck, run = small
    lses = run.lses()
    for b, m in enumerate(run.masks()):
        ql, kl = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        if ql == 0:
            continue
        ro, rl = O.bsa(_np(q[cq[b]:cq[b + 1]]), _np(k[ck[b]:ck[b + 1]]), _np(v[ck[b]:ck[b + 1]]), kl - ql, 0,
                       m.cpu().numpy(), 0, True)
        PAR.check_out_lse(_np(run.out[cq[b]:cq[b + 1]]), _np(lses[b]), ro, rl, PAR.OUT_ATOL_BF16)


def test_bsa_varlen_dense_vs_oracle():
    from block_sparse_attention_xattn_amd.varlen import VarlenPrefill
    lens = [(1024, 16384), (256, 256), (128, 4096), (0, 128), (640, 2176)]
    q, k, v, cq, ck = _batch(lens, 31)
    run = VarlenPrefill(q.to(DEV), k.to(DEV), v.to(DEV), cq, ck, 8, 0.9, sparse=False)
    run.run()
    torch.cuda.synchronize()
    lses = run.lses()
    for b in range(len(lens)):
        ql, kl = lens[b]
        if ql == 0:
            continue
        ro, rl = O.bsa(_np(q[cq[b]:cq[b + 1]]), _np(k[ck[b]:ck[b + 1]]), _np(v[ck[b]:ck[b + 1]]), kl - ql, 0,
                       None, 0, True)
        PAR.check_out_lse(_np(run.out[cq[b]:cq[b + 1]]), _np(lses[b]), ro, rl, PAR.OUT_ATOL_BF16)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (3, 1)], ids=["pairs", "single"])
@pytest.mark.parametrize("density", [1.0, 0.6])
def test_bsa_varlen_fp32_out_vs_oracle(hq, hkv, density):
    """fp32 output of the packed-batch attention (head-pair and single-head forms), dense and with a random block
    mask per sequence (rows whose mask keeps nothing visible return zeros and an LSE of -inf)."""
    from block_sparse_attention_xattn_amd import binding as B
    lens = [(512, 4096), (128, 128), (0, 256), (384, 1280)]
    q, k, v, cq, ck = _batch(lens, 32, hq=hq, hkv=hkv)
    qd, kd = q.to(DEV), k.to(DEV)
    packed = B.PackedV(ck[-1], hkv, 128, torch.bfloat16, DEV)
    B.bsa_pack_v(v.to(DEV), packed, 0)
    masks, flat = [], None
    if density < 1.0:
        rng = np.random.default_rng(7)
        masks = [(rng.random((hq, ql // 128, kl // 128)) < density).astype(np.uint8) for ql, kl in lens]
        flat = torch.from_numpy(np.concatenate([m.ravel() for m in masks])).to(DEV)
    out = torch.empty(cq[-1], hq, 128, dtype=torch.float32, device=DEV)
    out, lse = B.bsa_prefill_varlen(qd, kd, packed, cq, ck, flat, out=out)
    torch.cuda.synchronize()
    lses = B.varlen_lse(lse, cq, hq)
    for b, (ql, kl) in enumerate(lens):
        if ql == 0:
            continue
        ro, rl = O.bsa(_np(q[cq[b]:cq[b + 1]]), _np(k[ck[b]:ck[b + 1]]), _np(v[ck[b]:ck[b + 1]]), kl - ql, 0,
                       masks[b] if masks else None, 0, True)
        PAR.check_out_lse(_np(out[cq[b]:cq[b + 1]]), _np(lses[b]), ro, rl, PAR.OUT_ATOL_BF16)


def test_varlen_workload_full_size():
    from block_sparse_attention_xattn_amd import synthetic
    from block_sparse_attention_xattn_amd.varlen import VarlenPrefill
    w = synthetic.WORKLOADS["llama8b_varlen_8seq"]
    print("[varlen] generating the 8-sequence batch", flush=True)
    q, k, v, cu = synthetic.packed_batch(w["lengths"], w["hq"], w["hkv"], w["d"], w["n_needles"], w["seed"])
    S, tau = w["stride"], w["threshold"]
    run = VarlenPrefill(q.to(DEV), k.to(DEV), v.to(DEV), cu, cu, S, tau)
    run.run()
    torch.cuda.synchronize()
    assert torch.isfinite(run.out.float()).all() and torch.isfinite(run.lse).all()
    g = w["hq"] // w["hkv"]
    rng = np.random.default_rng(0)
    scores, masks, lses = run.block_scores(), run.masks(), run.lses()
    checked = 0
    for b, L in enumerate(w["lengths"]):
        sc = scores[b].cpu().numpy()
        m = masks[b].cpu().numpy().astype(bool)
        nqb = L // 128
        np.testing.assert_allclose(sc.sum(axis=2), np.full(sc.shape[:2], 128 // S), rtol=2e-4)
        for qb in range(nqb):
            assert m[:, qb, 0].all() and m[:, qb, qb].all() and not m[:, qb, qb + 1:].any()
        h = int(rng.integers(0, w["hq"]))
        qs, ks = slice(cu[b], cu[b + 1]), slice(cu[b], cu[b + 1])
        ref_s = O.estimate_head(_np(q[qs, h]), _np(k[ks, h // g]), 0, S, 128)[None]
        ref_m = O.select_blocks(ref_s, 0, tau, 128)
        PAR.check_scores(sc[h:h + 1], ref_s)
        PAR.check_mask(m[h:h + 1], ref_s, ref_m, 0, tau, label=f"sequence {b} head {h}")
        for qb in sorted({0, nqb // 2, nqb - 1}):
            # the GPU's own mask row (equal to the oracle's up to exempt flips) decides which blocks are attended
            rows = slice(qb * 128, (qb + 1) * 128)
            ro, rl = O.bsa(_np(q[qs][rows, h:h + 1]), _np(k[ks, h // g:h // g + 1]), _np(v[ks, h // g:h // g + 1]),
                           qb * 128, 0, m[h:h + 1, qb:qb + 1].astype(np.uint8), 0, True)
            PAR.check_out_lse(_np(run.out[qs][rows, h:h + 1]), _np(lses[b][h:h + 1, rows]), ro, rl,
                              PAR.OUT_ATOL_BF16)
            checked += 1
    assert checked == sum(len({0, L // 256, L // 128 - 1}) for L in w["lengths"])
