"""GPU parity at full workload sizes, in the launch configuration bench.py times.

Each test runs the chunked-prefill runner (the same calls the bench times) on a
full-size synthetic layer and checks
  * sampled heads / query blocks against the float64 oracle (scores 1e-3
    relative, masks with the threshold exemptions, attention out 2e-2 max-abs,
    LSE 1e-3), the oracle using its own masks;
  * properties that hold at any size on every row: each query block's scores
    sum to block/stride, nothing right of the diagonal is kept or scored,
    block 0 and the diagonal are kept, outputs and LSE are finite, and (for
    the cache-block form) the reducer output is the OR of the GPU mask.
"""
import numpy as np
import pytest
import torch

from oracle import xattn_oracle as O
from tests import parity as PAR

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
B = 128


def _f64(t):
    return t.detach().float().cpu().double().numpy()


def _run(name, L=None, chunk_starts=None, cache_block=None, threshold=None, stride=None):
    from block_sparse_attention_xattn_amd import synthetic
    from block_sparse_attention_xattn_amd.prefill import ChunkedPrefill
    w = synthetic.WORKLOADS[name]
    print(f"[full-size] {name}: generating inputs", flush=True)
    q, k, v = synthetic.workload_inputs(name, L)
    tau = w["threshold"] if threshold is None else threshold
    S = w["stride"] if stride is None else stride
    run = ChunkedPrefill(q.to(DEV), k.to(DEV), v.to(DEV), chunk=w["chunk"], stride=S, threshold=tau,
                         chunk_starts=chunk_starts, cache_block=cache_block)
    print(f"[full-size] {name}: running {len(run.starts)} chunk(s) on the GPU", flush=True)
    run.run()
    torch.cuda.synchronize()
    return w, q, k, v, run, tau, S


def _invariants(run, S):
    for b in run.bufs:
        sc = b.scores.cpu().numpy()
        m = b.mask.cpu().numpy().astype(bool)
        hq, nqb, nkb = m.shape
        cur = b.p // B
        np.testing.assert_allclose(sc.sum(axis=2), np.full((hq, nqb), B // S), rtol=2e-4)
        for qb in range(nqb):
            d = cur + qb
            assert m[:, qb, 0].all() and m[:, qb, d].all()
            assert not m[:, qb, d + 1:].any()
            assert (sc[:, qb, d + 1:] == 0).all()
        assert torch.isfinite(b.lse).all()
    assert torch.isfinite(run.out.float()).all()


def _check_head_chunk(q, k, v, run, i, h, g, S, tau, qbs):
    """Oracle estimate for one head of chunk i; attention for query blocks qbs."""
    b = run.bufs[i]
    p = b.p
    c = b.scores.shape[1] * B
    qh = _f64(q[p:p + c, h])
    kh = _f64(k[:p + c, h // g])
    ref_s = O.estimate_head(qh, kh, p, S, B)[None]
    ref_m = O.select_blocks(ref_s, p, tau, B)
    PAR.check_scores(b.scores[h:h + 1].cpu().numpy(), ref_s)
    n_diff, _ = PAR.check_mask(b.mask[h:h + 1].cpu().numpy(), ref_s, ref_m, p, tau)
    gm = b.mask[h].cpu().numpy().astype(bool)
    checked = 0
    for qb in qbs:
        if not np.array_equal(gm[qb], ref_m[0, qb].astype(bool)):
            continue  # an exempt flip changes the kept set of this row
        rows = slice(p + qb * B, p + (qb + 1) * B)
        ro, rl = O.bsa(_f64(q[rows, h:h + 1]), _f64(k[:p + c, h // g:h // g + 1]),
                       _f64(v[:p + c, h // g:h // g + 1]), p + qb * B, 0, ref_m[:, qb:qb + 1], 0, True)
        go = _f64(run.out[rows, h:h + 1])
        gl = _f64(b.lse[h:h + 1, qb * B:(qb + 1) * B])
        PAR.check_out_lse(go, gl, ro, rl, PAR.OUT_ATOL_BF16)
        checked += 1
    return n_diff, checked


def test_llama8b_32k_8x4k():
    w, q, k, v, run, tau, S = _run("llama8b_32k_8x4k")
    _invariants(run, S)
    g = w["hq"] // w["hkv"]
    checked = 0
    for i, h in [(0, 0), (3, 13), (7, 31)]:
        print(f"[full-size] chunk {i} head {h}: oracle estimate + attention", flush=True)
        _, c = _check_head_chunk(q, k, v, run, i, h, g, S, tau, [0, 17, 31])
        checked += c
    assert checked >= 6


def _cache_block_checks(w, q, k, v, run, tau, S, heads_for_oracle, attn_samples, all_heads):
    b = run.bufs[0]
    p = b.p
    g = w["hq"] // w["hkv"]
    sub = 1024 // B
    ncb = p // 1024
    # reducer output is the OR of the GPU's own mask (bit-exact), first/last forced
    gm = b.mask.cpu().numpy().astype(bool)
    hist = gm[:, :, :ncb * sub].reshape(gm.shape[0], gm.shape[1], ncb, sub).any(axis=3)
    assert np.array_equal(b.keep_per_head.cpu().numpy().astype(bool), hist)
    anyk = hist.any(axis=(0, 1))
    anyk[0] = anyk[-1] = True
    assert np.array_equal(b.keep_any.cpu().numpy().astype(bool), anyk)
    assert np.array_equal(b.keep_any_blocks.cpu().numpy().astype(bool), np.repeat(anyk, sub))
    print(f"[full-size] cache blocks: oracle estimate for {len(heads_for_oracle)} head(s)", flush=True)
    ref_s = np.stack([O.estimate_head(_f64(q[p:, h]), _f64(k[:, h // g]), p, S, B) for h in heads_for_oracle])
    ref_m = O.select_blocks(ref_s, p, tau, B)
    PAR.check_scores(b.scores[heads_for_oracle].cpu().numpy(), ref_s)
    PAR.check_mask(b.mask[heads_for_oracle].cpu().numpy(), ref_s, ref_m, p, tau)
    if not all_heads:
        return
    # the union keep list needs every head: oracle keep list, then attention with it
    _, ref_any = O.mask_to_cache_blocks(ref_m, 0, ncb, sub, True)
    assert np.array_equal(b.keep_any.cpu().numpy(), ref_any), "cache-block keep list differs from the oracle's"
    keep = O.expand_cache_keep(ref_any, sub, ncb * sub)
    for h, qb in attn_samples:
        rows = slice(p + qb * B, p + (qb + 1) * B)
        kvh = h // g
        o1, l1 = O.bsa(_f64(q[rows, h:h + 1]), _f64(k[:p, kvh:kvh + 1]), _f64(v[:p, kvh:kvh + 1]),
                       p + qb * B, 0, keep[None, None, :], 0, False)
        o2, l2 = O.bsa(_f64(q[rows, h:h + 1]), _f64(k[p:, kvh:kvh + 1]), _f64(v[p:, kvh:kvh + 1]),
                       p + qb * B, p, None, 0, True)
        ro, rl = O.merge(o1, l1, o2, l2)
        PAR.check_out_lse(_f64(run.out[rows, h:h + 1]), _f64(b.lse[h:h + 1, qb * B:(qb + 1) * B]), ro, rl,
                          PAR.OUT_ATOL_BF16)


def test_llama8b_128k_last_chunk_cache_blocks():
    """Full size (131072 keys, chunk at 126976): invariants, reducer = OR of the mask, two heads vs the oracle."""
    w, q, k, v, run, tau, S = _run("llama8b_128k_last_chunk", chunk_starts=[126976], cache_block=1024)
    _invariants(run, S)
    _cache_block_checks(w, q, k, v, run, tau, S, [0, 21], [], all_heads=False)


def test_llama8b_cache_blocks_16k_all_heads():
    """Same generator and launch form at 16384 keys (chunk at 12288): union keep list and attention vs oracle."""
    w, q, k, v, run, tau, S = _run("llama8b_128k_last_chunk", L=16384, chunk_starts=[12288], cache_block=1024)
    _invariants(run, S)
    _cache_block_checks(w, q, k, v, run, tau, S, list(range(w["hq"])), [(5, 0), (30, 31), (17, 12)],
                        all_heads=True)


def test_llama8b_64k_threshold_one_is_dense():
    w, q, k, v, run, tau, S = _run("llama8b_64k_sweep", threshold=1.0, stride=8,
                                   chunk_starts=[61440])
    _invariants(run, S)
    b = run.bufs[0]
    p = b.p
    m = b.mask.cpu().numpy().astype(bool)
    nqb, nkb = m.shape[1], m.shape[2]
    causal = np.arange(nkb)[None, :] <= (p // B + np.arange(nqb))[:, None]
    assert np.array_equal(m, np.broadcast_to(causal, m.shape))
    g = w["hq"] // w["hkv"]
    for h, qb in [(0, 0), (19, 31)]:
        rows = slice(p + qb * B, p + (qb + 1) * B)
        ro, rl = O.bsa(_f64(q[rows, h:h + 1]), _f64(k[:, h // g:h // g + 1]), _f64(v[:, h // g:h // g + 1]),
                       p + qb * B, 0, None, 0, True)
        PAR.check_out_lse(_f64(run.out[rows, h:h + 1]), _f64(b.lse[h:h + 1, qb * B:(qb + 1) * B]), ro, rl,
                          PAR.OUT_ATOL_BF16)


@pytest.mark.parametrize("stride", [8, 16])
def test_llama8b_64k_sweep_strides(stride):
    w, q, k, v, run, tau, S = _run("llama8b_64k_sweep", threshold=0.9, stride=stride,
                                   chunk_starts=[0, 28672, 61440])
    _invariants(run, S)
    g = w["hq"] // w["hkv"]
    for i, h in [(1, 7), (2, 26)]:
        _check_head_chunk(q, k, v, run, i, h, g, S, 0.9, [3, 30])


def test_gqa7_128k_32x4k():
    w, q, k, v, run, tau, S = _run("gqa7_128k_32x4k")
    _invariants(run, S)
    g = w["hq"] // w["hkv"]
    for i, h in [(0, 6), (16, 13), (31, 27)]:
        print(f"[full-size] gqa7 chunk {i} head {h}", flush=True)
        _check_head_chunk(q, k, v, run, i, h, g, S, tau, [31])
