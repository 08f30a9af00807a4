"""GPU parity at full workload sizes, in the launch configuration bench.py times.

Each test runs the chunked-prefill runner (the same calls the bench times) on a
full-size synthetic layer and checks
  * sampled heads / query blocks against the float64 oracle: scores 1e-3
    relative, masks with the threshold exemptions (counted and bounded), and
    attention out 2e-2 max-abs / LSE 1e-3 on every sampled row -- the oracle
    attends with the GPU's own mask row, which equals the oracle's up to the
    exempt flips, so no row is ever skipped;
  * properties that hold at any size on every row: each query block's scores
    sum to block/stride, nothing right of the diagonal is kept or scored,
    block 0 and the diagonal are kept, outputs and LSE are finite, and (for
    the cache-block form) the reducer output is the OR of the GPU mask;
  * the density counts of the whole run against the oracle's counts of the
    GPU's masks (integers, exact).
"""
import functools

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


@functools.lru_cache(maxsize=2)
def _inputs(name, L):
    from block_sparse_attention_xattn_amd import synthetic
    print(f"[full-size] {name}: generating inputs", flush=True)
    return synthetic.workload_inputs(name, L)


def _run(name, L=None, chunk_starts=None, cache_block=None, threshold=None, stride=None):
    from block_sparse_attention_xattn_amd import synthetic
    from block_sparse_attention_xattn_amd.prefill import ChunkedPrefill
    w = synthetic.WORKLOADS[name]
    q, k, v = _inputs(name, L)
    tau = w["threshold"] if threshold is None else threshold
    S = w["stride"] if stride is None else stride
    run = ChunkedPrefill(q.to(DEV), k.to(DEV), v.to(DEV), chunk=w["chunk"], stride=S, threshold=tau,
                         chunk_starts=chunk_starts, cache_block=cache_block)
    print(f"[full-size] {name}: running {len(run.starts)} chunk(s) on the GPU (S={S}, tau={tau})", flush=True)
    run.track_density = True
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


def _density_vs_oracle(run):
    """The library's density counts over the run equal the oracle's counts of the GPU's masks (and of the
    cache blocks those masks select)."""
    sel = tot = kept = avail = 0
    for b in run.bufs:
        m = b.mask.cpu().numpy()
        s, t = O.density_counts(m)
        sel, tot = sel + s, tot + t
        ncb = b.p // run.density_cache_block
        if ncb:
            sub = run.density_cache_block // B
            _, anyk = O.mask_to_cache_blocks(m, 0, ncb, sub, True)
            k_, a_ = O.comm_density_counts(anyk)
            kept, avail = kept + k_, avail + a_
    got = run.density()
    assert (got["selected"], got["causal"]) == (sel, tot), (got, sel, tot)
    assert (got["kept_cache_blocks"], got["cache_blocks"]) == (kept, avail), (got, kept, avail)
    print(f"[full-size] density {got['density']:.4f} ({sel}/{tot}), comm density "
          f"{got['comm_density'] if got['comm_density'] is None else round(got['comm_density'], 4)} "
          f"({kept}/{avail})", flush=True)
    return got


def _check_head_chunk(q, k, v, run, i, h, g, S, tau, qbs):
    """Oracle estimate for one head of chunk i; attention for query blocks qbs with the GPU's mask rows."""
    b = run.bufs[i]
    p = b.p
    c = b.scores.shape[1] * B
    qh = _f64(q[p:p + c, h])
    kh = _f64(k[:p + c, h // g])
    ref_s = O.estimate_head(qh, kh, p, S, B)[None]
    ref_m = O.select_blocks(ref_s, p, tau, B)
    PAR.check_scores(b.scores[h:h + 1].cpu().numpy(), ref_s)
    n_diff, _ = PAR.check_mask(b.mask[h:h + 1].cpu().numpy(), ref_s, ref_m, p, tau, label=f"chunk {i} head {h}")
    gm = b.mask[h:h + 1].cpu().numpy()
    checked = 0
    kv = slice(h // g, h // g + 1)
    for qb in qbs:
        rows = slice(p + qb * B, p + (qb + 1) * B)
        ro, rl = PAR.oracle_chunk_attention(O, _f64(q[rows, h:h + 1]), _f64(k[:p + c, kv]), _f64(v[:p + c, kv]),
                                            p + qb * B, p, gm[:, qb:qb + 1])
        go = _f64(run.out[rows, h:h + 1])
        gl = _f64(b.lse[h:h + 1, qb * B:(qb + 1) * B])
        PAR.check_out_lse(go, gl, ro, rl, PAR.OUT_ATOL_BF16)
        checked += 1
    return n_diff, checked


def test_llama8b_32k_8x4k():
    w, q, k, v, run, tau, S = _run("llama8b_32k_8x4k")
    _invariants(run, S)
    _density_vs_oracle(run)
    g = w["hq"] // w["hkv"]
    checked = 0
    pairs = [(0, 0), (3, 13), (7, 31)]
    for i, h in pairs:
        print(f"[full-size] chunk {i} head {h}: oracle estimate + attention", flush=True)
        _, c = _check_head_chunk(q, k, v, run, i, h, g, S, tau, [0, 17, 31])
        checked += c
    assert checked == 3 * len(pairs)


def _cache_block_checks(w, q, k, v, run, tau, S, heads_for_oracle, attn_samples, all_heads):
    b = run.bufs[0]
    p = b.p
    g = w["hq"] // w["hkv"]
    sub = 1024 // B
    ncb = p // 1024
    # reducer output is the OR of the GPU's own mask (bit-exact), first/last forced
    gm = b.mask.cpu().numpy().astype(bool)
    per_ref, any_ref = O.mask_to_cache_blocks(gm, 0, ncb, sub, True)
    assert np.array_equal(b.keep_per_head.cpu().numpy(), per_ref)
    assert np.array_equal(b.keep_any.cpu().numpy(), any_ref)
    assert np.array_equal(b.keep_any_blocks.cpu().numpy(), O.expand_cache_keep(any_ref, sub, ncb * sub))
    print(f"[full-size] cache blocks: oracle estimate for {len(heads_for_oracle)} head(s)", flush=True)
    ref_s = np.stack([O.estimate_head(_f64(q[p:, h]), _f64(k[:, h // g]), p, S, B) for h in heads_for_oracle])
    ref_m = O.select_blocks(ref_s, p, tau, B)
    PAR.check_scores(b.scores[heads_for_oracle].cpu().numpy(), ref_s)
    PAR.check_mask(b.mask[heads_for_oracle].cpu().numpy(), ref_s, ref_m, p, tau, label="cache-block chunk")
    if all_heads:
        # the union keep list needs every head: the oracle's own keep list equals the GPU's
        _, ref_any = O.mask_to_cache_blocks(ref_m, 0, ncb, sub, True)
        assert np.array_equal(b.keep_any.cpu().numpy(), ref_any), "cache-block keep list differs from the oracle's"
    # attention over the kept cache blocks (the GPU's keep list, proven above to be the OR of its mask) and the
    # chunk's own keys (dense causal), merged by LSE
    keep = O.expand_cache_keep(b.keep_any.cpu().numpy(), sub, ncb * sub)
    checked = 0
    for h, qb in attn_samples:
        print(f"[full-size] cache blocks: attention head {h} query block {qb}", flush=True)
        rows = slice(p + qb * B, p + (qb + 1) * B)
        kv = slice(h // g, h // g + 1)
        ro, rl = PAR.oracle_chunk_attention(O, _f64(q[rows, h:h + 1]), _f64(k[:p + 4096, kv]), _f64(v[:p + 4096, kv]),
                                            p + qb * B, p, keep[None, None, :], cur_mask="dense")
        PAR.check_out_lse(_f64(run.out[rows, h:h + 1]), _f64(b.lse[h:h + 1, qb * B:(qb + 1) * B]), ro, rl,
                          PAR.OUT_ATOL_BF16)
        checked += 1
    assert checked == len(attn_samples)


def test_llama8b_128k_last_chunk_cache_blocks():
    """Full size (131072 keys, chunk at 126976): invariants, reducer = OR of the mask, two heads' estimate vs the
    oracle, attention rows over the kept cache blocks + the chunk, density and comm density."""
    w, q, k, v, run, tau, S = _run("llama8b_128k_last_chunk", chunk_starts=[126976], cache_block=1024)
    _invariants(run, S)
    got = _density_vs_oracle(run)
    assert got["cache_blocks"] == 124
    _cache_block_checks(w, q, k, v, run, tau, S, [0, 21], [(0, 0), (21, 31), (13, 17)], all_heads=False)


def test_llama8b_cache_blocks_16k_all_heads():
    """Same generator and launch form at 16384 keys (chunk at 12288): union keep list and attention vs oracle."""
    w, q, k, v, run, tau, S = _run("llama8b_128k_last_chunk", L=16384, chunk_starts=[12288], cache_block=1024)
    _invariants(run, S)
    _density_vs_oracle(run)
    _cache_block_checks(w, q, k, v, run, tau, S, list(range(w["hq"])), [(5, 0), (30, 31), (17, 12)],
                        all_heads=True)


def _dense_rows(w, q, k, v, run, pairs):
    b = run.bufs[0]
    p = b.p
    g = w["hq"] // w["hkv"]
    for h, qb in pairs:
        rows = slice(p + qb * B, p + (qb + 1) * B)
        ro, rl = O.bsa(_f64(q[rows, h:h + 1]), _f64(k[:p + 4096, h // g:h // g + 1]),
                       _f64(v[:p + 4096, h // g:h // g + 1]), p + qb * B, 0, None, 0, True)
        PAR.check_out_lse(_f64(run.out[rows, h:h + 1]), _f64(b.lse[h:h + 1, qb * B:(qb + 1) * B]), ro, rl,
                          PAR.OUT_ATOL_BF16)


@pytest.mark.parametrize("stride", [8, 16])
def test_llama8b_64k_threshold_one_is_dense(stride):
    w, q, k, v, run, tau, S = _run("llama8b_64k_sweep", threshold=1.0, stride=stride, chunk_starts=[61440])
    _invariants(run, S)
    got = _density_vs_oracle(run)
    assert got["selected"] == got["causal"]
    m = run.bufs[0].mask.cpu().numpy().astype(bool)
    p = run.bufs[0].p
    nqb, nkb = m.shape[1], m.shape[2]
    causal = np.arange(nkb)[None, :] <= (p // B + np.arange(nqb))[:, None]
    assert np.array_equal(m, np.broadcast_to(causal, m.shape))
    _dense_rows(w, q, k, v, run, [(0, 0), (19, 31), (9, 16)])


@pytest.mark.parametrize("stride", [8, 16])
def test_llama8b_64k_sweep_strides(stride):
    w, q, k, v, run, tau, S = _run("llama8b_64k_sweep", threshold=0.9, stride=stride,
                                   chunk_starts=[0, 28672, 61440])
    _invariants(run, S)
    _density_vs_oracle(run)
    g = w["hq"] // w["hkv"]
    checked = 0
    for i, h in [(1, 7), (2, 26)]:
        checked += _check_head_chunk(q, k, v, run, i, h, g, S, 0.9, [3, 30])[1]
    assert checked == 4


@pytest.mark.parametrize("stride,tau", [(8, 0.8), (8, 0.95), (8, 0.99), (16, 0.8), (16, 0.95), (16, 0.99)])
def test_llama8b_64k_threshold_points(stride, tau):
    """The 64K sweep's other (stride, threshold) points on one chunk each (the middle and the last)."""
    p = 28672 if tau < 0.99 else 61440
    w, q, k, v, run, tau, S = _run("llama8b_64k_sweep", threshold=tau, stride=stride, chunk_starts=[p])
    _invariants(run, S)
    _density_vs_oracle(run)
    g = w["hq"] // w["hkv"]
    h = {0.8: 3, 0.95: 22, 0.99: 30}[tau]
    _, checked = _check_head_chunk(q, k, v, run, 0, h, g, S, tau, [0, 15, 31])
    assert checked == 3


def test_gqa7_128k_32x4k():
    w, q, k, v, run, tau, S = _run("gqa7_128k_32x4k")
    _invariants(run, S)
    _density_vs_oracle(run)
    g = w["hq"] // w["hkv"]
    checked = 0
    for i, h in [(0, 6), (16, 13), (31, 27)]:
        print(f"[full-size] gqa7 chunk {i} head {h}", flush=True)
        checked += _check_head_chunk(q, k, v, run, i, h, g, S, tau, [0, 15, 31])[1]
    assert checked == 9
