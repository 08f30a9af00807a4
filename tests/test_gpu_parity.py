"""GPU parity: every entry point of libxattn.so against the CPU oracle.

Inputs are seeded; the oracle runs in float64 on exactly the values the GPU
sees (bf16 inputs are rounded once on the host, then upcast).  Shapes span
several tiles and ragged tails (partial key blocks, empty rows, GQA groups of
1, 2, 4 and 7).
"""
import os

import numpy as np
import pytest
import torch

from oracle import xattn_oracle as O
from tests import parity as PAR

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from block_sparse_attention_xattn_amd import binding
    binding.lib()  # raises if the library is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


def _np(t):
    return t.detach().float().cpu().double().numpy()


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(*shape, generator=g)).to(dtype)


# --------------------------------------------------------------------------- merge
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("q_len,heads,d", [(256, 4, 128), (384, 3, 64), (1, 1, 8), (128, 2, 96)])
def test_merge(dtype, q_len, heads, d):
    from block_sparse_attention_xattn_amd import binding as B
    oa = _rand((q_len, heads, d), dtype, 1)
    ob = _rand((q_len, heads, d), dtype, 2)
    la = _rand((heads, q_len), torch.float32, 3, 4.0)
    lb = _rand((heads, q_len), torch.float32, 4, 4.0)
    la.view(-1)[::7] = -float("inf")
    lb.view(-1)[::5] = -float("inf")
    ro, rl = O.merge(_np(oa), _np(la), _np(ob), _np(lb))
    go, gl = B.attn_merge(oa.to(DEV), la.to(DEV), ob.to(DEV), lb.to(DEV))
    torch.cuda.synchronize()
    tol = PAR.OUT_ATOL_BF16 if dtype == torch.bfloat16 else 1e-5
    PAR.check_out_lse(_np(go), _np(gl), ro, rl, tol)
    # in place: out aliases o_a, lse_out aliases lse_a
    ia, il = oa.to(DEV), la.to(DEV)
    B.attn_merge(ia, il, ob.to(DEV), lb.to(DEV), o_out=ia, lse_out=il)
    torch.cuda.synchronize()
    PAR.check_out_lse(_np(ia), _np(il), ro, rl, tol)


# --------------------------------------------------------------------------- reducer
@pytest.mark.parametrize("seed,H,nqb,ncols,kb_begin,sub,force", [
    (0, 32, 32, 992, 0, 8, True), (1, 4, 3, 37, 0, 8, True), (2, 2, 5, 40, 3, 4, False), (3, 1, 1, 8, 0, 8, True)])
def test_reducer(seed, H, nqb, ncols, kb_begin, sub, force):
    from block_sparse_attention_xattn_amd import binding as B
    rng = np.random.default_rng(seed)
    mask = (rng.random((H, nqb, ncols)) < 0.02).astype(np.uint8)
    ncb = (ncols - kb_begin + sub - 1) // sub
    rp, ra = O.mask_to_cache_blocks(mask, kb_begin, ncb, sub, force)
    gp, ga, gb = B.xattn_mask_to_cache_blocks(torch.from_numpy(mask).to(DEV), kb_begin, ncb, sub, force)
    torch.cuda.synchronize()
    assert np.array_equal(gp.cpu().numpy(), rp)
    assert np.array_equal(ga.cpu().numpy(), ra)
    assert np.array_equal(gb.cpu().numpy(), O.expand_cache_keep(ra, sub, ncb * sub))


# --------------------------------------------------------------------------- bsa
BSA_CASES = [
    # hq, hkv, d, dtype, q_len, q_start, kv_start, kv_len, causal, density, seed
    (2, 1, 64, torch.float32, 256, 0, 0, 256, True, 1.0, 0),
    (4, 2, 128, torch.bfloat16, 384, 256, 0, 640, True, 0.5, 1),
    (4, 1, 128, torch.bfloat16, 256, 512, 0, 512, False, 0.4, 2),
    (7, 1, 128, torch.bfloat16, 256, 384, 384, 256, True, 0.6, 3),
    (2, 2, 64, torch.bfloat16, 128, 1024, 128, 901, False, 0.5, 4),   # ragged key tail
    (8, 4, 128, torch.float32, 256, 128, 0, 384, True, 0.5, 5),
    (4, 4, 128, torch.bfloat16, 512, 0, 0, 512, True, 0.0, 6),       # only forced-free empty rows
]


def _bsa_case(hq, hkv, d, dtype, q_len, q_start, kv_start, kv_len, causal, density, seed):
    from block_sparse_attention_xattn_amd import binding as B
    q = _rand((q_len, hq, d), dtype, 10 + seed)
    k = _rand((kv_len, hkv, d), dtype, 20 + seed)
    v = _rand((kv_len, hkv, d), dtype, 30 + seed)
    ncols = (kv_start + kv_len + 127) // 128
    rng = np.random.default_rng(seed)
    mask = (rng.random((hq, q_len // 128, ncols)) < density).astype(np.uint8)
    ro, rl = O.bsa(_np(q), _np(k), _np(v), q_start, kv_start, mask, 0, causal, None, 128)
    go, gl = B.bsa_prefill(q.to(DEV), k.to(DEV), v.to(DEV), q_start, kv_start, torch.from_numpy(mask).to(DEV),
                           0, causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    tol = PAR.OUT_ATOL_BF16 if dtype == torch.bfloat16 else PAR.OUT_ATOL_F32
    return PAR.check_out_lse(_np(go), _np(gl), ro, rl, tol)


@pytest.mark.parametrize("case", BSA_CASES, ids=[f"bsa{i}" for i in range(len(BSA_CASES))])
def test_bsa(case):
    _bsa_case(*case)


def test_bsa_dense_and_broadcast_mask():
    from block_sparse_attention_xattn_amd import binding as B
    hq, hkv, d, q_len, p = 4, 2, 128, 256, 512
    q = _rand((q_len, hq, d), torch.bfloat16, 40)
    k = _rand((p, hkv, d), torch.bfloat16, 41)
    v = _rand((p, hkv, d), torch.bfloat16, 42)
    row = np.array([1, 0, 0, 1], dtype=np.uint8)
    full = np.broadcast_to(row, (hq, q_len // 128, 4)).copy()
    ro, rl = O.bsa(_np(q), _np(k), _np(v), p, 0, full, 0, False)
    go, gl = B.bsa_prefill(q.to(DEV), k.to(DEV), v.to(DEV), p, 0, torch.from_numpy(row).to(DEV).view(1, 1, -1), 0,
                           False, out_dtype=torch.float32, mask_head_stride=0, mask_row_stride=0)
    torch.cuda.synchronize()
    PAR.check_out_lse(_np(go), _np(gl), ro, rl, PAR.OUT_ATOL_BF16)
    ro, rl = O.bsa(_np(q), _np(k), _np(v), p, 0, None, 0, False)
    go, gl = B.bsa_prefill(q.to(DEV), k.to(DEV), v.to(DEV), p, 0, None, 0, False)
    torch.cuda.synchronize()
    PAR.check_out_lse(_np(go), _np(gl), ro, rl, PAR.OUT_ATOL_BF16)


# --------------------------------------------------------------------------- estimate
EST_CASES = [
    # hq, hkv, d, dtype, q_len, q_start, stride, threshold, seed
    (2, 1, 64, torch.float32, 1024, 0, 8, 0.9, 0),
    (4, 2, 128, torch.bfloat16, 512, 512, 8, 0.95, 1),
    (4, 1, 128, torch.bfloat16, 256, 768, 16, 0.9, 2),
    (2, 2, 128, torch.bfloat16, 384, 128, 4, 0.8, 3),
    (2, 1, 64, torch.bfloat16, 256, 256, 2, 0.9, 4),
    (7, 1, 128, torch.bfloat16, 256, 1792, 8, 1.0, 5),
    (4, 2, 64, torch.float32, 640, 1280, 8, 0.5, 6),
    (4, 2, 128, torch.bfloat16, 128, 3968, 8, 0.0, 7),   # threshold 0: only block 0 and the diagonal, one query block
]


@pytest.mark.parametrize("case", EST_CASES, ids=[f"est{i}" for i in range(len(EST_CASES))])
def test_estimate(case):
    from block_sparse_attention_xattn_amd import binding as B
    hq, hkv, d, dtype, q_len, p, S, tau, seed = case
    k_len = p + q_len
    q = _rand((q_len, hq, d), dtype, 50 + seed)
    k = _rand((k_len, hkv, d), dtype, 60 + seed)
    rs, rm = O.estimate(_np(q), _np(k), p, S, tau)
    gs, gm = B.xattn_estimate(q.to(DEV), k.to(DEV), p, S, tau)
    torch.cuda.synchronize()
    PAR.check_scores(gs.cpu().numpy(), rs)
    PAR.check_mask(gm.cpu().numpy(), rs, rm, p, tau)


def test_estimate_tile_walk_ragged():
    """More 256 x 256 score tiles than the GPU has compute units, so each workgroup walks several of them and skips
    the ones right of the causal limit; the last row and column tiles are partial (q_len 4992 at q_start 4096:
    624 reshaped rows, 1136 reshaped columns at stride 8; 32 query / 8 kv heads, 480 tiles).  Three heads are
    compared with the oracle."""
    from block_sparse_attention_xattn_amd import binding as B
    hq, hkv, d, q_len, p, S, tau = 32, 8, 128, 4992, 4096, 8, 0.9
    k_len = p + q_len
    q = _rand((q_len, hq, d), torch.bfloat16, 91)
    k = _rand((k_len, hkv, d), torch.bfloat16, 92)
    gs, gm = B.xattn_estimate(q.to(DEV), k.to(DEV), p, S, tau)
    torch.cuda.synchronize()
    gs, gm = gs.cpu().numpy(), gm.cpu().numpy()
    for h in (0, 13, 31):
        kvh = h // (hq // hkv)
        rs, rm = O.estimate(_np(q[:, h:h + 1]), _np(k[:, kvh:kvh + 1]), p, S, tau)
        PAR.check_scores(gs[h:h + 1], rs)
        PAR.check_mask(gm[h:h + 1], rs, rm, p, tau)


def test_estimate_long_history_rows():
    """Rows of 4096 key blocks (q_len 256 at q_start 524032, 2 query heads on one kv head): the selection sorts
    4096 keys per row (16 per thread) and the GEMM walks 512 tiles; compared whole with the oracle."""
    from block_sparse_attention_xattn_amd import binding as B
    hq, hkv, d, q_len, p, S, tau = 2, 1, 128, 256, 524032, 8, 0.9
    q = _rand((q_len, hq, d), torch.bfloat16, 93)
    k = _rand((p + q_len, hkv, d), torch.bfloat16, 94)
    rs, rm = O.estimate(_np(q), _np(k), p, S, tau)
    gs, gm = B.xattn_estimate(q.to(DEV), k.to(DEV), p, S, tau)
    torch.cuda.synchronize()
    PAR.check_scores(gs.cpu().numpy(), rs)
    PAR.check_mask(gm.cpu().numpy(), rs, rm, p, tau)


def test_estimate_max_key_blocks():
    """The largest key length the estimate accepts, 8192 key blocks (q_len 128 at q_start 1048448): the selection
    keeps 8192 sort keys in 64 KiB of dynamic LDS (above the default limit, raised at launch); compared whole with
    the oracle."""
    from block_sparse_attention_xattn_amd import binding as B
    hq, hkv, d, q_len, p, S, tau = 1, 1, 128, 128, 1048448, 8, 0.9
    q = _rand((q_len, hq, d), torch.bfloat16, 95)
    k = _rand((p + q_len, hkv, d), torch.bfloat16, 96)
    rs, rm = O.estimate(_np(q), _np(k), p, S, tau)
    gs, gm = B.xattn_estimate(q.to(DEV), k.to(DEV), p, S, tau)
    torch.cuda.synchronize()
    assert gs.shape[-1] == 8192
    PAR.check_scores(gs.cpu().numpy(), rs)
    PAR.check_mask(gm.cpu().numpy(), rs, rm, p, tau)


# --------------------------------------------------------------------------- composed
def test_tiny_chunked_prefill_end_to_end():
    """The 1K fp32 workload: 2 query heads sharing 1 kv head, d 64, stride 8, threshold 0.9."""
    from block_sparse_attention_xattn_amd import synthetic
    from block_sparse_attention_xattn_amd.prefill import ChunkedPrefill
    q, k, v = synthetic.tiny(0)
    ref = O.chunk_prefill(_np(q), _np(k), _np(v), 0, 8, 0.9)
    run = ChunkedPrefill(q.to(DEV), k.to(DEV), v.to(DEV), chunk=1024, stride=8, threshold=0.9)
    out = run.run()
    torch.cuda.synchronize()
    b = run.bufs[0]
    PAR.check_scores(b.scores.cpu().numpy(), ref["scores"])
    n_diff, _ = PAR.check_mask(b.mask.cpu().numpy(), ref["scores"], ref["mask"], 0, 0.9)
    assert n_diff == 0
    PAR.check_out_lse(_np(out), _np(b.lse), ref["out"], ref["lse"], PAR.OUT_ATOL_F32)


@pytest.mark.parametrize("fused", [True, False])
def test_small_multichunk_prefill_end_to_end(fused):
    """Four chunks against the oracle's chunked prefill (history + chunk attention, LSE merge), with the GPU
    running each chunk as one causal pass (fused) or as the two segments and the merge."""
    from block_sparse_attention_xattn_amd import synthetic
    from block_sparse_attention_xattn_amd.prefill import ChunkedPrefill
    q, k, v = synthetic.long_context(4096, 8, 2, 128, n_needles=4, seed=7)
    ref = O.chunked_prefill(_np(q), _np(k), _np(v), 1024, 8, 0.9)
    run = ChunkedPrefill(q.to(DEV), k.to(DEV), v.to(DEV), chunk=1024, stride=8, threshold=0.9, fused=fused)
    assert run.fused == fused
    out = run.run()
    torch.cuda.synchronize()
    same = True
    qn, kn, vn = _np(q), _np(k), _np(v)
    for i, b in enumerate(run.bufs):
        PAR.check_scores(b.scores.cpu().numpy(), ref["scores"][i])
        n_diff, _ = PAR.check_mask(b.mask.cpu().numpy(), ref["scores"][i], ref["masks"][i], b.p, 0.9,
                                   label=f"chunk {i}")
        same &= n_diff == 0
        # attention is always checked: the oracle attends with the GPU's own mask (an exempt flip changes only
        # which blocks are attended, not how), history + chunk merged by LSE
        rows = slice(b.p, b.p + 1024)
        ro, rl = PAR.oracle_chunk_attention(O, qn[rows], kn[:b.p + 1024], vn[:b.p + 1024], b.p, b.p,
                                            b.mask.cpu().numpy())
        PAR.check_out_lse(_np(out[rows]), _np(b.lse), ro, rl, PAR.OUT_ATOL_BF16)
    if same:
        # and the oracle's whole chunked prefill (its own masks) where they agree
        PAR.check_out_lse(_np(out), np.concatenate([_np(b.lse) for b in run.bufs], axis=1), ref["out"], ref["lse"],
                          PAR.OUT_ATOL_BF16)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_packed_v_appends_and_offsets(dtype):
    """V packed chunk by chunk, then attention over history and chunk from the packed buffer."""
    from block_sparse_attention_xattn_amd import binding as B
    hq, hkv, d, L, C = 4, 2, 128, 1024, 384
    q = _rand((L, hq, d), dtype, 70)
    k = _rand((L, hkv, d), dtype, 71)
    v = _rand((L, hkv, d), dtype, 72)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    packed = B.PackedV(L, hkv, d, dtype, DEV)
    for p0 in range(0, L, C):                     # last piece is ragged (256 tokens)
        B.bsa_pack_v(vd[p0:p0 + C], packed, p0)
    p = 768
    rng = np.random.default_rng(7)
    mask = (rng.random((hq, (L - p) // 128, L // 128)) < 0.6).astype(np.uint8)
    md = torch.from_numpy(mask).to(DEV)
    tol = PAR.OUT_ATOL_BF16 if dtype == torch.bfloat16 else PAR.OUT_ATOL_F32
    ro, rl = O.bsa(_np(q[p:]), _np(k[:p]), _np(v[:p]), p, 0, mask, 0, False)
    go, gl = B.bsa_prefill_packed(qd[p:], kd[:p], packed, 0, p, 0, md, 0, False, out_dtype=torch.float32)
    torch.cuda.synchronize()
    PAR.check_out_lse(_np(go), _np(gl), ro, rl, tol)
    ro, rl = O.bsa(_np(q[p:]), _np(k[p:]), _np(v[p:]), p, p, mask, 0, True)
    go, gl = B.bsa_prefill_packed(qd[p:], kd[p:], packed, p, p, p, md, 0, True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    PAR.check_out_lse(_np(go), _np(gl), ro, rl, tol)


def test_segments_in_one_launch():
    """History (non-causal, mask offset), the chunk's own keys (causal) and a broadcast-mask segment in one grid."""
    from block_sparse_attention_xattn_amd import binding as B
    hq, hkv, d, L, p = 8, 2, 128, 1280, 768
    q = _rand((L, hq, d), torch.bfloat16, 80)
    k = _rand((L, hkv, d), torch.bfloat16, 81)
    v = _rand((L, hkv, d), torch.bfloat16, 82)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    packed = B.PackedV(L, hkv, d, torch.bfloat16, DEV)
    B.bsa_pack_v(vd, packed, 0)
    rng = np.random.default_rng(9)
    nqb, nkb = (L - p) // 128, L // 128
    mask = (rng.random((hq, nqb, nkb)) < 0.5).astype(np.uint8)
    row = (rng.random(p // 128) < 0.5).astype(np.uint8)
    md, rowd = torch.from_numpy(mask).to(DEV), torch.from_numpy(row).to(DEV).view(1, 1, -1)
    outs = [(torch.empty(L - p, hq, d, dtype=torch.float32, device=DEV),
             torch.empty(hq, L - p, dtype=torch.float32, device=DEV)) for _ in range(3)]
    segs = [dict(k=kd[128:p], kv_start=128, v_token_offset=128, block_mask=md, causal=False,
                 out=outs[0][0], lse=outs[0][1]),
            dict(k=kd[p:], kv_start=p, v_token_offset=p, block_mask=md, causal=True, out=outs[1][0], lse=outs[1][1]),
            dict(k=kd[:p], kv_start=0, v_token_offset=0, block_mask=rowd, mask_head_stride=0, mask_row_stride=0,
                 causal=False, out=outs[2][0], lse=outs[2][1])]
    B.bsa_prefill_segments(qd[p:], packed, p, segs)
    torch.cuda.synchronize()
    refs = [O.bsa(_np(q[p:]), _np(k[128:p]), _np(v[128:p]), p, 128, mask, 0, False),
            O.bsa(_np(q[p:]), _np(k[p:]), _np(v[p:]), p, p, mask, 0, True),
            O.bsa(_np(q[p:]), _np(k[:p]), _np(v[:p]), p, 0, np.broadcast_to(row, (hq, nqb, p // 128)), 0, False)]
    for (go, gl), (ro, rl) in zip(outs, refs):
        PAR.check_out_lse(_np(go), _np(gl), ro, rl, PAR.OUT_ATOL_BF16)


def test_attention_event_hook():
    """The measurement hook: the events land around the attention kernel, inside the call's own interval,
    and the results are the same as without them."""
    from block_sparse_attention_xattn_amd import binding as B
    hq, hkv, d, L, p = 8, 2, 128, 1280, 768
    qd, kd, vd = (_rand((L, h, d), torch.bfloat16, 90 + i).to(DEV) for i, h in enumerate((hq, hkv, hkv)))
    packed = B.PackedV(L, hkv, d, torch.bfloat16, DEV)
    B.bsa_pack_v(vd, packed, 0)
    md = torch.from_numpy((np.random.default_rng(3).random((hq, (L - p) // 128, L // 128)) < 0.5)
                          .astype(np.uint8)).to(DEV)

    def call():
        outs = [(torch.empty(L - p, hq, d, dtype=torch.float32, device=DEV),
                 torch.empty(hq, L - p, dtype=torch.float32, device=DEV)) for _ in range(2)]
        segs = [dict(k=kd[:p], kv_start=0, v_token_offset=0, block_mask=md, causal=False,
                     out=outs[0][0], lse=outs[0][1]),
                dict(k=kd[p:], kv_start=p, v_token_offset=p, block_mask=md, causal=True,
                     out=outs[1][0], lse=outs[1][1])]
        B.bsa_prefill_segments(qd[p:], packed, p, segs)
        return outs

    plain = call()
    c0, c1, k0, k1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    c0.record()
    try:
        B.xattn_set_attention_events(k0, k1)
        hooked = call()
    finally:
        B.xattn_set_attention_events(None, None)
    c1.record()
    torch.cuda.synchronize()
    t_call, t_kernel = c0.elapsed_time(c1), k0.elapsed_time(k1)
    assert 0.0 < t_kernel <= t_call
    assert c0.elapsed_time(k0) >= 0.0 and k1.elapsed_time(c1) >= 0.0
    for (a, b), (x, y) in zip(plain, hooked):
        assert torch.equal(a, x) and torch.equal(b, y)


def test_segments_work_order():
    """The work order of a segmented launch, read back from its workspace.

    Exact integer checks: every item's kept-tile count equals the mask row's
    count up to the causal limit (as a multiset over items); the split items
    are the ones of at least 32 tiles longer than total / compute units
    (none here: rows of at most 10 blocks), each with a median inside its row;
    the entries are the unsplit items once (part 0) and the split items twice
    (parts 1 and 2), sorted by descending count, and every entry was taken (the
    ticket passed the entry count).  The outputs of this call match the oracle.
    """
    from block_sparse_attention_xattn_amd import binding as B
    hq, hkv, d, L, p = 8, 2, 128, 1280, 768
    q = _rand((L, hq, d), torch.bfloat16, 83)
    k = _rand((L, hkv, d), torch.bfloat16, 84)
    v = _rand((L, hkv, d), torch.bfloat16, 85)
    qd, kd = q.to(DEV), k.to(DEV)
    packed = B.PackedV(L, hkv, d, torch.bfloat16, DEV)
    B.bsa_pack_v(v.to(DEV), packed, 0)
    rng = np.random.default_rng(10)
    nqb, nkb = (L - p) // 128, L // 128
    mask = (rng.random((hq, nqb, nkb)) < 0.5).astype(np.uint8)
    row = (rng.random(p // 128) < 0.5).astype(np.uint8)
    md, rowd = torch.from_numpy(mask).to(DEV), torch.from_numpy(row).to(DEV).view(1, 1, -1)
    outs = [(torch.empty(L - p, hq, d, dtype=torch.float32, device=DEV),
             torch.empty(hq, L - p, dtype=torch.float32, device=DEV)) for _ in range(3)]
    segs = [dict(k=kd[128:p], kv_start=128, v_token_offset=128, block_mask=md, causal=False,
                 out=outs[0][0], lse=outs[0][1]),
            dict(k=kd[p:], kv_start=p, v_token_offset=p, block_mask=md, causal=True, out=outs[1][0], lse=outs[1][1]),
            dict(k=kd[:p], kv_start=0, v_token_offset=0, block_mask=rowd, mask_head_stride=0, mask_row_stride=0,
                 causal=False, out=outs[2][0], lse=outs[2][1])]
    n1 = 3 * hq * nqb              # single-head items (the workspace layout is sized for these)
    ws = B.workspace(B.bsa_prefill_segments_workspace_size(L - p, hq, d, 3), DEV)
    ws.fill_(0xAB)
    B.bsa_prefill_segments(qd[p:], packed, p, segs, ws=ws)
    torch.cuda.synchronize()
    # with an even number of query heads per kv head the items are head pairs (2j, 2j + 1) whose count is the
    # number of blocks either head kept
    pair = (hq // hkv) % 2 == 0 and os.environ.get("XATTN_PAIR", "1") != "0"
    heads = [(2 * j, 2 * j + 1) for j in range(hq // 2)] if pair else [(h,) for h in range(hq)]
    n = 3 * len(heads) * nqb
    a = lambda b: (b + 255) // 256 * 256  # noqa: E731
    w32 = ws.cpu().numpy().view(np.int32)
    ms = min(n1, 512)
    off = 256
    ctl = w32[0:3]
    weights = w32[off // 4:off // 4 + n]; off += a(4 * n1)
    mids = w32[off // 4:off // 4 + n]; off += a(4 * n1)
    off += a(4 * n1)  # slots
    off += a(4 * ms)  # split items
    n_split = int(ctl[2])
    order = w32[off // 4:off // 4 + n + n_split]
    union = lambda hs, qb, c0, c1: int(np.any(mask[list(hs), qb, c0:c1], axis=0).sum())  # noqa: E731
    expect = [union(hs, qb, 1, 6) for hs in heads for qb in range(nqb)]
    expect += [union(hs, qb, 6, 6 + min(qb + 1, 4)) for hs in heads for qb in range(nqb)]
    expect += [int(row.sum())] * (len(heads) * nqb)
    assert sorted(weights.tolist()) == sorted(expect)
    slots = torch.cuda.get_device_properties(0).multi_processor_count  # one attention workgroup per CU
    thr = int(weights.sum()) // slots
    split = {i for i in range(n) if weights[i] >= 20 and weights[i] > thr}
    # every entry was taken: the first min(slots, grid) workgroups read entries 0 .. slots-1 without a ticket,
    # the others take tickets (counted in ctl[0]) from there on
    assert ctl[1] == n + n_split and n_split == len(split) and slots + ctl[0] >= ctl[1]
    items, parts = order // 4, order % 4
    assert {int(i) for i, pt in zip(items, parts) if pt == 0} == set(range(n)) - split
    for pt in (1, 2):
        assert sorted(int(i) for i, x in zip(items, parts) if x == pt) == sorted(split)
    ew = np.where(parts == 0, weights[items], np.where(parts == 1, weights[items] // 2,
                                                        weights[items] - weights[items] // 2))
    assert np.all(np.diff(ew) <= 0)
    for i in split:
        assert 0 <= mids[i] <= nkb
    refs = [O.bsa(_np(q[p:]), _np(k[128:p]), _np(v[128:p]), p, 128, mask, 0, False),
            O.bsa(_np(q[p:]), _np(k[p:]), _np(v[p:]), p, p, mask, 0, True),
            O.bsa(_np(q[p:]), _np(k[:p]), _np(v[:p]), p, 0, np.broadcast_to(row, (hq, nqb, p // 128)), 0, False)]
    for (go, gl), (ro, rl) in zip(outs, refs):
        PAR.check_out_lse(_np(go), _np(gl), ro, rl, PAR.OUT_ATOL_BF16)


def test_segments_split_items():
    """Rows of ~40 kept tiles on a small grid: every such item is split in two at its median kept block,
    the halves run as separate entries and are merged by LSE; out and LSE match the oracle."""
    from block_sparse_attention_xattn_amd import binding as B
    hq, hkv, d, L, p = 4, 2, 128, 8192, 7680
    q = _rand((L, hq, d), torch.bfloat16, 86)
    k = _rand((L, hkv, d), torch.bfloat16, 87)
    v = _rand((L, hkv, d), torch.bfloat16, 88)
    qd, kd = q.to(DEV), k.to(DEV)
    packed = B.PackedV(L, hkv, d, torch.bfloat16, DEV)
    B.bsa_pack_v(v.to(DEV), packed, 0)
    rng = np.random.default_rng(11)
    nqb, nkb = (L - p) // 128, L // 128
    mask = (rng.random((hq, nqb, nkb)) < 0.7).astype(np.uint8)
    mask[:, :, 0] = 1
    md = torch.from_numpy(mask).to(DEV)
    outs = [(torch.empty(L - p, hq, d, dtype=torch.bfloat16, device=DEV),
             torch.empty(hq, L - p, dtype=torch.float32, device=DEV)) for _ in range(2)]
    segs = [dict(k=kd[:p], kv_start=0, v_token_offset=0, block_mask=md, causal=False, out=outs[0][0],
                 lse=outs[0][1]),
            dict(k=kd[p:], kv_start=p, v_token_offset=p, block_mask=md, causal=True, out=outs[1][0], lse=outs[1][1])]
    ws = B.workspace(B.bsa_prefill_segments_workspace_size(L - p, hq, d, 2), DEV)
    B.bsa_prefill_segments(qd[p:], packed, p, segs, ws=ws)
    torch.cuda.synchronize()
    ctl = ws[:12].cpu().numpy().view(np.int32)
    hist_rows = mask[:, :, :p // 128].sum(axis=2)
    assert (hist_rows >= 32).all()
    pair = (hq // hkv) % 2 == 0 and os.environ.get("XATTN_PAIR", "1") != "0"   # items are head pairs
    assert ctl[2] == (hq // 2 if pair else hq) * nqb, f"expected every history item split, got {ctl[2]}"
    refs = [O.bsa(_np(q[p:]), _np(k[:p]), _np(v[:p]), p, 0, mask, 0, False),
            O.bsa(_np(q[p:]), _np(k[p:]), _np(v[p:]), p, p, mask, 0, True)]
    for (go, gl), (ro, rl) in zip(outs, refs):
        PAR.check_out_lse(_np(go), _np(gl), ro, rl, PAR.OUT_ATOL_BF16)


def test_rows_longer_than_one_block_list():
    """Rows of more than 1024 candidate key blocks are listed 1024 blocks at a time: dense attention over
    1100 blocks (no work order), and a segmented call over 2200 blocks at mask density 0.9 whose rows are
    split in two (each half again longer than 1024 blocks); out and LSE match the oracle."""
    from block_sparse_attention_xattn_amd import binding as B
    hq, hkv, d = 4, 2, 128
    for n_kb, dense in ((1100, True), (2200, False)):
        kv = n_kb * 128
        q = _rand((128, hq, d), torch.bfloat16, 90 + n_kb)
        k = _rand((kv, hkv, d), torch.bfloat16, 91 + n_kb)
        v = _rand((kv, hkv, d), torch.bfloat16, 92 + n_kb)
        qd, kd = q.to(DEV), k.to(DEV)
        packed = B.PackedV(kv, hkv, d, torch.bfloat16, DEV)
        B.bsa_pack_v(v.to(DEV), packed, 0)
        if dense:
            out, lse = B.bsa_prefill_packed(qd, kd, packed, 0, kv, 0, None, 0, False)
            mask = None
        else:
            rng = np.random.default_rng(12)
            mask = (rng.random((hq, 1, n_kb)) < 0.9).astype(np.uint8)
            out = torch.empty(128, hq, d, dtype=torch.bfloat16, device=DEV)
            lse = torch.empty(hq, 128, dtype=torch.float32, device=DEV)
            segs = [dict(k=kd, kv_start=0, v_token_offset=0, block_mask=torch.from_numpy(mask).to(DEV), causal=False,
                         out=out, lse=lse)]
            ws = B.workspace(B.bsa_prefill_segments_workspace_size(128, hq, d, 1), DEV)
            B.bsa_prefill_segments(qd, packed, kv, segs, ws=ws)
            torch.cuda.synchronize()
            pair = (hq // hkv) % 2 == 0 and os.environ.get("XATTN_PAIR", "1") != "0"   # items are head pairs
            assert int(ws[:12].cpu().numpy().view(np.int32)[2]) == (hq // 2 if pair else hq), \
                "expected every item split"
        torch.cuda.synchronize()
        ro, rl = O.bsa(_np(q), _np(k), _np(v), kv, 0, mask, 0, False)
        PAR.check_out_lse(_np(out), _np(lse), ro, rl, PAR.OUT_ATOL_BF16)


@pytest.mark.parametrize("hq,hkv,density", [(7, 1, 0.5), (6, 2, 0.3), (4, 1, 0.9), (16, 2, 0.4)])
def test_segments_head_pairs(hq, hkv, density):
    """Segmented calls whose items pair up the query heads of a kv head (an odd group size leaves a one-head item
    per kv head), with per-head random masks (the heads' kept lists differ, so each head must skip the blocks only
    its partner kept), a history segment long enough to be split and the chunk's own causal segment; out and
    LSE of every head match the oracle."""
    from block_sparse_attention_xattn_amd import binding as B
    d, L, p = 128, 6144, 5632
    q = _rand((L, hq, d), torch.bfloat16, 95 + hq)
    k = _rand((L, hkv, d), torch.bfloat16, 96 + hq)
    v = _rand((L, hkv, d), torch.bfloat16, 97 + hq)
    qd, kd = q.to(DEV), k.to(DEV)
    packed = B.PackedV(L, hkv, d, torch.bfloat16, DEV)
    B.bsa_pack_v(v.to(DEV), packed, 0)
    rng = np.random.default_rng(hq * 10 + hkv)
    nqb, nkb = (L - p) // 128, L // 128
    mask = (rng.random((hq, nqb, nkb)) < density).astype(np.uint8)
    mask[:, :, 0] = 1
    md = torch.from_numpy(mask).to(DEV)
    outs = [(torch.empty(L - p, hq, d, dtype=torch.bfloat16, device=DEV),
             torch.empty(hq, L - p, dtype=torch.float32, device=DEV)) for _ in range(2)]
    segs = [dict(k=kd[:p], kv_start=0, v_token_offset=0, block_mask=md, causal=False, out=outs[0][0],
                 lse=outs[0][1]),
            dict(k=kd[p:], kv_start=p, v_token_offset=p, block_mask=md, causal=True, out=outs[1][0], lse=outs[1][1])]
    ws = B.workspace(B.bsa_prefill_segments_workspace_size(L - p, hq, d, 2), DEV)
    B.bsa_prefill_segments(qd[p:], packed, p, segs, ws=ws)
    torch.cuda.synchronize()
    refs = [O.bsa(_np(q[p:]), _np(k[:p]), _np(v[:p]), p, 0, mask, 0, False),
            O.bsa(_np(q[p:]), _np(k[p:]), _np(v[p:]), p, p, mask, 0, True)]
    for (go, gl), (ro, rl) in zip(outs, refs):
        PAR.check_out_lse(_np(go), _np(gl), ro, rl, PAR.OUT_ATOL_BF16)
