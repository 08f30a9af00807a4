"""GPU parity of the estimate against downsampled history keys.

* xattn_downsample_keys equals K[::stride] bit for bit (bf16 and fp32, at an
  offset into a larger buffer, strided input);
* xattn_estimate_history_ds against the oracle's
  estimate_history_downsampled: block scores within 1e-3 relative, masks
  identical up to threshold-boundary exemptions (block 0 the only forced
  block), at strides 4, 8 and 16, bf16 and fp32, GQA;
* at full size (the 128K last chunk: 126976 history tokens, 15872
  downsampled keys, 4096 queries, 32/8 heads) two heads against the oracle,
  row sums and the forced block on every row, and the cache-block union of
  the GPU mask by xattn_mask_to_cache_blocks equal to the OR of that mask.
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


def _rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_downsample_keys_exact(dtype):
    from block_sparse_attention_xattn_amd import binding as B
    full = _rand((512, 3, 128), dtype, 1).to(DEV)
    k = full[:, :2]                               # strided: token stride 3*128, head stride 128
    ds = torch.full((200, 2, 128), 7.0, dtype=dtype, device=DEV)
    B.xattn_downsample_keys(k, 8, ds, ds_offset=10)
    torch.cuda.synchronize()
    assert torch.equal(ds[10:74].cpu(), k[::8].cpu())
    assert (ds[:10] == 7.0).all() and (ds[74:] == 7.0).all()


@pytest.mark.parametrize("S,dtype,hq,hkv,d", [(8, torch.bfloat16, 4, 2, 128), (4, torch.bfloat16, 4, 4, 128),
                                              (16, torch.bfloat16, 7, 1, 128), (8, torch.float32, 2, 1, 64)])
def test_estimate_history_ds_vs_oracle(S, dtype, hq, hkv, d):
    from block_sparse_attention_xattn_amd import binding as B
    b = 128 // S
    q = _rand((512, hq, d), dtype, 2)
    k = _rand((3072, hkv, d), dtype, 3)
    kd = k.to(DEV)
    ds = torch.empty(3072 // S, hkv, d, dtype=dtype, device=DEV)
    B.xattn_downsample_keys(kd, S, ds)
    sc, m = B.xattn_estimate_history_ds(q.to(DEV), ds, S, 0.9)
    torch.cuda.synchronize()
    ref_s, ref_m = O.estimate_history_downsampled(_np(q), O.downsample_keys(_np(k), S), S, 0.9)
    assert sc.shape == (hq, 512 // b, 3072 // 128)
    PAR.check_scores(sc.cpu().numpy(), ref_s)
    PAR.check_mask(m.cpu().numpy(), ref_s, ref_m, 0, 0.9, hist_only=True)


def test_estimate_history_ds_128k_last_chunk():
    from block_sparse_attention_xattn_amd import binding as B, synthetic
    w = synthetic.WORKLOADS["llama8b_128k_last_chunk"]
    print("[downsampled] generating 128K inputs", flush=True)
    q, k, _ = synthetic.workload_inputs("llama8b_128k_last_chunk")
    p, S, tau = w["q_start_pos"], w["stride"], w["threshold"]
    qd, kd = q[p:].to(DEV), k[:p].to(DEV)
    ds = torch.empty(p // S, w["hkv"], w["d"], dtype=torch.bfloat16, device=DEV)
    B.xattn_downsample_keys(kd, S, ds)
    sc, m = B.xattn_estimate_history_ds(qd, ds, S, tau)
    n_cb = p // 1024
    _, keep_any, _ = B.xattn_mask_to_cache_blocks(m, 0, n_cb, 8, False)
    torch.cuda.synchronize()
    scn, mn = sc.cpu().numpy(), m.cpu().numpy().astype(bool)
    b = 128 // S
    np.testing.assert_allclose(scn.sum(axis=2), np.full(scn.shape[:2], b), rtol=2e-4)
    assert mn[:, :, 0].all()
    want = mn.reshape(mn.shape[0] * mn.shape[1], n_cb, 8).any(axis=(0, 2))
    assert np.array_equal(keep_any.cpu().numpy().astype(bool), want)
    g = w["hq"] // w["hkv"]
    kds = O.downsample_keys(_np(k[:p]), S)
    for h in (0, 29):
        print(f"[downsampled] oracle head {h}", flush=True)
        rs, rm = O.estimate_history_downsampled(_np(q[p:, h:h + 1]), kds[:, h // g:h // g + 1], S, tau)
        PAR.check_scores(scn[h:h + 1], rs)
        PAR.check_mask(mn[h:h + 1], rs, rm, 0, tau, hist_only=True)


def test_chunked_prefill_downsampled_16k():
    """The cache-block chunked prefill with the downsampled estimator (16384 keys, chunk at 12288):
    GPU mask vs oracle, keep list = OR of the GPU mask, and, where the oracle's keep list is the
    same, attention (kept cache blocks, dense causal chunk, merge) vs the oracle."""
    from block_sparse_attention_xattn_amd import synthetic
    from block_sparse_attention_xattn_amd.prefill import ChunkedPrefill
    w = synthetic.WORKLOADS["llama8b_128k_last_chunk"]
    q, k, v = synthetic.workload_inputs("llama8b_128k_last_chunk", 16384)
    p, S, tau = 12288, w["stride"], w["threshold"]
    run = ChunkedPrefill(q.to(DEV), k.to(DEV), v.to(DEV), chunk=4096, stride=S, threshold=tau, chunk_starts=[p],
                         cache_block=1024, estimator="downsampled")
    run.run()
    torch.cuda.synchronize()
    b = run.bufs[0]
    gm = b.mask.cpu().numpy().astype(bool)
    ncb = p // 1024
    want = gm.reshape(gm.shape[0] * gm.shape[1], ncb, 8).any(axis=(0, 2))
    assert np.array_equal(b.keep_any.cpu().numpy().astype(bool), want)
    rs, rm = O.estimate_history_downsampled(_np(q[p:]), O.downsample_keys(_np(k[:p]), S), S, tau)
    PAR.check_scores(b.scores.cpu().numpy(), rs)
    PAR.check_mask(gm, rs, rm, 0, tau, hist_only=True)
    ref_keep = O.history_cache_blocks_downsampled(rm, ncb)
    assert np.array_equal(ref_keep.astype(bool), want), "keep list differs from the oracle's"
    keep = O.expand_cache_keep(ref_keep, 8, ncb * 8)
    g = w["hq"] // w["hkv"]
    for h, qb in [(3, 0), (22, 31), (31, 9)]:
        rows = slice(p + qb * 128, p + (qb + 1) * 128)
        kvh = h // g
        o1, l1 = O.bsa(_np(q[rows, h:h + 1]), _np(k[:p, kvh:kvh + 1]), _np(v[:p, kvh:kvh + 1]), p + qb * 128, 0,
                       keep[None, None, :], 0, False)
        o2, l2 = O.bsa(_np(q[rows, h:h + 1]), _np(k[p:, kvh:kvh + 1]), _np(v[p:, kvh:kvh + 1]), p + qb * 128, p,
                       None, 0, True)
        ro, rl = O.merge(o1, l1, o2, l2)
        PAR.check_out_lse(_np(run.out[rows, h:h + 1]), _np(b.lse[h:h + 1, qb * 128:(qb + 1) * 128]), ro, rl,
                          PAR.OUT_ATOL_BF16)
