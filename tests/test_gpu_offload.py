"""GPU parity of the offloaded history path (pinned host cache blocks, device ring).

* xattn_offload_blocks stores K bit for bit in the host blocks;
* bsa_history_offloaded over a keep list of host blocks equals the oracle's
  attention over exactly those cache blocks without the causal rule, with
  the ring reused (three groups of two), with one group, and with an empty
  list (out 0, lse -inf);
* the offloaded chunked prefill (downsampled estimate, kept cache blocks
  through the ring, dense causal chunk, merge) matches the oracle and keeps
  the same cache blocks as the resident path with the same estimator.

The host packed V is bsa_pack_v of the whole store, byte for byte; keep
lists include runs of consecutive ids (one copy per run) and runs cut by a
group boundary.

The estimate over host-resident history keys (xattn_estimate_offloaded)
equals xattn_estimate over the same keys on the device bit for bit, and the
oracle's three-stage streaming form (key chunks of one ring group) to the
score / mask tolerances; the offloaded prefill with that estimate keeps the
cache blocks that the oracle's estimate and reducer keep and matches the
oracle's attention over them.
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


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(torch.bfloat16)


@pytest.fixture(scope="module")
def offloaded():
    from block_sparse_attention_xattn_amd import binding as B
    hq, hkv, d, cb, p = 4, 2, 128, 1024, 12288
    q = _rand((1024, hq, d), 20)
    k = _rand((p, hkv, d), 21)
    v = _rand((p, hkv, d), 22)
    kd, vd = k.to(DEV), v.to(DEV)
    stores = {}
    for group in (2, 8):
        st = B.OffloadedKV(p // cb, hkv, d, DEV, cb, group, max_offload_blocks=4)
        for b0 in range(0, p, 4 * cb):
            B.xattn_offload_blocks(st, kd[b0:b0 + 4 * cb], vd[b0:b0 + 4 * cb], b0 // cb)
        stores[group] = st
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, stores=stores, p=p, cb=cb, hq=hq, d=d)


def test_host_k_blocks_exact(offloaded):
    st = offloaded["stores"][2]
    k = offloaded["k"]
    assert torch.equal(st.host_k.view(k.shape), k)


def test_host_vt_is_the_packed_v_of_the_whole_store(offloaded):
    from block_sparse_attention_xattn_amd import binding as B
    st, v, p = offloaded["stores"][8], offloaded["v"], offloaded["p"]
    packed = B.PackedV(p, v.shape[1], v.shape[2], torch.bfloat16, DEV)
    B.bsa_pack_v(v.to(DEV), packed, 0)
    torch.cuda.synchronize()
    ref = packed.buf[:p * v.shape[1] * v.shape[2] * 2].cpu()
    assert torch.equal(st.host_vt.view(torch.uint8), ref)


@pytest.mark.parametrize("group,keep", [(2, [0, 2, 3, 7, 8, 11]), (8, [1, 4, 5, 10]), (2, []),
                                        (2, [0, 1, 2, 3, 4, 5, 6]), (8, [2, 3, 4, 5, 6, 7, 9, 10, 11]),
                                        (8, list(range(12)))])
def test_history_offloaded_vs_oracle(offloaded, group, keep):
    from block_sparse_attention_xattn_amd import binding as B
    q, k, v, p, cb, hq, d = (offloaded[x] for x in ("q", "k", "v", "p", "cb", "hq", "d"))
    st = offloaded["stores"][group]
    qd = q.to(DEV)
    mk = lambda *s, dt=torch.float32: torch.empty(*s, dtype=dt, device=DEV)  # noqa: E731
    out, lse = mk(1024, hq, d, dt=torch.bfloat16), mk(hq, 1024)
    po, pl = mk(1024, hq, d, dt=torch.bfloat16), mk(hq, 1024)
    B.bsa_history_offloaded(qd, p, st, keep, out, lse, po, pl)
    torch.cuda.synchronize()
    keep_any = np.zeros(p // cb, dtype=np.uint8)
    keep_any[keep] = 1
    mask = np.broadcast_to(O.expand_cache_keep(keep_any, cb // 128, p // 128), (hq, 1024 // 128, p // 128))
    ro, rl = O.bsa(_np(q), _np(k), _np(v), p, 0, mask, 0, False)
    PAR.check_out_lse(_np(out), _np(lse), ro, rl, PAR.OUT_ATOL_BF16)


def test_offloaded_chunked_prefill_16k():
    from block_sparse_attention_xattn_amd import synthetic
    from block_sparse_attention_xattn_amd.offload import OffloadedChunkedPrefill
    from block_sparse_attention_xattn_amd.prefill import ChunkedPrefill
    w = synthetic.WORKLOADS["llama8b_128k_last_chunk"]
    q, k, v = synthetic.workload_inputs("llama8b_128k_last_chunk", 16384)
    p, S, tau = 12288, w["stride"], w["threshold"]
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    off = OffloadedChunkedPrefill(qd, kd, vd, chunk=4096, stride=S, threshold=tau, cache_block=1024, group=4,
                                  chunk_starts=[p])
    off.run()
    res = ChunkedPrefill(qd, kd, vd, chunk=4096, stride=S, threshold=tau, chunk_starts=[p], cache_block=1024,
                         estimator="downsampled")
    res.run()
    torch.cuda.synchronize()
    keep_res = [i for i, x in enumerate(res.bufs[0].keep_any.cpu().tolist()) if x]
    assert off.kept[p] == keep_res
    _, rm = O.estimate_history_downsampled(_np(q[p:]), O.downsample_keys(_np(k[:p]), S), S, tau)
    ref_keep = O.history_cache_blocks_downsampled(rm, p // 1024)
    keep = O.expand_cache_keep(ref_keep, 8, p // 128)
    g = w["hq"] // w["hkv"]
    for h, qb in [(0, 0), (13, 17), (31, 31)]:
        rows = slice(p + qb * 128, p + (qb + 1) * 128)
        kvh = h // g
        o1, l1 = O.bsa(_np(q[rows, h:h + 1]), _np(k[:p, kvh:kvh + 1]), _np(v[:p, kvh:kvh + 1]), p + qb * 128, 0,
                       keep[None, None, :], 0, False)
        o2, l2 = O.bsa(_np(q[rows, h:h + 1]), _np(k[p:, kvh:kvh + 1]), _np(v[p:, kvh:kvh + 1]), p + qb * 128, p,
                       None, 0, True)
        ro, rl = O.merge(o1, l1, o2, l2)
        PAR.check_out_lse(_np(off.out[rows, h:h + 1]), _np(off.lse[p][h:h + 1, qb * 128:(qb + 1) * 128]), ro, rl,
                          PAR.OUT_ATOL_BF16)


@pytest.mark.parametrize("group,q_start", [(2, 12288), (8, 12288), (2, 4096), (8, 0)])
def test_estimate_offloaded(offloaded, group, q_start):
    from block_sparse_attention_xattn_amd import binding as B
    q, k, cb = offloaded["q"], offloaded["k"], offloaded["cb"]
    S, tau = 8, 0.9
    st = offloaded["stores"][group]
    k_cur = _rand((1024, k.shape[1], k.shape[2]), 23)
    qd, kcd = q.to(DEV), k_cur.to(DEV)
    sc, m = B.xattn_estimate_offloaded(qd, kcd, q_start, st, S, tau)
    k_all = torch.cat([k[:q_start], k_cur])
    rs, rm = B.xattn_estimate(qd, k_all.to(DEV), q_start, S, tau)
    torch.cuda.synchronize()
    assert torch.equal(sc, rs) and torch.equal(m, rm)
    ref_s = O.estimate_scores_kv_chunked(_np(q), _np(k_all), q_start, S, 128, group * cb)
    ref_m = O.select_blocks(ref_s, q_start, tau)
    PAR.check_scores(_np(sc), ref_s)
    PAR.check_mask(m.cpu().numpy(), ref_s, ref_m, q_start, tau)


def test_offloaded_chunked_prefill_streamed_16k():
    from block_sparse_attention_xattn_amd import synthetic
    from block_sparse_attention_xattn_amd.offload import OffloadedChunkedPrefill
    from block_sparse_attention_xattn_amd.prefill import ChunkedPrefill
    w = synthetic.WORKLOADS["llama8b_128k_last_chunk"]
    q, k, v = synthetic.workload_inputs("llama8b_128k_last_chunk", 16384)
    p, S, tau = 12288, w["stride"], w["threshold"]
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    off = OffloadedChunkedPrefill(qd, kd, vd, chunk=4096, stride=S, threshold=tau, cache_block=1024, group=4,
                                  chunk_starts=[p], estimator="streamed")
    off.run()
    res = ChunkedPrefill(qd, kd, vd, chunk=4096, stride=S, threshold=tau, chunk_starts=[p], cache_block=1024)
    res.run()
    torch.cuda.synchronize()
    keep_res = [i for i, x in enumerate(res.bufs[0].keep_any.cpu().tolist()) if x]
    assert off.kept[p] == keep_res
    rs, rm = O.estimate(_np(q[p:]), _np(k), p, S, tau)
    ref_keep = O.mask_to_cache_blocks(rm, 0, p // 1024)[1]
    assert off.kept[p] == [i for i in range(p // 1024) if ref_keep[i]]
    keep = O.expand_cache_keep(ref_keep, 8, p // 128)
    g = w["hq"] // w["hkv"]
    for h, qb in [(0, 0), (13, 17), (31, 31)]:
        rows = slice(p + qb * 128, p + (qb + 1) * 128)
        kvh = h // g
        o1, l1 = O.bsa(_np(q[rows, h:h + 1]), _np(k[:p, kvh:kvh + 1]), _np(v[:p, kvh:kvh + 1]), p + qb * 128, 0,
                       keep[None, None, :], 0, False)
        o2, l2 = O.bsa(_np(q[rows, h:h + 1]), _np(k[p:, kvh:kvh + 1]), _np(v[p:, kvh:kvh + 1]), p + qb * 128, p,
                       None, 0, True)
        ro, rl = O.merge(o1, l1, o2, l2)
        PAR.check_out_lse(_np(off.out[rows, h:h + 1]), _np(off.lse[p][h:h + 1, qb * 128:(qb + 1) * 128]), ro, rl,
                          PAR.OUT_ATOL_BF16)
