"""Chunked prefill of one layer with the history offloaded to host cache blocks.

XAttentionBSAPolicy page (compute_chunked_prefill over the offload engine's
CPU cache blocks, brought back through a ring of GPU slots) and the task plan
page ("Metadata 存储策略" scheme A, "Phase 3: select_blocks 实现"): only
K[::stride] of the history stays on the GPU; a chunk's estimate runs against
it, the union of its mask over heads and query blocks picks the 1024-token
cache blocks, only those are copied back (overlapped with the attention over
the blocks already copied), the chunk's own keys are attended densely with the
causal rule, the two parts are merged by LSE, and the chunk's K / V are then
offloaded as cache blocks for the chunks after it.

With estimator="streamed" the chunk's estimate is instead the full one of
select_blocks on the XAttentionBSAPolicy page, computed as the history K
arrives from the host through the same ring (xattn_estimate_offloaded); its
mask is reduced to cache blocks with the first and last history cache block
forced, as the resident path does, and no K[::stride] is kept.

Device memory per layer: the chunk's rows, K[::stride] of the whole layer
(downsampled estimator), a ring of 2 x group cache blocks of K and packed V,
and per-chunk buffers; the history K / V live in pinned host memory.
"""
from __future__ import annotations

import torch

from . import binding as B


class OffloadedChunkedPrefill:
    """q, k, v [L, H, d] bf16 on the GPU (only the current chunk's rows are read there); `starts` chunks run."""

    def __init__(self, q, k, v, chunk: int, stride: int, threshold: float, cache_block: int = 1024,
                 group: int = 8, chunk_starts=None, block: int = 128, estimator: str = "downsampled"):
        if estimator not in ("downsampled", "streamed"):
            raise ValueError("estimator must be 'downsampled' or 'streamed'")
        self.estimator = estimator
        self.q, self.k, self.v = q, k, v
        self.L, self.hq, self.d = q.shape
        self.hkv = k.shape[1]
        self.chunk, self.stride, self.threshold, self.block = chunk, stride, threshold, block
        self.cb = cache_block
        if chunk % cache_block or self.L % cache_block:
            raise ValueError("chunk and layer length must be whole cache blocks")
        dev = q.device
        self.starts = list(range(0, self.L, chunk)) if chunk_starts is None else list(chunk_starts)
        self.store = B.OffloadedKV(self.L // cache_block, self.hkv, self.d, dev, cache_block, group,
                                   max_offload_blocks=max(chunk // cache_block, 1))
        self.packed = B.PackedV(chunk, self.hkv, self.d, q.dtype, dev)
        max_p = max(self.starts)
        if estimator == "downsampled":
            self.k_ds = torch.empty(self.L // stride, self.hkv, self.d, dtype=k.dtype, device=dev)
            est_ws = max([B.xattn_estimate_history_ds_workspace_size(chunk, p // stride, self.hq, self.hkv, self.d,
                                                                      stride, block) for p in self.starts if p > 0]
                         or [0])
            rows, cols = chunk // (block // stride), max(max_p // block, 1)
        else:
            est_ws = max(B.xattn_estimate_workspace_size(chunk, p + chunk, self.hq, self.hkv, self.d, stride, block)
                         for p in self.starts)
            rows, cols = chunk // block, (max_p + chunk) // block
        self.est_ws = B.workspace(est_ws, dev)
        self.scores = torch.empty(self.hq, rows, cols, dtype=torch.float32, device=dev)
        self.mask = torch.empty(self.hq, rows, cols, dtype=torch.uint8, device=dev)
        ncb = max(max_p // cache_block, 1)
        self.keep_per_head = torch.empty(self.hq, rows, ncb, dtype=torch.uint8, device=dev)
        self.keep_any = torch.empty(ncb, dtype=torch.uint8, device=dev)
        self.keep_any_blocks = torch.empty(ncb * (cache_block // block), dtype=torch.uint8, device=dev)
        self.keep_host = torch.empty(ncb, dtype=torch.uint8, pin_memory=True)
        mk = lambda *s, dt=torch.float32: torch.empty(*s, dtype=dt, device=dev)  # noqa: E731
        self.o_hist, self.l_hist = mk(chunk, self.hq, self.d, dt=q.dtype), mk(self.hq, chunk)
        self.o_part, self.l_part = mk(chunk, self.hq, self.d, dt=q.dtype), mk(self.hq, chunk)
        self.o_cur, self.l_cur = mk(chunk, self.hq, self.d, dt=q.dtype), mk(self.hq, chunk)
        self.out = torch.empty(self.L, self.hq, self.d, dtype=q.dtype, device=dev)
        self.lse = {p: mk(self.hq, chunk) for p in self.starts}
        self.kept = {}

    def prepare(self):
        """State before the first selected chunk: its history offloaded and K[::stride] of it on the GPU."""
        p0 = self.starts[0]
        for b0 in range(0, p0, self.chunk):
            n = min(self.chunk, p0 - b0)
            B.xattn_offload_blocks(self.store, self.k[b0:b0 + n], self.v[b0:b0 + n], b0 // self.cb)
        if p0 > 0 and self.estimator == "downsampled":
            B.xattn_downsample_keys(self.k[:p0], self.stride, self.k_ds, 0)

    def select(self, p: int):
        """Queue the chunk's estimate and cache-block union; the kept ids reach the host with the returned event."""
        c = self.chunk
        ncb = p // self.cb
        if self.estimator == "downsampled":
            n_blk = p // self.block
            sc, m = self.scores[:, :, :n_blk], self.mask[:, :, :n_blk]
            B.xattn_estimate_history_ds(self.q[p:p + c], self.k_ds[:p // self.stride], self.stride, self.threshold,
                                        self.block, block_scores=sc, block_mask=m, ws=self.est_ws)
        else:
            n_blk = (p + c) // self.block
            sc, m = self.scores[:, :, :n_blk], self.mask[:, :, :n_blk]
            B.xattn_estimate_offloaded(self.q[p:p + c], self.k[p:p + c], p, self.store, self.stride, self.threshold,
                                       self.block, block_scores=sc, block_mask=m, ws=self.est_ws)
        # the downsampled estimate keeps the union only; the full estimate also forces the first / last block
        B.xattn_mask_to_cache_blocks(m, 0, ncb, self.cb // self.block, self.estimator == "streamed",
                                     keep_per_head=self.keep_per_head[:, :, :ncb], keep_any=self.keep_any[:ncb],
                                     keep_any_blocks=self.keep_any_blocks[:ncb * (self.cb // self.block)])
        self.keep_host[:ncb].copy_(self.keep_any[:ncb], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        return ev

    def run_chunk(self, p: int):
        c = self.chunk
        qc = self.q[p:p + c]
        if self.estimator == "downsampled":
            B.xattn_downsample_keys(self.k[p:p + c], self.stride, self.k_ds, p // self.stride)
        B.bsa_pack_v(self.v[p:p + c], self.packed, 0)
        lse = self.lse[p]
        if p > 0:
            ready = self.select(p)
            # the chunk's own keys do not depend on the selection: queued before the host waits for it
            B.bsa_prefill_packed(qc, self.k[p:p + c], self.packed, 0, p, p, None, 0, True, out=self.o_cur,
                                 lse=self.l_cur)
            ready.synchronize()
            keep = [i for i in range(p // self.cb) if self.keep_host[i]]
            self.kept[p] = keep
            B.bsa_history_offloaded(qc, p, self.store, keep, self.o_hist, self.l_hist, self.o_part, self.l_part)
            B.attn_merge(self.o_hist, self.l_hist, self.o_cur, self.l_cur, o_out=self.out[p:p + c], lse_out=lse)
        else:
            B.bsa_prefill_packed(qc, self.k[p:p + c], self.packed, 0, p, p, None, 0, True, out=self.out[p:p + c],
                                 lse=lse)
        B.xattn_offload_blocks(self.store, self.k[p:p + c], self.v[p:p + c], p // self.cb)

    def run(self):
        self.prepare()
        for p in self.starts:
            self.run_chunk(p)
        return self.out
