"""One attention layer's chunked prefill through the C ABI.

XAttentionBSAPolicy (nano-vllm xattn_bsa.py page), select_blocks +
compute_chunked_prefill: for the query chunk at global position p,
  1. estimate block scores and the block mask against K[0 : p+C];
  2. attend the history K/V[0 : p) without the causal rule, kept blocks only;
  3. attend the chunk's own K/V[p : p+C) with the causal rule, kept blocks only;
  4. merge the two partial results by their LSE.
The cache-block variant first reduces the history part of the mask to
1024-token cache blocks (union over heads and query blocks, first and last
forced) and attends every 128-token block of the kept cache blocks, with
dense causal attention inside the chunk.  With estimator="downsampled" (task
plan page, "Metadata 存储策略" and "Phase 3: select_blocks 实现") the cache
blocks are chosen instead from an estimate of the chunk against K[::stride]
of the history, which each chunk appends for its own keys; the full K is
then not read by the estimate.

V is kept packed once per layer in the attention kernel's layout: each chunk
packs its own V rows when it starts (bsa_pack_v), and both attention calls
read the packed buffer (one bsa_prefill_segments launch for bf16, head_dim
128; two bsa_prefill_packed calls otherwise).  With a block mask per chunk
(bf16, head_dim 128, fused=True) steps 2-4 are one causal pass over keys
[0 : p+C) with the chunk's mask row: the history lies before every query,
so the causal rule only acts on the chunk's own keys and the result is the
merged one (up to rounding) without writing the two partial results.  All
buffers are allocated up front; a step only enqueues library calls on the
current stream.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B


@dataclass
class ChunkBuffers:
    p: int
    scores: torch.Tensor
    mask: torch.Tensor
    o_hist: torch.Tensor | None
    l_hist: torch.Tensor | None
    o_cur: torch.Tensor
    l_cur: torch.Tensor
    lse: torch.Tensor
    keep_per_head: torch.Tensor | None = None
    keep_any: torch.Tensor | None = None
    keep_any_blocks: torch.Tensor | None = None


class ChunkedPrefill:
    """Preallocated chunked prefill of one layer (batch 1).

    q [L, Hq, d], k/v [L, Hkv, d] on the GPU.  ``chunk_starts`` selects which
    chunks to run (default: all, in order).  ``cache_block`` switches the
    history attention to the cache-block form.
    """

    def __init__(self, q, k, v, chunk: int, stride: int, threshold: float, block: int = 128,
                 chunk_starts=None, cache_block: int | None = None, out_dtype=None, estimator: str = "full",
                 fused: bool = True):
        self.q, self.k, self.v = q, k, v
        self.L, self.hq, self.d = q.shape
        self.hkv = k.shape[1]
        self.chunk, self.stride, self.threshold, self.block = chunk, stride, threshold, block
        self.cache_block = cache_block
        if estimator not in ("full", "downsampled"):
            raise ValueError("estimator must be 'full' or 'downsampled'")
        if estimator == "downsampled" and not cache_block:
            raise ValueError("the downsampled estimator selects cache blocks: pass cache_block")
        self.estimator = estimator
        # fused: with a block mask per chunk (not the cache-block form), a chunk's history and own keys as one
        # causal pass over keys [0, p + C) (bf16, head_dim 128)
        self.fused = fused and q.dtype == torch.bfloat16 and self.d == 128 and not cache_block
        dev = q.device
        self.out_dtype = q.dtype if out_dtype is None else out_dtype
        self.starts = list(range(0, self.L, chunk)) if chunk_starts is None else list(chunk_starts)
        dt = B.XA_BF16 if q.dtype == torch.bfloat16 else B.XA_F32
        max_k = max(p + min(chunk, self.L - p) for p in self.starts)
        est_ws = max(B.xattn_estimate_workspace_size(min(chunk, self.L - p), p + min(chunk, self.L - p),
                                                     self.hq, self.hkv, self.d, stride, block, dt)
                     for p in self.starts)
        bsa_ws = B.bsa_prefill_packed_workspace_size(chunk, max_k, self.hq, self.hkv, self.d, dt)
        if estimator == "downsampled":
            bds = block // stride
            est_ws = max([B.xattn_estimate_history_ds_workspace_size(min(chunk, self.L - p), p // stride, self.hq,
                                                                      self.hkv, self.d, stride, block, dt)
                          for p in self.starts if p > 0] or [0])
            self.k_ds = torch.empty(self.L // stride, self.hkv, self.d, dtype=k.dtype, device=dev)
        self.est_ws = B.workspace(est_ws, dev)
        self.bsa_ws = B.workspace(bsa_ws, dev) if bsa_ws > 0 else None
        self.seg_ws = B.workspace(B.bsa_prefill_segments_workspace_size(chunk, self.hq, self.d, 2), dev)
        self.packed = B.PackedV(self.L, self.hkv, self.d, q.dtype, dev)
        self.out = torch.empty(self.L, self.hq, self.d, dtype=self.out_dtype, device=dev)
        # density counts (select_blocks step 5 and the comm density after step 6), accumulated over the
        # chunks run while track_density is set: [kept causal pairs, causal pairs, kept cache blocks, cache
        # blocks].  Chunks without the cache-block form count the cache blocks their mask would load
        # (1024-token cache blocks, or cache_block tokens).
        self.track_density = False
        self.density_counts = torch.zeros(4, dtype=torch.int64, device=dev)
        self.density_cache_block = cache_block or 1024
        self._keep_scratch = torch.empty(max(self.L // self.density_cache_block, 1), dtype=torch.uint8, device=dev)
        self.bufs = []
        for p in self.starts:
            c = min(chunk, self.L - p)
            nqb, nkb = c // block, (p + c) // block
            hist = p > 0
            kb = None
            if estimator == "downsampled":
                # scores / mask over (query blocks of block/stride tokens, history blocks)
                shp = (self.hq, c // (block // stride), max(p // block, 1))
            else:
                shp = (self.hq, nqb, nkb)
            if hist and cache_block:
                sub = cache_block // block
                ncb = p // cache_block
                kb = dict(keep_per_head=torch.empty(self.hq, shp[1], ncb, dtype=torch.uint8, device=dev),
                          keep_any=torch.empty(ncb, dtype=torch.uint8, device=dev),
                          keep_any_blocks=torch.empty(ncb * sub, dtype=torch.uint8, device=dev))
            self.bufs.append(ChunkBuffers(
                p=p,
                scores=torch.empty(*shp, dtype=torch.float32, device=dev),
                mask=torch.empty(*shp, dtype=torch.uint8, device=dev),
                o_hist=torch.empty(c, self.hq, self.d, dtype=self.out_dtype, device=dev) if hist else None,
                l_hist=torch.empty(self.hq, c, dtype=torch.float32, device=dev) if hist else None,
                o_cur=torch.empty(c, self.hq, self.d, dtype=self.out_dtype, device=dev) if hist else self.out[p:p + c],
                l_cur=torch.empty(self.hq, c, dtype=torch.float32, device=dev),
                lse=torch.empty(self.hq, c, dtype=torch.float32, device=dev),
                **(kb or {})))

    # -- the calls of one chunk --------------------------------------------------
    def _len(self, b: ChunkBuffers) -> int:
        return min(self.chunk, self.L - b.p)

    def pack_history(self):
        """Pack V rows (and K[::stride] for the downsampled estimator) before the first selected chunk."""
        p0 = self.starts[0]
        if p0 > 0:
            B.bsa_pack_v(self.v[:p0], self.packed, 0)
            if self.estimator == "downsampled":
                B.xattn_downsample_keys(self.k[:p0], self.stride, self.k_ds, 0)

    def pack(self, b: ChunkBuffers):
        c = self._len(b)
        B.bsa_pack_v(self.v[b.p:b.p + c], self.packed, b.p)
        if self.estimator == "downsampled":
            B.xattn_downsample_keys(self.k[b.p:b.p + c], self.stride, self.k_ds, b.p // self.stride)

    def estimate(self, b: ChunkBuffers):
        c = self._len(b)
        if self.estimator == "downsampled":
            if b.p > 0:
                B.xattn_estimate_history_ds(self.q[b.p:b.p + c], self.k_ds[:b.p // self.stride], self.stride,
                                            self.threshold, self.block, block_scores=b.scores, block_mask=b.mask,
                                            ws=self.est_ws)
            return
        B.xattn_estimate(self.q[b.p:b.p + c], self.k[:b.p + c], b.p, self.stride, self.threshold, self.block,
                         block_scores=b.scores, block_mask=b.mask, ws=self.est_ws)

    def reduce(self, b: ChunkBuffers):
        if b.keep_any is None:
            return
        ncb = b.keep_any.shape[0]
        # the downsampled estimate's sketch keeps the union only (no forced first / last cache block)
        B.xattn_mask_to_cache_blocks(b.mask, 0, ncb, self.cache_block // self.block, self.estimator == "full",
                                     keep_per_head=b.keep_per_head, keep_any=b.keep_any,
                                     keep_any_blocks=b.keep_any_blocks)

    def attend(self, b: ChunkBuffers):
        """History (no causal rule) and the chunk's own keys (causal) in one segmented launch, or, fused,
        one causal pass over both with the chunk's mask row (the history lies before every query, so the causal
        rule only acts on the chunk's own keys), written straight to the output with no merge."""
        p = b.p
        c = self._len(b)
        qc = self.q[p:p + c]
        if self.fused:
            seg = dict(k=self.k[:p + c], kv_start=0, v_token_offset=0, block_mask=b.mask, causal=True,
                       out=self.out[p:p + c], lse=b.lse)
            B.bsa_prefill_segments(qc, self.packed, p, [seg], ws=self.seg_ws)
            return
        segs = []
        if p > 0:
            if b.keep_any_blocks is not None:
                segs.append(dict(k=self.k[:p], kv_start=0, v_token_offset=0, block_mask=b.keep_any_blocks.view(1, 1, -1),
                                 mask_head_stride=0, mask_row_stride=0, causal=False, out=b.o_hist, lse=b.l_hist))
            else:
                segs.append(dict(k=self.k[:p], kv_start=0, v_token_offset=0, block_mask=b.mask, causal=False,
                                 out=b.o_hist, lse=b.l_hist))
        # the cache-block form and the downsampled estimator attend the chunk's own keys densely
        cur_mask = None if (b.keep_any_blocks is not None or self.estimator == "downsampled") else b.mask
        segs.append(dict(k=self.k[p:p + c], kv_start=p, v_token_offset=p, block_mask=cur_mask, causal=True,
                         out=b.o_cur, lse=b.l_cur if p > 0 else b.lse))
        if self.q.dtype == torch.bfloat16 and self.d == 128:
            B.bsa_prefill_segments(qc, self.packed, p, segs, ws=self.seg_ws)
        else:
            for g in segs:
                B.bsa_prefill_packed(qc, g["k"], self.packed, g["v_token_offset"], p, g["kv_start"], g["block_mask"],
                                     0, g["causal"], out=g["out"], lse=g["lse"], ws=self.bsa_ws,
                                     mask_head_stride=g.get("mask_head_stride"),
                                     mask_row_stride=g.get("mask_row_stride"))

    def merge(self, b: ChunkBuffers):
        if b.p == 0 or self.fused:
            return
        c = self._len(b)
        B.attn_merge(b.o_hist, b.l_hist, b.o_cur, b.l_cur, o_out=self.out[b.p:b.p + c], lse_out=b.lse)

    def record_density(self, b: ChunkBuffers):
        """Add chunk b's compute and comm density counts to density_counts (on the stream, no host wait)."""
        diag0 = b.p // self.block
        if self.estimator == "downsampled":
            diag0 = b.mask.shape[2]  # history-only mask: every column precedes the chunk
        keep = b.keep_any
        ncb = b.p // self.density_cache_block
        if keep is None and ncb > 0 and self.estimator == "full":
            keep = self._keep_scratch[:ncb]
            B.xattn_mask_to_cache_blocks(b.mask, 0, ncb, self.density_cache_block // self.block, True,
                                         keep_any=keep, want=("any",))
        B.xattn_density_counts(self.density_counts, b.mask, diag0, keep if ncb > 0 else None)

    def reset_density(self):
        self.density_counts.zero_()

    def density(self) -> dict:
        """Compute and comm density of the chunks recorded since the last reset (one host read)."""
        c = [int(x) for x in self.density_counts.cpu().tolist()]
        return dict(selected=c[0], causal=c[1], density=c[0] / c[1] if c[1] else None,
                    kept_cache_blocks=c[2], cache_blocks=c[3], comm_density=c[2] / c[3] if c[3] else None)

    def run_chunk(self, i: int):
        b = self.bufs[i]
        self.pack(b)
        self.estimate(b)
        self.reduce(b)
        if self.track_density:
            self.record_density(b)
        self.attend(b)
        self.merge(b)

    def run(self):
        self.pack_history()
        for i in range(len(self.bufs)):
            self.run_chunk(i)
        return self.out
