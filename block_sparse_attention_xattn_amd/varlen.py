"""Prefill of a packed batch of sequences (varlen) in three calls.

XAttentionBSAPolicy page, compute_prefill (GPU-only mode): Q, K, V of several
sequences packed one after the other with cumulative lengths; each sequence
gets its own estimate, selection and causal block-sparse attention, its
queries at the end of its keys.  Here the whole batch is one pack of V, one
estimate (one GEMM grid and one selection grid over every sequence) and one
attention launch whose work order spans every sequence, so short sequences
fill the tail of long ones.  Every buffer is allocated up front.
"""
from __future__ import annotations

import torch

from . import binding as B


class VarlenPrefill:
    """q [total_q, Hq, d], k, v [total_k, Hkv, d] bf16 on the GPU; cu_seqlens_q / cu_seqlens_k host lists."""

    def __init__(self, q, k, v, cu_seqlens_q, cu_seqlens_k, stride: int, threshold: float, block: int = 128,
                 sparse: bool = True):
        self.q, self.k, self.v = q, k, v
        self.cu_q = [int(x) for x in cu_seqlens_q]
        self.cu_k = [int(x) for x in cu_seqlens_k]
        self.stride, self.threshold, self.block, self.sparse = stride, threshold, block, sparse
        _, self.hq, self.d = q.shape
        self.hkv = k.shape[1]
        dev = q.device
        total_k = self.cu_k[-1]
        self.packed = B.PackedV(total_k, self.hkv, self.d, q.dtype, dev)
        n = B.xattn_varlen_mask_elems(self.cu_q, self.cu_k, self.hq)
        self.scores = torch.empty(max(n, 1), dtype=torch.float32, device=dev)
        self.mask = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        self.est_ws = B.workspace(B.xattn_estimate_varlen_workspace_size(self.cu_q, self.cu_k, self.hq, self.hkv,
                                                                         stride), dev)
        self.bsa_ws = B.workspace(B.bsa_prefill_varlen_workspace_size(self.cu_q, self.cu_k, self.hq, self.d), dev)
        self.out = torch.empty_like(q)
        self.lse = torch.empty(max(self.hq * self.cu_q[-1], 1), dtype=torch.float32, device=dev)

    def pack(self):
        B.bsa_pack_v(self.v, self.packed, 0)

    def estimate(self):
        B.xattn_estimate_varlen(self.q, self.k, self.cu_q, self.cu_k, self.stride, self.threshold, self.block,
                                block_scores=self.scores, block_mask=self.mask, ws=self.est_ws)

    def attend(self):
        B.bsa_prefill_varlen(self.q, self.k, self.packed, self.cu_q, self.cu_k,
                             self.mask if self.sparse else None, out=self.out, lse=self.lse, ws=self.bsa_ws)

    def run(self):
        self.pack()
        if self.sparse:
            self.estimate()
        self.attend()
        return self.out

    def masks(self):
        return B.varlen_blocks(self.mask, self.cu_q, self.cu_k, self.hq, self.block)

    def block_scores(self):
        return B.varlen_blocks(self.scores, self.cu_q, self.cu_k, self.hq, self.block)

    def lses(self):
        return B.varlen_lse(self.lse, self.cu_q, self.hq)
