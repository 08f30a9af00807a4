"""Plain CPU oracle for XAttention block-sparse chunked prefill (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's ``cpu_baseline`` leg may import this module.  The product path
(the HIP library and its Python binding) never calls it and shares no code
with it.

Sources (the pages this follows; each function names its passage):

* "XAttention algorithm guide" -- the nano-vllm docs page
  ``docs/xattention_algorithm_guide.md`` (compare view of the nano-vllm
  ``tzj/vs_offload`` branch): sections "算法流程" (algorithm flow),
  "Stride Reshape 详解 / Inverse 模式" (stride reshape, inverse mode),
  "Triton Kernels 详解" (flat_group_gemm_fuse_reshape, softmax_fuse_block_sum),
  "块选择算法 (find_blocks_chunked)" with its "示例" (worked example),
  "BSA (Block Sparse Attention)", "计算复杂度" (complexity).
* "XAttentionBSAPolicy" -- the nano-vllm page
  ``nanovllm/kvcache/sparse/xattn_bsa.py``: methods ``compute_prefill``,
  ``select_blocks`` (softmax scale, chunk_start/current_index, causal
  post-processing, reduction to CPU blocks) and ``compute_chunked_prefill``
  (history non-causal + current chunk causal + LSE merge).
* "Online Softmax Merge" -- the nano-vllm ``CLAUDE.md`` section
  "Online Softmax Merge - Triton Fused Kernel" (merge formula).
* "Task plan" -- the nano-vllm ``task_plan.md`` page, section
  "select_blocks 设计" (OR of eight 128-token blocks into one 1024-token
  cache block), "Metadata 存储策略" (scheme A: keep K[::stride] of each
  offloaded block) and "Phase 3: select_blocks 实现" (estimate the chunk
  against the downsampled history with stride 1).

Readings where the pages are open (each is restated where it is used):

* Selection keeps the block that crosses the threshold (the worked example
  selects four blocks whose running sum first reaches 0.95 >= 0.9).
* The always-kept blocks (block 0 and the diagonal block) count toward the
  running mass first; the other blocks follow in descending score order,
  equal scores by ascending block index.  ``rule="literal"`` instead applies
  the printed pseudo-code (forced mass not counted, inclusive running sum
  compared strictly), kept for comparison only.
* threshold >= 1 keeps every causal block.
* Reshaped causality: reshaped column c is visible to reshaped row r iff
  c <= q_start_pos / stride + r.  Parity unpinned for stride > 1 beyond the
  stride-1 reduction and the invariants the tests check.
* LSE is natural-log, laid out [heads, q_len]; an empty key set gives out 0
  and lse -inf; merging with an lse of -inf returns the other input.
* Estimate against the downsampled history: every history key precedes the
  chunk, so no causal limit applies, and the chunk's diagonal block lies past
  the history keys, so block 0 is the only forced block.
* Packed batch (``compute_prefill`` handles one sequence and leaves larger
  batches to dense attention): each sequence is its own problem, its queries
  at the end of its keys (q_start_pos = k_len - q_len), with no attention
  across sequences.

All arrays are numpy float64 unless stated; token-major layouts
``[tokens, heads, head_dim]`` as in the pages' varlen tensors.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# Part 1: importance estimate
# ---------------------------------------------------------------------------

def reshape_q_inverse(q: np.ndarray, stride: int) -> np.ndarray:
    """Inverse-mode query reshape of one head.

    XAttention algorithm guide, "Stride Reshape 详解 / Inverse 模式": the
    reshaped query concatenates, along the feature axis, the strided slices
    starting at stride-1, stride-2, ..., 0.  Row r therefore holds tokens
    r*S+S-1, r*S+S-2, ..., r*S (in that order).

    q: [L, d] -> [L/S, S*d]
    """
    L, _ = q.shape
    assert L % stride == 0
    parts = [q[(stride - 1 - t)::stride] for t in range(stride)]
    return np.concatenate(parts, axis=1)


def reshape_k_forward(k: np.ndarray, stride: int) -> np.ndarray:
    """Forward-mode key reshape of one head.

    XAttention algorithm guide, "Stride Reshape 详解 / Inverse 模式": the
    reshaped key concatenates the strided slices starting at 0, 1, ...,
    stride-1.  Column c holds tokens c*S, c*S+1, ..., c*S+S-1.

    k: [L, d] -> [L/S, S*d]
    """
    L, _ = k.shape
    assert L % stride == 0
    parts = [k[t::stride] for t in range(stride)]
    return np.concatenate(parts, axis=1)


def reshaped_logits(q: np.ndarray, k: np.ndarray, stride: int) -> np.ndarray:
    """Scaled reshaped scores of one head, before masking.

    XAttention algorithm guide, "Triton Kernels 详解 / flat_group_gemm_fuse_reshape"
    (the product of the two reshaped matrices) and XAttentionBSAPolicy
    ``select_blocks`` (scale log2(e)/sqrt(d)/stride/norm with norm = 1, used
    with exp2; the same function in natural base is 1/(stride*sqrt(d))).

    q: [Lq, d], k: [Lk, d] -> [Lq/S, Lk/S]
    """
    d = q.shape[1]
    qr = reshape_q_inverse(q, stride)
    kr = reshape_k_forward(k, stride)
    return (qr @ kr.T) / (stride * math.sqrt(d))


def reshaped_causal_allowed(n_rows: int, n_cols: int, q_start_pos: int,
                            stride: int) -> np.ndarray:
    """Reshaped causal visibility: column c visible to row r iff c <= p/S + r.

    XAttentionBSAPolicy ``select_blocks`` passes the chunk's start in
    reshaped units (chunk_start) with is_causal; the query chunk sits at
    global position p, so row r of the chunk is global reshaped row p/S + r.
    Parity unpinned for stride > 1 (the pages give no numbers); at stride 1
    it is ordinary token causality.
    """
    assert q_start_pos % stride == 0
    r = np.arange(n_rows)[:, None]
    c = np.arange(n_cols)[None, :]
    return c <= (q_start_pos // stride + r)


def row_softmax_causal(z: np.ndarray, allowed: np.ndarray):
    """Row softmax over the allowed columns; returns (probabilities, max, sum).

    XAttention algorithm guide, "softmax_fuse_block_sum": per row the maximum
    and the sum of exponentials, then the normalised probabilities.
    """
    zm = np.where(allowed, z, NEG_INF)
    m = zm.max(axis=1)
    e = np.where(allowed, np.exp(zm - m[:, None]), 0.0)
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def block_sums(prob: np.ndarray, block: int, stride: int) -> np.ndarray:
    """Sum each (block/S x block/S) tile of the reshaped probabilities.

    XAttention algorithm guide, "softmax_fuse_block_sum" (pass 2: group the
    normalised row into block_size/stride columns and sum, then sum the rows
    of one query block).  Output [n_q_blocks, n_k_blocks].
    """
    b = block // stride
    R, N = prob.shape
    assert R % b == 0 and N % b == 0
    return prob.reshape(R // b, b, N // b, b).sum(axis=(1, 3))


def estimate_head(q: np.ndarray, k: np.ndarray, q_start_pos: int, stride: int,
                  block: int) -> np.ndarray:
    """Block scores of one query head against its key head.

    q: [Lq, d] (query chunk at global position q_start_pos),
    k: [Lk, d] with Lk == q_start_pos + Lq.  Returns [Lq/block, Lk/block].
    """
    Lq, Lk = q.shape[0], k.shape[0]
    assert Lk == q_start_pos + Lq
    assert Lq % block == 0 and q_start_pos % block == 0 and block % stride == 0
    z = reshaped_logits(q, k, stride)
    allowed = reshaped_causal_allowed(z.shape[0], z.shape[1], q_start_pos, stride)
    prob, _, _ = row_softmax_causal(z, allowed)
    return block_sums(prob, block, stride)


def estimate_scores(q: np.ndarray, k: np.ndarray, q_start_pos: int, stride: int,
                    block: int = 128) -> np.ndarray:
    """Block scores for all query heads (GQA: query head h reads key head h // g).

    XAttentionBSAPolicy ``expand_kv_for_gqa`` (repeat_interleave over the
    head axis).  q: [Lq, Hq, d], k: [Lk, Hkv, d] -> [Hq, Lq/block, Lk/block].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    Hq, Hkv = q.shape[1], k.shape[1]
    assert Hq % Hkv == 0
    g = Hq // Hkv
    return np.stack([estimate_head(q[:, h], k[:, h // g], q_start_pos, stride, block)
                     for h in range(Hq)])


def estimate_scores_kv_chunked(q: np.ndarray, k: np.ndarray, q_start_pos: int,
                               stride: int, block: int, kv_chunk: int) -> np.ndarray:
    """The same block scores by the pages' three-stage streaming form.

    XAttentionBSAPolicy ``select_blocks``: pass 1 computes per-row partial
    (max, sum of exp) for each key chunk under the causal rule; the partials
    are merged by online-softmax rescaling; pass 2 recomputes each chunk's
    scores, normalises with the merged statistics and sums blocks; the
    per-chunk block sums are concatenated along the key-block axis.
    kv_chunk must be a multiple of block.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    Lq, Hq, d = q.shape
    Lk, Hkv, _ = k.shape
    g = Hq // Hkv
    assert kv_chunk % block == 0 and Lk == q_start_pos + Lq
    R = Lq // stride
    out = []
    for h in range(Hq):
        qr = reshape_q_inverse(q[:, h], stride)
        kh = k[:, h // g]
        starts = list(range(0, Lk, kv_chunk))
        ms, ls = [], []
        for s0 in starts:                                    # pass 1
            kr = reshape_k_forward(kh[s0:s0 + kv_chunk], stride)
            z = (qr @ kr.T) / (stride * math.sqrt(d))
            c = s0 // stride + np.arange(kr.shape[0])[None, :]
            allowed = c <= (q_start_pos // stride + np.arange(R)[:, None])
            zm = np.where(allowed, z, NEG_INF)
            m = zm.max(axis=1)
            with np.errstate(invalid="ignore"):
                e = np.where(allowed, np.exp(zm - np.where(np.isfinite(m), m, 0.0)[:, None]), 0.0)
            ms.append(m)
            ls.append(e.sum(axis=1))
        m_g = np.max(np.stack(ms), axis=0)                   # merge of partial stats
        l_g = np.zeros(R)
        for m, l in zip(ms, ls):
            l_g += np.where(np.isfinite(m), l * np.exp(np.where(np.isfinite(m), m, 0.0) - m_g), 0.0)
        sums = []
        for s0 in starts:                                    # pass 2
            kr = reshape_k_forward(kh[s0:s0 + kv_chunk], stride)
            z = (qr @ kr.T) / (stride * math.sqrt(d))
            c = s0 // stride + np.arange(kr.shape[0])[None, :]
            allowed = c <= (q_start_pos // stride + np.arange(R)[:, None])
            p = np.where(allowed, np.exp(np.where(allowed, z, 0.0) - m_g[:, None]) / l_g[:, None], 0.0)
            sums.append(block_sums(p, block, stride))
        out.append(np.concatenate(sums, axis=1))
    return np.stack(out)


# ---------------------------------------------------------------------------
# Part 1b: cumulative-threshold selection
# ---------------------------------------------------------------------------

def select_row(scores: np.ndarray, forced: list[int], threshold: float,
               rule: str = "greedy") -> np.ndarray:
    """Cumulative-threshold selection of one row of block scores.

    XAttention algorithm guide, "块选择算法 (find_blocks_chunked)": total the
    row, keep the forced blocks, rank the others by score (descending) and
    keep them while the running mass is below threshold * total; the worked
    example ("示例") keeps the block at which the running sum first reaches
    the threshold.

    rule="greedy" (the reading used everywhere): forced mass counts first; a
    non-forced block is kept iff forced mass + mass of the blocks ranked
    before it < threshold * total.  Equal scores rank by ascending index.
    rule="literal": the printed pseudo-code (forced blocks zeroed before the
    sort, inclusive running sum of the others compared with <).
    threshold >= 1 keeps every block of the row.

    scores: [n] (only the causal prefix of a row is passed) -> bool [n]
    """
    n = scores.shape[0]
    keep = np.zeros(n, dtype=bool)
    if threshold >= 1.0:
        keep[:] = True
        return keep
    forced = sorted(set(int(f) for f in forced if 0 <= f < n))
    keep[forced] = True
    total = float(scores.sum())
    need = threshold * total
    others = [i for i in range(n) if i not in forced]
    order = sorted(others, key=lambda i: (-scores[i], i))
    if rule == "greedy":
        run = float(scores[forced].sum()) if forced else 0.0
        for i in order:
            if run < need:
                keep[i] = True
            run += float(scores[i])
    elif rule == "literal":
        run = 0.0
        for i in order:
            run += float(scores[i])
            if run < need:
                keep[i] = True
    else:
        raise ValueError(rule)
    return keep


def select_blocks(scores: np.ndarray, q_start_pos: int, threshold: float,
                  block: int = 128, rule: str = "greedy") -> np.ndarray:
    """Block mask for one query chunk.

    XAttentionBSAPolicy ``select_blocks``: current_index = number of key
    blocks before the chunk; query block qb's diagonal block is
    current_index + qb; block 0 (sink) and the diagonal are always kept;
    finally blocks right of the diagonal are cleared (the tril post-step).

    scores: [H, nQB, nKB] -> uint8 mask [H, nQB, nKB]
    """
    H, nQB, nKB = scores.shape
    cur = q_start_pos // block
    assert nKB == cur + nQB
    mask = np.zeros((H, nQB, nKB), dtype=np.uint8)
    for h in range(H):
        for qb in range(nQB):
            diag = cur + qb
            row = scores[h, qb, :diag + 1]
            keep = select_row(row, [0, diag], threshold, rule)
            mask[h, qb, :diag + 1] = keep
    return mask


def estimate(q, k, q_start_pos: int, stride: int, threshold: float,
             block: int = 128, rule: str = "greedy"):
    """xattn_estimate_chunked: (block scores, block mask) for one query chunk.

    XAttentionBSAPolicy ``compute_prefill`` / ``select_blocks`` (estimate,
    then find_blocks_chunked, then causal post-processing).
    """
    scores = estimate_scores(q, k, q_start_pos, stride, block)
    return scores, select_blocks(scores, q_start_pos, threshold, block, rule)


# ---------------------------------------------------------------------------
# Part 2: block-sparse attention with LSE
# ---------------------------------------------------------------------------

def bsa(q, k, v, q_start_pos: int, kv_start: int, mask, mask_kb_offset: int = 0,
        causal: bool = True, softmax_scale: float | None = None, block: int = 128):
    """Attention of a query chunk over the selected key blocks, with LSE.

    XAttention algorithm guide, "BSA (Block Sparse Attention)": exact softmax
    attention restricted to the 128x128 blocks the mask keeps, with token
    causality.  Plain definition, per query row i (global position p+i):
    J_i = {j : mask[h, i//block, (kv_start+j)//block - mask_kb_offset] and
    (not causal or kv_start+j <= p+i)};
    lse_i = log sum_{j in J_i} exp(s q_i.k_j),  out_i = sum_j exp(s q_i.k_j - lse_i) v_j.
    Empty J_i gives out 0 and lse -inf.

    q: [Lq, Hq, d]; k, v: [Lkv, Hkv, d]; mask: [Hq, nQB, nCols] (or None for
    all blocks).  Returns out [Lq, Hq, d], lse [Hq, Lq].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, Hq, d = q.shape
    Lkv, Hkv, _ = k.shape
    g = Hq // Hkv
    s = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    assert Lq % block == 0 and kv_start % block == 0 and q_start_pos % block == 0
    nQB = Lq // block
    nKBs = (Lkv + block - 1) // block
    out = np.zeros((Lq, Hq, d))
    lse = np.full((Hq, Lq), NEG_INF)
    for h in range(Hq):
        kh, vh = k[:, h // g], v[:, h // g]
        for qb in range(nQB):
            cols = []
            for jb in range(nKBs):
                gb = kv_start // block + jb
                if mask is None or mask[h, qb, gb - mask_kb_offset]:
                    cols.append(np.arange(jb * block, min((jb + 1) * block, Lkv)))
            if not cols:
                continue
            j = np.concatenate(cols)
            rows = np.arange(qb * block, (qb + 1) * block)
            logit = s * (q[rows, h] @ kh[j].T)
            if causal:
                vis = (kv_start + j)[None, :] <= (q_start_pos + rows)[:, None]
                logit = np.where(vis, logit, NEG_INF)
            m = logit.max(axis=1)
            ok = np.isfinite(m)
            m0 = np.where(ok, m, 0.0)
            e = np.exp(logit - m0[:, None])
            ssum = e.sum(axis=1)
            lse[h, rows] = np.where(ok, m0 + np.log(np.where(ok, ssum, 1.0)), NEG_INF)
            o = (e @ vh[j]) / np.where(ok, ssum, 1.0)[:, None]
            out[rows, h] = np.where(ok[:, None], o, 0.0)
    return out, lse


# ---------------------------------------------------------------------------
# Part 3: LSE merge
# ---------------------------------------------------------------------------

def merge(o1, lse1, o2, lse2):
    """Merge two partial attention results by their log-sum-exp.

    Online Softmax Merge (nano-vllm CLAUDE.md, merge_attention_outputs):
    m = max(lse1, lse2), e_i = exp(lse_i - m), lse = m + log(e1 + e2),
    o = (o1 e1 + o2 e2) / (e1 + e2).  Both -inf gives o = 0, lse = -inf.

    o: [Lq, H, d]; lse: [H, Lq].
    """
    o1 = np.asarray(o1, dtype=np.float64)
    o2 = np.asarray(o2, dtype=np.float64)
    lse1 = np.asarray(lse1, dtype=np.float64)
    lse2 = np.asarray(lse2, dtype=np.float64)
    m = np.maximum(lse1, lse2)
    ok = np.isfinite(m)
    m0 = np.where(ok, m, 0.0)
    e1 = np.where(np.isfinite(lse1), np.exp(np.where(np.isfinite(lse1), lse1, 0.0) - m0), 0.0)
    e2 = np.where(np.isfinite(lse2), np.exp(np.where(np.isfinite(lse2), lse2, 0.0) - m0), 0.0)
    den = np.where(ok, e1 + e2, 1.0)
    lse = np.where(ok, m0 + np.log(den), NEG_INF)
    w1 = (e1 / den).T[:, :, None]
    w2 = (e2 / den).T[:, :, None]
    o = np.where(ok.T[:, :, None], o1 * w1 + o2 * w2, 0.0)
    return o, lse


# ---------------------------------------------------------------------------
# 128-token block mask -> 1024-token cache blocks
# ---------------------------------------------------------------------------

def mask_to_cache_blocks(mask, kb_begin: int, n_cache_blocks: int, sub_blocks: int = 8,
                         force_first_last: bool = True):
    """Reduce a block mask to cache blocks of sub_blocks 128-token blocks.

    Task plan, "select_blocks 设计" step 3 (keep a cache block if any of its
    eight 128-token blocks is selected) and XAttentionBSAPolicy
    ``select_blocks`` step 6 (union over heads and query blocks, then the
    first and last history block are always included).  The last cache block
    may be partial (fewer columns than sub_blocks remain).

    mask: [H, nQB, nCols]; cache block cb covers mask columns
    kb_begin + cb*sub_blocks ... (clipped to nCols).
    Returns (keep_per_head uint8 [H, nQB, n_cache_blocks], keep_any uint8 [n_cache_blocks]).
    """
    mask = np.asarray(mask).astype(bool)
    H, nQB, nCols = mask.shape
    per = np.zeros((H, nQB, n_cache_blocks), dtype=np.uint8)
    for cb in range(n_cache_blocks):
        c0 = kb_begin + cb * sub_blocks
        c1 = min(c0 + sub_blocks, nCols)
        if c1 > c0:
            per[:, :, cb] = mask[:, :, c0:c1].any(axis=2)
    keep_any = per.reshape(H * nQB, n_cache_blocks).any(axis=0).astype(np.uint8)
    if force_first_last and n_cache_blocks > 0:
        keep_any[0] = 1
        keep_any[n_cache_blocks - 1] = 1
    return per, keep_any


def expand_cache_keep(keep_any, sub_blocks: int, n_cols: int) -> np.ndarray:
    """128-token-block view of a cache-block keep vector (column kb kept iff its cache block is)."""
    keep_any = np.asarray(keep_any).astype(np.uint8)
    return np.array([keep_any[kb // sub_blocks] for kb in range(n_cols)], dtype=np.uint8)


# ---------------------------------------------------------------------------
# Composition: chunked prefill of one layer
# ---------------------------------------------------------------------------

def chunk_prefill(q_chunk, k_prefix, v_prefix, q_start_pos: int, stride: int,
                  threshold: float, block: int = 128, softmax_scale=None, rule: str = "greedy"):
    """One query chunk of chunked prefill.

    XAttentionBSAPolicy ``select_blocks`` + ``compute_chunked_prefill``:
    estimate against K[0 : p+C]; attend the history [0, p) without the
    causal rule and the chunk's own keys [p, p+C) with it, each restricted to
    the selected blocks; merge the two partials by LSE.
    Returns dict(out, lse, scores, mask).
    """
    p = q_start_pos
    Lq = q_chunk.shape[0]
    scores, mask = estimate(q_chunk, k_prefix[:p + Lq], p, stride, threshold, block, rule)
    o_c, l_c = bsa(q_chunk, k_prefix[p:p + Lq], v_prefix[p:p + Lq], p, p, mask, 0,
                   True, softmax_scale, block)
    if p > 0:
        o_h, l_h = bsa(q_chunk, k_prefix[:p], v_prefix[:p], p, 0, mask, 0, False,
                       softmax_scale, block)
        out, lse = merge(o_h, l_h, o_c, l_c)
    else:
        out, lse = o_c, l_c
    return dict(out=out, lse=lse, scores=scores, mask=mask)


def chunked_prefill(q, k, v, chunk: int, stride: int, threshold: float, block: int = 128,
                    softmax_scale=None, rule: str = "greedy"):
    """Whole-layer chunked prefill: every chunk of ``chunk`` tokens in order."""
    L = q.shape[0]
    outs, lses, scores, masks = [], [], [], []
    for p in range(0, L, chunk):
        r = chunk_prefill(q[p:p + chunk], k, v, p, stride, threshold, block, softmax_scale, rule)
        outs.append(r["out"])
        lses.append(r["lse"])
        scores.append(r["scores"])
        masks.append(r["mask"])
    return dict(out=np.concatenate(outs, axis=0), lse=np.concatenate(lses, axis=1),
                scores=scores, masks=masks)


def density(mask, q_start_pos: int, block: int = 128) -> float:
    """Selected / causal block count of one chunk's mask.

    XAttentionBSAPolicy ``select_blocks`` step 5 (selected ∩ causal over the
    causal count).
    """
    mask = np.asarray(mask).astype(bool)
    H, nQB, nKB = mask.shape
    cur = q_start_pos // block
    causal = np.arange(nKB)[None, :] <= (cur + np.arange(nQB))[:, None]
    return float((mask & causal[None]).sum()) / float(causal.sum() * H)


def density_counts(mask) -> tuple[int, int]:
    """(selected, total) block counts of one chunk's mask, as integers.

    XAttentionBSAPolicy ``select_blocks`` step 5: the mask is [H, valid query
    blocks, valid key blocks]; the query blocks sit at the end of the keys
    (offset = key blocks - query blocks), a (query block, key block) pair is
    causal iff its key block is at most the query block plus that offset; the
    total is the causal pair count times the head count, the selected count the
    mask's kept pairs among them.
    """
    mask = np.asarray(mask).astype(bool)
    H, nQB, nKB = mask.shape
    q_offset = nKB - nQB
    causal = np.arange(nKB)[None, :] <= (np.arange(nQB)[:, None] + q_offset)
    total = int(causal.sum()) * H
    selected = int((mask & causal[None]).sum())
    return selected, total


def comm_density_counts(keep_any) -> tuple[int, int]:
    """(selected, available) cache-block counts of one chunk.

    XAttentionBSAPolicy ``select_blocks`` after step 6: the cache blocks to
    load (the union keep list, first and last already forced) over the cache
    blocks the history holds.
    """
    keep_any = np.asarray(keep_any).astype(bool)
    return int(keep_any.sum()), int(keep_any.size)


# ---------------------------------------------------------------------------
# Next step: the estimate against downsampled history keys (metadata of
# offloaded K)
# ---------------------------------------------------------------------------

def downsample_keys(k, stride: int) -> np.ndarray:
    """Task plan, "Metadata 存储策略", scheme A (``on_prefill_offload``): of
    each offloaded block keep every stride-th key token, K[::stride].

    k: [n, Hkv, d] -> [ceil(n / stride), Hkv, d].
    """
    return np.asarray(k)[::stride]


def estimate_history_downsampled(q, k_ds, stride: int, threshold: float, block: int = 128,
                                 rule: str = "greedy"):
    """Block scores and mask of a query chunk against the downsampled history.

    Task plan, "Phase 3: select_blocks 实现": the chunked estimate is run with
    stride 1 on (Q, K[::stride]) with block size block / stride, so a block of
    the downsampled key axis stands for one block-token block of the history
    and the query axis is cut into blocks of block / stride tokens.  At
    stride 1 the logits are q.k / sqrt(d) per (query token, downsampled key);
    each row is normalised over all history keys (all precede the chunk) and
    the probabilities are summed over (block/stride x block/stride) tiles.
    Selection per row as ``select_row`` with block 0 the only forced block
    (the chunk's diagonal block lies past the history keys).

    q: [Lq, Hq, d]; k_ds: [n_ds, Hkv, d].
    Returns (scores [Hq, Lq / b, n_ds / b], mask uint8 of the same shape), b = block / stride.
    """
    q = np.asarray(q, dtype=np.float64)
    k_ds = np.asarray(k_ds, dtype=np.float64)
    Lq, Hq, d = q.shape
    n_ds, Hkv, _ = k_ds.shape
    b = block // stride
    assert block % stride == 0 and Lq % b == 0 and n_ds % b == 0
    g = Hq // Hkv
    scores = []
    for h in range(Hq):
        z = q[:, h] @ k_ds[:, h // g].T / math.sqrt(d)
        prob, _, _ = row_softmax_causal(z, np.ones_like(z, dtype=bool))
        scores.append(block_sums(prob, b, 1))
    scores = np.stack(scores)
    mask = np.zeros(scores.shape, dtype=np.uint8)
    for h in range(Hq):
        for qb in range(scores.shape[1]):
            mask[h, qb] = select_row(scores[h, qb], [0], threshold, rule)
    return scores, mask


def history_cache_blocks_downsampled(mask, n_cache_blocks: int, sub_blocks: int = 8) -> np.ndarray:
    """Task plan, "Phase 3: select_blocks 实现" steps 5-6: OR of the mask over
    heads and query blocks, then a cache block of sub_blocks 128-token blocks
    is kept when any of them is (no forced first / last block in this sketch).

    mask: [Hq, nQB, n_blocks] -> keep uint8 [n_cache_blocks].
    """
    return mask_to_cache_blocks(mask, 0, n_cache_blocks, sub_blocks, force_first_last=False)[1]


# ---------------------------------------------------------------------------
# Next step: a packed batch of sequences (varlen)
# ---------------------------------------------------------------------------

def prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, stride: int, threshold: float, block: int = 128,
                   softmax_scale=None, rule: str = "greedy"):
    """GPU-only prefill of a packed batch, one sequence at a time.

    XAttentionBSAPolicy ``compute_prefill``: Q, K, V packed sequence after
    sequence with cumulative lengths; for a sequence, the estimate of its
    queries against its keys (causal, queries at the end of the keys:
    q_start_pos = k_len - q_len), the selection, and block-sparse causal
    attention with that mask.  The page handles one sequence and falls back
    to dense attention for more; here every sequence runs the same method
    on its own rows and keys.

    q: [total_q, Hq, d]; k, v: [total_k, Hkv, d]; cu_seqlens_*: [batch + 1].
    Returns dict(out [total_q, Hq, d], lse (list of [Hq, q_len_b]),
    scores, masks (lists of [Hq, q_len_b/block, k_len_b/block])).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    out = np.zeros(q.shape)
    lses, scores, masks = [], [], []
    for b in range(len(cq) - 1):
        qb, kb, vb = q[cq[b]:cq[b + 1]], k[ck[b]:ck[b + 1]], v[ck[b]:ck[b + 1]]
        p = kb.shape[0] - qb.shape[0]
        if qb.shape[0] == 0:
            lses.append(np.zeros((q.shape[1], 0)))
            scores.append(np.zeros((q.shape[1], 0, kb.shape[0] // block)))
            masks.append(np.zeros((q.shape[1], 0, kb.shape[0] // block), dtype=np.uint8))
            continue
        sc, m = estimate(qb, kb, p, stride, threshold, block, rule)
        o, lse = bsa(qb, kb, vb, p, 0, m, 0, True, softmax_scale, block)
        out[cq[b]:cq[b + 1]] = o
        lses.append(lse)
        scores.append(sc)
        masks.append(m)
    return dict(out=out, lse=lses, scores=scores, masks=masks)
