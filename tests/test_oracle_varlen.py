"""Pins of the oracle's packed-batch (varlen) prefill.

* threshold 1 keeps every causal block, so each sequence's output and LSE
  equal dense causal attention of its own queries (at the end of its own
  keys) from torch: SDPA with an explicit bottom-right causal mask for the
  output, logsumexp of the explicit scores for the LSE (library routines,
  not the oracle's formula), GQA by head index;
* no attention across sequences: changing another sequence's keys and
  values leaves a sequence's output, LSE and mask unchanged;
* order: reversing the sequences of the batch reverses the per-sequence
  results;
* a sequence with no queries contributes nothing and shifts nothing.
"""
import math

import numpy as np
import torch

from oracle import xattn_oracle as O

LENS = [(256, 512), (128, 128), (384, 896)]   # (q_len, k_len) per sequence


def _batch(seed, lens=LENS, hq=4, hkv=2, d=16):
    rng = np.random.default_rng(seed)
    cq = np.cumsum([0] + [a for a, _ in lens])
    ck = np.cumsum([0] + [b for _, b in lens])
    q = rng.standard_normal((cq[-1], hq, d))
    k = rng.standard_normal((ck[-1], hkv, d))
    v = rng.standard_normal((ck[-1], hkv, d))
    return q, k, v, cq, ck


def test_threshold_one_is_dense_causal_per_sequence():
    q, k, v, cq, ck = _batch(0)
    r = O.prefill_varlen(q, k, v, cq, ck, 8, 1.0)
    hq, hkv, d = q.shape[1], k.shape[1], q.shape[2]
    for b in range(len(cq) - 1):
        qb = torch.from_numpy(q[cq[b]:cq[b + 1]])
        kb = torch.from_numpy(k[ck[b]:ck[b + 1]])
        vb = torch.from_numpy(v[ck[b]:ck[b + 1]])
        Lq, Lk = qb.shape[0], kb.shape[0]
        allowed = torch.arange(Lk)[None, :] <= (Lk - Lq + torch.arange(Lq))[:, None]
        for h in range(hq):
            kh, vh = kb[:, h // (hq // hkv)], vb[:, h // (hq // hkv)]
            o = torch.nn.functional.scaled_dot_product_attention(qb[None, None, :, h], kh[None, None], vh[None, None],
                                                                 attn_mask=allowed[None, None])[0, 0]
            np.testing.assert_allclose(r["out"][cq[b]:cq[b + 1], h], o.numpy(), rtol=1e-10, atol=1e-12)
            z = (qb[:, h] @ kh.T) / math.sqrt(d)
            lse = torch.logsumexp(z.masked_fill(~allowed, -math.inf), dim=1)
            np.testing.assert_allclose(r["lse"][b][h], lse.numpy(), rtol=1e-12, atol=1e-12)


def test_no_attention_across_sequences():
    q, k, v, cq, ck = _batch(1)
    a = O.prefill_varlen(q, k, v, cq, ck, 8, 0.9)
    k2, v2 = k.copy(), v.copy()
    k2[ck[0]:ck[1]] += 3.0                       # disturb sequence 0 only
    v2[ck[0]:ck[1]] *= -2.0
    b = O.prefill_varlen(q, k2, v2, cq, ck, 8, 0.9)
    for s in (1, 2):
        np.testing.assert_array_equal(a["out"][cq[s]:cq[s + 1]], b["out"][cq[s]:cq[s + 1]])
        np.testing.assert_array_equal(a["lse"][s], b["lse"][s])
        np.testing.assert_array_equal(a["masks"][s], b["masks"][s])
    assert not np.allclose(a["out"][cq[0]:cq[1]], b["out"][cq[0]:cq[1]])


def test_reversed_batch_reverses_results():
    q, k, v, cq, ck = _batch(2)
    a = O.prefill_varlen(q, k, v, cq, ck, 8, 0.9)
    n = len(cq) - 1
    qr = np.concatenate([q[cq[s]:cq[s + 1]] for s in reversed(range(n))])
    kr = np.concatenate([k[ck[s]:ck[s + 1]] for s in reversed(range(n))])
    vr = np.concatenate([v[ck[s]:ck[s + 1]] for s in reversed(range(n))])
    cqr = np.cumsum([0] + [cq[s + 1] - cq[s] for s in reversed(range(n))])
    ckr = np.cumsum([0] + [ck[s + 1] - ck[s] for s in reversed(range(n))])
    b = O.prefill_varlen(qr, kr, vr, cqr, ckr, 8, 0.9)
    for s in range(n):
        t = n - 1 - s
        np.testing.assert_array_equal(a["out"][cq[s]:cq[s + 1]], b["out"][cqr[t]:cqr[t + 1]])
        np.testing.assert_array_equal(a["masks"][s], b["masks"][t])


def test_sequence_without_queries():
    lens = [(256, 512), (0, 384), (128, 256)]
    q, k, v, cq, ck = _batch(3, lens)
    r = O.prefill_varlen(q, k, v, cq, ck, 8, 0.9)
    assert r["lse"][1].shape == (4, 0) and r["masks"][1].shape == (4, 0, 3)
    alone = O.prefill_varlen(q[cq[2]:], k[ck[2]:], v[ck[2]:], [0, 128], [0, 256], 8, 0.9)
    np.testing.assert_array_equal(r["out"][cq[2]:], alone["out"])
    np.testing.assert_array_equal(r["masks"][2], alone["masks"][0])
