"""Seeded synthetic long-context Q/K/V for XAttention prefill.

This module only draws random tensors; it holds none of the method's
arithmetic.  It serves both the parity tests (which feed the same tensors to
the CPU checker and to the HIP library) and the benchmark.

Two recipes:

* ``tiny``: Q [L, Hq, d], K [L, Hkv, d], V [L, Hkv, d], each N(0, 1) in
  float32, drawn in that order from ``torch.Generator().manual_seed(seed)``.
* ``long_context``: a Llama-3.1-8B-shaped attention layer.  Per key/value
  head group:
    - Q = 0.5*N(0,1), K = 0.5*N(0,1);
    - a shared rank-4 component: basis U (4 x d, N(0,1) entries) and an
      AR(1) coefficient path c(t) (correlation exp(-1/256) between adjacent
      tokens, stationary std 0.35 per coefficient); K[t] += c(t) U and
      Q[t] += c(t) U + 0.1 * N(0,1) U per query head.  Nearby tokens share a
      positive score (a local band) and distant ones a slowly varying random
      one, so key blocks differ coherently in importance;
    - an attention sink: unit vector w; Q[t] += 5.8 w for all t,
      K[0:128] += 5.8 w (about +3 nats at 1/sqrt(128));
    - needles: each needle n picks a kv head group, a target query block
      qb_n >= 1, a key position k_n < 128*qb_n and a unit vector u_n;
      Q rows of block qb_n (all query heads of the group) += 5.8 u_n and
      K[k_n] += 11.6 u_n (about +6 nats);
    - V = N(0,1).
  Generated in float32 on the host and rounded to bfloat16 once.
"""

from __future__ import annotations

import math

import numpy as np
import torch


def tiny(seed: int = 0, L: int = 1024, hq: int = 2, hkv: int = 1, d: int = 64):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(L, hq, d, generator=g, dtype=torch.float32)
    k = torch.randn(L, hkv, d, generator=g, dtype=torch.float32)
    v = torch.randn(L, hkv, d, generator=g, dtype=torch.float32)
    return q, k, v


def _unit(g: torch.Generator, n: int, d: int) -> torch.Tensor:
    x = torch.randn(n, d, generator=g, dtype=torch.float64)
    return (x / x.norm(dim=1, keepdim=True)).to(torch.float32)


def _ar1(g: torch.Generator, L: int, n: int, corr: float, std: float) -> torch.Tensor:
    """AR(1) paths of length L for n coefficients, stationary std ``std``."""
    from scipy.signal import lfilter  # plain IIR filter for the recursion

    e = torch.randn(L, n, generator=g, dtype=torch.float64).numpy()
    e *= std * math.sqrt(1.0 - corr * corr)
    e[0] = e[0] / math.sqrt(1.0 - corr * corr)
    c = lfilter([1.0], [1.0, -corr], e, axis=0)
    return torch.from_numpy(np.ascontiguousarray(c)).to(torch.float32)


def long_context(L: int, hq: int, hkv: int, d: int = 128, n_needles: int = 16,
                 seed: int = 2, dtype: torch.dtype = torch.bfloat16, block: int = 128,
                 rank: int = 4):
    """Q [L, hq, d], K [L, hkv, d], V [L, hkv, d] in ``dtype`` (see module doc)."""
    assert hq % hkv == 0 and L % block == 0
    grp = hq // hkv
    g = torch.Generator().manual_seed(seed)
    q = 0.5 * torch.randn(L, hq, d, generator=g, dtype=torch.float32)
    k = 0.5 * torch.randn(L, hkv, d, generator=g, dtype=torch.float32)
    for kvh in range(hkv):
        u = torch.randn(rank, d, generator=g, dtype=torch.float32)  # [rank, d]
        c = _ar1(g, L, rank, math.exp(-1.0 / 256.0), 0.35)         # [L, rank]
        shared = c @ u                                          # [L, d]
        k[:, kvh] += shared
        for j in range(grp):
            noise = 0.1 * torch.randn(L, rank, generator=g, dtype=torch.float32)
            q[:, kvh * grp + j] += shared + noise @ u
    w = _unit(g, hkv, d)
    for kvh in range(hkv):
        q[:, kvh * grp:(kvh + 1) * grp] += 5.8 * w[kvh]
        k[:block, kvh] += 5.8 * w[kvh]
    n_qb = L // block
    if n_needles and n_qb > 1:
        for n in range(n_needles):
            kvh = n % hkv
            qb = int(torch.randint(1, n_qb, (1,), generator=g))
            kpos = int(torch.randint(0, qb * block, (1,), generator=g))
            un = _unit(g, 1, d)[0]
            q[qb * block:(qb + 1) * block, kvh * grp:(kvh + 1) * grp] += 5.8 * un
            k[kpos, kvh] += 11.6 * un
    v = torch.randn(L, hkv, d, generator=g, dtype=torch.float32)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def packed_batch(lengths, hq: int, hkv: int, d: int = 128, n_needles: int = 16, seed: int = 6):
    """A packed batch of whole prompts: sequence i is ``long_context(lengths[i], ..., seed + i)``.

    Returns Q [total, hq, d], K, V [total, hkv, d] (sequences one after the other) and the cumulative
    lengths [batch + 1] (the same for queries and keys).
    """
    qs, ks, vs = [], [], []
    for i, n in enumerate(lengths):
        q, k, v = long_context(n, hq, hkv, d, n_needles, seed + i)
        qs.append(q)
        ks.append(k)
        vs.append(v)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    return torch.cat(qs), torch.cat(ks), torch.cat(vs), cu


# Named workloads (token counts, heads, head_dim, chunking, estimate settings).
WORKLOADS = {
    "tiny_1k_fp32": dict(L=1024, hq=2, hkv=1, d=64, chunk=1024, stride=8, threshold=0.9,
                         dtype="f32", seed=0),
    "llama8b_32k_8x4k": dict(L=32768, hq=32, hkv=8, d=128, chunk=4096, stride=8,
                             threshold=0.95, dtype="bf16", seed=2, n_needles=16),
    "llama8b_128k_last_chunk": dict(L=131072, hq=32, hkv=8, d=128, chunk=4096, stride=8,
                                    threshold=0.9, dtype="bf16", seed=3, n_needles=16,
                                    q_start_pos=126976, cache_block=1024),
    "llama8b_64k_sweep": dict(L=65536, hq=32, hkv=8, d=128, chunk=4096,
                              strides=(8, 16), thresholds=(0.8, 0.9, 0.95, 0.99, 1.0),
                              dtype="bf16", seed=4, n_needles=16),
    "gqa7_128k_32x4k": dict(L=131072, hq=28, hkv=4, d=128, chunk=4096, stride=8,
                            threshold=0.9, dtype="bf16", seed=5, n_needles=64),
    # packed batch of whole prompts (GPU-only prefill of several sequences at once)
    "llama8b_varlen_8seq": dict(lengths=(16384, 12288, 8192, 4096, 4096, 2048, 1024, 1024), hq=32, hkv=8,
                                d=128, stride=8, threshold=0.95, dtype="bf16", seed=6, n_needles=16,
                                varlen=True),
}


def workload_inputs(name: str, L: int | None = None):
    """Q, K, V for a named workload (optionally truncated to the first L tokens)."""
    w = WORKLOADS[name]
    if w.get("varlen"):
        q, k, v, _ = packed_batch(w["lengths"], w["hq"], w["hkv"], w["d"], w.get("n_needles", 16), w["seed"])
        return q, k, v
    if w["dtype"] == "f32":
        return tiny(w["seed"], w["L"], w["hq"], w["hkv"], w["d"])
    n = w["L"] if L is None else L
    return long_context(n, w["hq"], w["hkv"], w["d"], w.get("n_needles", 16), w["seed"])
