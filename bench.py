"""Benchmark: XAttention block-sparse chunked prefill of one attention layer on one MI355X.

Step = the whole hot path over one layer's prefill: for every 4096-token
chunk, pack the chunk's V rows, estimate block scores and the block mask,
block-sparse attention over the history and over the chunk, LSE merge.
Inputs are seeded synthetic tensors already resident in HBM.

Prints one JSON line.  Extra fields: per-part times, mask density,
effective TFLOP/s on computed blocks, the attention kernel's roofline entry
(HIP events around every attention launch in the timed region) and the CPU
oracle timed on one key/value-head group of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--stride S] [--threshold T] [--no-cpu-baseline]
  python bench.py --workload llama8b_64k_sweep --sweep   # one line per (stride, threshold)
  python bench.py --copy-mib N   # plain device copy of N MiB (HBM counter calibration)
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_xattn_amd", "csrc", "bsa.hip")

# HBM bytes per attention launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# passes over this bench (profiles/ holds the summaries and the commands),
# scaled by the same counters' reading for a plain copy of known size.  Valid
# only for the attention code they were taken on (source_sha of bsa.hip: its code without comments).
TRAFFIC = {
    "llama8b_32k_8x4k": [
        {"bsa_code_sha256": "6d816bdc561e74ce02b5ef8660bd3174e7864ee27c5de32b2b2fdd7953965947",
         "stride": 8, "threshold": 0.95, "fused": False,
         "hbm_bytes_per_launch": 1.0083e9},   # fetch 9.359e8 (x1.9999) + write 7.24e7 (x1.0), mean of 8 chunks
    ],
    "llama8b_128k_last_chunk": [
        {"bsa_code_sha256": "6d816bdc561e74ce02b5ef8660bd3174e7864ee27c5de32b2b2fdd7953965947",
         "stride": 8, "threshold": 0.9, "fused": False,
         "hbm_bytes_per_launch": 8.9808e9},   # fetch 8.9043e9 (x1.9999) + write 7.66e7 (x1.0)
    ],
    "llama8b_varlen_8seq": [
        {"bsa_code_sha256": "6d816bdc561e74ce02b5ef8660bd3174e7864ee27c5de32b2b2fdd7953965947",
         "stride": 8, "threshold": 0.95, "fused": False,
         "hbm_bytes_per_launch": 6.3071e9},   # fetch 5.8476e9 (x1.9999) + write 4.595e8 (x1.0), head-pair form
    ],
    "gqa7_128k_32x4k": [
        {"bsa_code_sha256": "6d816bdc561e74ce02b5ef8660bd3174e7864ee27c5de32b2b2fdd7953965947",
         "stride": 8, "threshold": 0.9, "fused": False,
         "hbm_bytes_per_launch": 3.3164e9},   # fetch 3.2576e9 (x1.9999) + write 5.88e7 (x1.0), mean of 32 chunks
    ],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama8b_32k_8x4k")
    ap.add_argument("--stride", type=int, default=None, help="override the workload's stride")
    ap.add_argument("--threshold", type=float, default=None, help="override the workload's threshold")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-groups", type=int, default=1, help="kv-head groups timed for the CPU baseline")
    ap.add_argument("--copy-mib", type=int, default=0, help="only run a plain device copy of this many MiB")
    ap.add_argument("--sweep", action="store_true", help="every (stride, threshold) of the workload, one line each")
    ap.add_argument("--estimator", choices=("full", "downsampled"), default="full",
                    help="downsampled: cache blocks chosen from K[::stride] of the history (cache-block workloads); "
                         "with --offload, full streams the host-resident history K through the ring")
    ap.add_argument("--offload", action="store_true",
                    help="history K/V in pinned host cache blocks, kept blocks copied back through a device ring")
    ap.add_argument("--group", type=int, default=8, help="cache blocks per ring group (offload)")
    ap.add_argument("--default-events", action="store_true",
                    help="time with torch's default events (system-scope fence at every record) instead of "
                         "timing-only events")
    ap.add_argument("--no-sub", action="store_true",
                    help="the 32K line without its 128K sub-records (last chunk with cache blocks; 28/4-head layer)")
    ap.add_argument("--fused", action="store_true",
                    help="time each chunk's history + chunk attention as one causal pass (no partials, no merge); "
                         "by default a step is the pages' composition (two segments, LSE merge)")
    return ap.parse_args()


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: recording it performs no system-scope
    cache writeback / invalidate (the HIP runtime documents the flag for timing events; a default event's fence
    would cool the caches for the next kernel and stretch the interval).  Interface as torch.cuda.Event's
    record / elapsed_time; `cuda_event` is the raw handle (the library's measurement hook takes it)."""
    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence (timing stays enabled)

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            import re
            import torch  # noqa: F401  (loads the HIP runtime torch and the library share)
            maps = open("/proc/self/maps").read()
            paths = sorted(set(re.findall(r"(/\S*libamdhip64\.so\S*)", maps)))
            lib = ctypes.CDLL(paths[0] if paths else "libamdhip64.so")
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    def __init__(self, enable_timing=True):
        import ctypes
        h = ctypes.c_void_p()
        st = self.hip().hipEventCreateWithFlags(ctypes.byref(h), self.FLAGS)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")
        self.cuda_event = h.value

    def __del__(self):
        if self._hip is not None and getattr(self, "cuda_event", None):
            self._hip.hipEventDestroy(self.cuda_event)
            self.cuda_event = None

    def record(self, stream):
        st = self.hip().hipEventRecord(self.cuda_event, stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        st = self.hip().hipEventElapsedTime(ctypes.byref(ms), self.cuda_event, end.cuda_event)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value


def timing_event():
    import torch
    return torch.cuda.Event(enable_timing=True) if DEFAULT_EVENTS else TimingEvent()


DEFAULT_EVENTS = False


def copy_probe(mib):
    """A plain device-to-device copy of known size, five times (counter calibration)."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}))


def source_sha(path):
    """sha256 of a C++ source's code: '//' comments, trailing blanks and blank lines removed, so that an edit of
    comments alone (identical device code) keeps a traffic record valid."""
    lines = []
    with open(path, encoding="utf-8") as f:
        for ln in f:
            code = ln.split("//", 1)[0].rstrip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def count_flops(run):
    """Algorithmic work of one step from the step's own block masks.

    attention: 4*d*128^2 flop per computed (head, query block, key block) tile
    (QK^T and PV), diagonal tiles counted whole; estimate: 2*(d*S) flop per
    visible (reshaped row, reshaped column) pair.
    Returns (attention flops per launch in launch order, estimate flops,
    density, attention flops split {history, in_chunk, useful}); "useful"
    counts only the causally allowed (query, key) pairs of the computed tiles.
    """
    import numpy as np
    d, S, blk = run.d, run.stride, run.block
    per_tile = 4.0 * d * blk * blk
    fused = run.q.dtype.is_floating_point and run.q.element_size() == 2 and d == 128
    launches = []
    split = {"history": 0.0, "in_chunk": 0.0, "useful": 0.0}
    est = 0.0
    sel = tot = 0
    ds = getattr(run, "estimator", "full") == "downsampled"
    for b in run.bufs:
        if ds:
            # estimate against K[::S] of the history; history attention over the kept cache blocks
            hq, nqb = run.hq, min(run.chunk, run.L - b.p) // blk
            parts = [("in_chunk", per_tile * hq * nqb * (nqb + 1) / 2)]
            if b.p > 0:
                kept = int(b.keep_any_blocks.cpu().numpy().astype(bool).sum())
                parts.insert(0, ("history", per_tile * kept * hq * nqb))
                est += 2.0 * d * (nqb * blk) * (b.p // S) * hq
                sel += kept * hq * nqb
            sel += hq * nqb * (nqb + 1) // 2
            tot += hq * nqb * (b.p // blk) + hq * nqb * (nqb + 1) // 2
            for kind, f in parts:
                split[kind] += f
            split["useful"] += sum(f for _, f in parts) - per_tile * hq * nqb * (1.0 - (blk + 1) / (2.0 * blk))
            launches.append(sum(f for _, f in parts))
            continue
        m = b.mask.cpu().numpy().astype(bool)
        hq, nqb, nkb = m.shape
        cur = b.p // blk
        parts = []
        if b.p > 0:
            if b.keep_any_blocks is not None:
                kept = int(b.keep_any_blocks.cpu().numpy().astype(bool).sum())
                parts.append(("history", per_tile * kept * hq * nqb))
            else:
                parts.append(("history", per_tile * float(m[:, :, :cur].sum())))
        if b.keep_any_blocks is not None:
            parts.append(("in_chunk", per_tile * hq * nqb * (nqb + 1) / 2))
        else:
            parts.append(("in_chunk", per_tile * float(m[:, :, cur:].sum())))
        for kind, f in parts:
            split[kind] += f
        # in-chunk diagonal tiles hold 128*129/2 allowed pairs of 128*128
        n_diag = hq * nqb
        split["useful"] += sum(f for _, f in parts) - per_tile * n_diag * (1.0 - (blk + 1) / (2.0 * blk))
        if fused:
            launches.append(sum(f for _, f in parts))
        else:
            launches.extend(f for _, f in parts)
        causal = np.arange(nkb)[None, :] <= (cur + np.arange(nqb))[:, None]
        sel += int((m & causal[None]).sum())
        tot += int(causal.sum()) * hq
        R = nqb * blk // S
        cdiag = b.p // S
        vis = float(np.sum(cdiag + np.arange(R) + 1))
        est += 2.0 * d * S * vis * hq
    return launches, est, sel / max(tot, 1), split


def measured_gemm_peak():
    """Dense bf16 GEMM rate of the platform library on this GPU (torch.mm, 8192^3, contiguous operands): the
    best dense matrix rate measured on the same GPU, reported beside the 2.5 PFLOP/s spec figure."""
    import torch
    n = 8192
    a = torch.randn(n, n, device="cuda:0").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda:0").to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda:0", dtype=torch.bfloat16)
    for _ in range(3):
        torch.mm(a, b, out=c)
    stream = torch.cuda.current_stream()
    e0, e1 = timing_event(), timing_event()
    reps = 20
    e0.record(stream)
    for _ in range(reps):
        torch.mm(a, b, out=c)
    e1.record(stream)
    torch.cuda.synchronize()
    tflops = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    return {"tflops": round(tflops, 1), "how": "torch.mm bf16 8192x8192x8192 (hipBLASLt), 20 timed calls"}


def cpu_baseline(name, groups, w):
    """Time the oracle on `groups` kv-head groups of the workload.

    Every chunk is timed when there are at most 8; otherwise chunks {first,
    middle, last} are timed and the per-chunk time, linear in the history
    length p (estimate and attention both scale with p + C), is fitted by least
    squares and summed over all chunks.
    """
    import numpy as np
    from block_sparse_attention_xattn_amd import synthetic
    from oracle import xattn_oracle as O
    q, k, v = synthetic.workload_inputs(name)
    g = w["hq"] // w["hkv"]
    hs = list(range(groups * g))
    f = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    qs, ks, vs = f(q[:, hs]), f(k[:, :groups]), f(v[:, :groups])
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    c = w["chunk"]
    starts = [w["q_start_pos"]] if "q_start_pos" in w else list(range(0, w["L"], c))
    sample = starts if len(starts) <= 8 else [starts[0], starts[len(starts) // 2], starts[-1]]
    times = []
    for p in sample:
        t0 = time.perf_counter()
        O.chunk_prefill(qs[p:p + c], ks, vs, p, w["stride"], w["threshold"])
        times.append(time.perf_counter() - t0)
    if len(sample) == len(starts):
        total = sum(times)
        how = f"all {len(starts)} chunk(s) timed"
    else:
        b1, b0 = np.polyfit(np.array(sample, dtype=np.float64), np.array(times), 1)
        total = float(sum(b0 + b1 * p for p in starts))
        how = (f"chunks at p = {sample} timed ({sum(times):.1f} s), per-chunk time fitted linearly in p and summed "
               f"over all {len(starts)} chunks")
    frac = groups / w["hkv"]
    value = len(starts) * c * frac / total
    return {"value": round(value, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 numpy oracle (chunk_prefill: estimate, selection, sparse history and in-chunk "
                      f"attention, merge) for {groups} of {w['hkv']} kv-head groups ({len(hs)} of {w['hq']} query "
                      f"heads); {how}; tokens/s scaled by the head fraction (heads are independent); "
                      f"{sum(times):.1f} s of CPU time"}


def varlen_flops(run):
    """(attention computed-block flops, estimate flops, density) of a packed-batch step from its masks."""
    import numpy as np
    d, S, blk = run.d, run.stride, run.block
    per_tile = 4.0 * d * blk * blk
    att = est = 0.0
    sel = tot = 0
    for b, m in enumerate(run.masks()):
        ql, kl = run.cu_q[b + 1] - run.cu_q[b], run.cu_k[b + 1] - run.cu_k[b]
        if ql == 0:
            continue
        m = m.cpu().numpy().astype(bool)
        hq, nqb, nkb = m.shape
        cur = (kl - ql) // blk
        causal = np.arange(nkb)[None, :] <= (cur + np.arange(nqb))[:, None]
        n = int((m & causal[None]).sum())
        att += per_tile * n
        sel += n
        tot += int(causal.sum()) * hq
        R = ql // S
        est += 2.0 * d * S * float(np.sum((kl - ql) // S + np.arange(R) + 1)) * hq
    return att, est, sel / max(tot, 1)


def measure_varlen(a, w, q, k, v):
    """Packed batch: one pack + estimate + attention per step over every sequence; also the same calls made
    sequence by sequence (single-sequence entry points) on the same inputs, for comparison."""
    import torch
    from block_sparse_attention_xattn_amd import binding as B
    from block_sparse_attention_xattn_amd.varlen import VarlenPrefill
    cu = [0]
    for n in w["lengths"]:
        cu.append(cu[-1] + n)
    S, tau = w["stride"], w["threshold"]
    run = VarlenPrefill(q, k, v, cu, cu, S, tau)
    for _ in range(a.warmup):
        run.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # every event is created before the timed region (creating one can stall the host)
    ev_pool = [[timing_event() for _ in range(6)] for _ in range(a.steps)]
    for e in ev_pool:  # torch creates an event at its first record
        for x in e:
            x.record(stream)
    torch.cuda.synchronize()
    ev = []
    t0 = time.perf_counter()
    for st in range(a.steps):
        e = ev_pool[st]
        e[0].record(stream)
        run.pack()
        e[1].record(stream)
        run.estimate()
        e[2].record(stream)
        B.xattn_set_attention_events(e[4], e[5])  # the library records these around the attention kernel
        run.attend()
        e[3].record(stream)
        ev.append(e)
    B.xattn_set_attention_events(None, None)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / a.steps
    pack_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / a.steps
    est_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / a.steps
    att_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / a.steps
    kern_ms = sum(e[4].elapsed_time(e[5]) for e in ev) / a.steps
    att_f, est_f, dens = varlen_flops(run)

    # the same work as one call per sequence (buffers allocated up front)
    seqs = []
    for b in range(len(cu) - 1):
        n = cu[b + 1] - cu[b]
        qs, ks, vs = q[cu[b]:cu[b + 1]], k[cu[b]:cu[b + 1]], v[cu[b]:cu[b + 1]]
        pk = B.PackedV(n, run.hkv, run.d, q.dtype, q.device)
        nb = n // 128
        seqs.append(dict(q=qs, k=ks, v=vs, packed=pk,
                         sc=torch.empty(run.hq, nb, nb, dtype=torch.float32, device=q.device),
                         m=torch.empty(run.hq, nb, nb, dtype=torch.uint8, device=q.device),
                         ews=B.workspace(B.xattn_estimate_workspace_size(n, n, run.hq, run.hkv, run.d, S), q.device),
                         bws=B.workspace(B.bsa_prefill_packed_workspace_size(n, n, run.hq, run.hkv, run.d),
                                         q.device),
                         out=torch.empty_like(qs), lse=torch.empty(run.hq, n, dtype=torch.float32, device=q.device)))

    def loop():
        for x in seqs:
            B.bsa_pack_v(x["v"], x["packed"], 0)
            B.xattn_estimate(x["q"], x["k"], 0, S, tau, block_scores=x["sc"], block_mask=x["m"], ws=x["ews"])
            B.bsa_prefill_packed(x["q"], x["k"], x["packed"], 0, 0, 0, x["m"], 0, True, out=x["out"], lse=x["lse"],
                                 ws=x["bws"])
    for _ in range(a.warmup):
        loop()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        loop()
    torch.cuda.synchronize()
    loop_ms = (time.perf_counter() - t0) * 1e3 / a.steps
    tokens = cu[-1]
    achieved = att_f / (kern_ms * 1e-3) / 1e12
    # the library takes the head-pair form when the query heads per kv head are even (XATTN_PAIR=0 disables it);
    # the stored counter bytes are those of that form
    pair = (run.hq // run.hkv) % 2 == 0 and os.environ.get("XATTN_PAIR", "1") != "0"
    traffic = None
    for rec in TRAFFIC.get(a.workload, []):
        if pair and rec["bsa_code_sha256"] == source_sha(ATTN_SRC) and (rec["stride"], rec["threshold"]) == (S, tau):
            traffic = rec["hbm_bytes_per_launch"]
    return {
        "metric": "sparse prefill tokens/s per layer (estimate+BSA), packed batch of whole prompts",
        "value": round(tokens / (step_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(step_ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": a.workload, "lengths": list(w["lengths"]), "tokens": tokens, "q_heads": run.hq,
                   "kv_heads": run.hkv, "head_dim": run.d, "stride": S, "threshold": tau, "block": 128},
        "roofline": {"bound": "mfma",
                     "kernel": ("bsa_pair_kernel<128, bf16> packed-batch form (block-sparse attention, two query heads "
                                "per workgroup)" if pair else "bsa3_kernel<128, bf16> packed-batch form (block-sparse attention)"),
                     "achieved": round(achieved, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(achieved / 2500.0, 4), "traffic": traffic,
                     "avg_launch_ms": round(kern_ms, 4),
                     "timed_call": "the attention kernel alone (events the library records around its launch)"},
        "density": round(dens, 4),
        "parts_ms": {"pack": round(pack_ms, 3), "estimate": round(est_ms, 3), "attention": round(att_ms, 3),
                     "attention_kernel": round(kern_ms, 3)},
        "estimate_gflop": round(est_f / 1e9, 1), "bsa_gflop": round(att_f / 1e9, 1),
        "per_sequence_calls_ms_per_step": round(loop_ms, 3),
        "speedup_vs_per_sequence_calls": round(loop_ms / step_ms, 3),
    }


def cpu_baseline_varlen(w, groups):
    """The oracle's packed-batch prefill on `groups` kv-head groups of every sequence, scaled by the head
    fraction."""
    import numpy as np
    from block_sparse_attention_xattn_amd import synthetic
    from oracle import xattn_oracle as O
    q, k, v, cu = synthetic.packed_batch(w["lengths"], w["hq"], w["hkv"], w["d"], w.get("n_needles", 16), w["seed"])
    g = w["hq"] // w["hkv"]
    f = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    qs, ks, vs = f(q[:, :groups * g]), f(k[:, :groups]), f(v[:, :groups])
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    t0 = time.perf_counter()
    O.prefill_varlen(qs, ks, vs, cu, cu, w["stride"], w["threshold"])
    dt = time.perf_counter() - t0
    frac = groups / w["hkv"]
    return {"value": round(cu[-1] * frac / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 numpy oracle (prefill_varlen: estimate, selection, causal sparse attention of every "
                      f"sequence) for {groups} of {w['hkv']} kv-head groups ({groups * g} of {w['hq']} query heads) "
                      f"of all {len(w['lengths'])} sequences; tokens/s scaled by the head fraction (heads are "
                      f"independent); {dt:.1f} s of CPU time"}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark measures exactly one GPU; runs on several GPUs are not "
                                   "supported (the path shards by kv-head group with no exchange)",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    if a.copy_mib:
        copy_probe(a.copy_mib)
        return
    global DEFAULT_EVENTS
    DEFAULT_EVENTS = a.default_events
    # no garbage-collector pauses inside the timed regions; collected explicitly between measurements
    gc.disable()
    from block_sparse_attention_xattn_amd import synthetic

    base = dict(synthetic.WORKLOADS[a.workload])
    q, k, v = (t.to("cuda:0") for t in synthetic.workload_inputs(a.workload))
    if base.get("varlen"):
        w = dict(base)
        w["stride"] = a.stride if a.stride is not None else w["stride"]
        w["threshold"] = a.threshold if a.threshold is not None else w["threshold"]
        out = measure_varlen(a, w, q, k, v)
        if not a.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_varlen(w, a.cpu_groups)
        print(json.dumps(out))
        return
    if a.sweep:
        # every (stride, threshold) point of the workload on the same inputs, one line each
        for stride in base.get("strides", (base.get("stride", 8),)):
            for tau in base.get("thresholds", (base.get("threshold", 0.9),)):
                w = dict(base, stride=stride, threshold=tau)
                gc.collect()
                print(json.dumps(measure(a, w, q, k, v)), flush=True)
        return
    w = dict(base)
    w["stride"] = a.stride if a.stride is not None else w.get("stride", 8)
    w["threshold"] = a.threshold if a.threshold is not None else w.get("threshold", 0.9)
    out = measure_offload(a, w, q, k, v) if a.offload else measure(a, w, q, k, v)
    if not a.offload:
        gc.collect()
        peak = measured_gemm_peak()
        out["roofline"]["peak_measured"] = peak
        out["roofline"]["frac_of_measured"] = round(out["roofline"]["achieved"] / peak["tflops"], 4)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(a.workload, a.cpu_groups, w)
    subs = [] if (a.no_sub or a.offload or a.stride is not None or a.threshold is not None) else \
        [n for n in SUB_RECORDS.get(a.workload, ())]
    if subs:
        del q, k, v
        gc.collect()
        out["sub_records"] = {}
        for name in subs:
            out["sub_records"][name] = sub_record(a, name)
            gc.collect()
            torch_empty_cache()
    print(json.dumps(out))


# the metric is quoted at 32K and 128K: the 32K line also carries the 128K workloads, each measured the same way
SUB_RECORDS = {"llama8b_32k_8x4k": ("llama8b_128k_last_chunk", "gqa7_128k_32x4k")}


def torch_empty_cache():
    import torch
    torch.cuda.empty_cache()


def sub_record(a, name):
    """The measure() record of another workload (its own roofline, parts, density and CPU-oracle sample)."""
    from block_sparse_attention_xattn_amd import synthetic
    w = dict(synthetic.WORKLOADS[name])
    w["stride"] = w.get("stride", 8)
    w["threshold"] = w.get("threshold", 0.9)
    print(f"[bench] {name}: generating inputs", file=sys.stderr, flush=True)
    q, k, v = (t.to("cuda:0") for t in synthetic.workload_inputs(name))
    # the 32-chunk layer takes ~45 ms a step: fewer steps keep the run within the same time
    steps = a.steps if w["L"] // w["chunk"] <= 8 or "q_start_pos" in w else max(3, a.steps // 3)
    sa = argparse.Namespace(**{**vars(a), "steps": steps, "warmup": max(1, min(a.warmup, 2)), "workload": name})
    print(f"[bench] {name}: {steps} timed steps", file=sys.stderr, flush=True)
    rec = measure(sa, w, q, k, v)
    for key in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data"):
        rec.pop(key, None)
    del q, k, v
    if not a.no_cpu_baseline:
        print(f"[bench] {name}: CPU oracle sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(name, a.cpu_groups, w)
    return rec


def measure(a, w, q, k, v, fused=None):
    """Warm up, time a.steps steps of the workload w on resident q, k, v; return the JSON record."""
    if fused is None:
        fused = a.fused
    import torch
    from block_sparse_attention_xattn_amd.prefill import ChunkedPrefill
    starts = None
    if "q_start_pos" in w:
        starts = [w["q_start_pos"]]
    run = ChunkedPrefill(q, k, v, chunk=w["chunk"], stride=w["stride"], threshold=w["threshold"],
                         chunk_starts=starts, cache_block=w.get("cache_block"), estimator=a.estimator,
                         fused=fused)
    run.pack_history()
    torch.cuda.synchronize()
    for _ in range(a.warmup):
        run.run()
    torch.cuda.synchronize()

    from block_sparse_attention_xattn_amd import binding as B
    stream = torch.cuda.current_stream()
    ev = []
    # events are created before they are needed (creating one mid-run can stall the host)
    ev_pool = [timing_event() for _ in range(24 * len(run.bufs) * a.steps + 16)]

    def mark(tag):
        e = ev_pool.pop() if ev_pool else timing_event()
        e.record(stream)
        ev.append((tag, e))

    orig_est, orig_merge, orig_pack, orig_reduce = run.estimate, run.merge, run.pack, run.reduce
    orig_bsa, orig_seg = B.bsa_prefill_packed, B.bsa_prefill_segments

    # the ping-pong kernel (bf16, head_dim 128) is timed alone: the library records a pair of these events
    # immediately around its launch; other forms are timed by events around the whole call
    kernel_events = q.dtype == torch.bfloat16 and w["d"] == 128
    for e in ev_pool:  # torch creates an event at its first record
        e.record(stream)
    torch.cuda.synchronize()

    def wrap(fn, tag="bsa_launch"):
        def inner(*args, **kw):
            if kernel_events and tag == "bsa_launch":
                ea, eb = ev_pool.pop(), ev_pool.pop()
                B.xattn_set_attention_events(ea, eb)
                r = fn(*args, **kw)
                ev.append((tag + ":start", ea))
                ev.append((tag + ":end", eb))
                return r
            mark(tag + ":start")
            r = fn(*args, **kw)
            mark(tag + ":end")
            return r
        return inner

    def timed(tag, fn):
        def inner(b):
            mark(tag + ":start")
            fn(b)
            mark(tag + ":end")
        return inner

    # timed region: a.steps steps with events only around each attention call (each recorded event leaves the
    # GPU idle for a few microseconds between calls)
    B.bsa_prefill_packed, B.bsa_prefill_segments = wrap(orig_bsa), wrap(orig_seg)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0 = timing_event()
    e1 = timing_event()
    e0.record(stream)
    for _ in range(a.steps):
        run.run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    B.bsa_prefill_packed, B.bsa_prefill_segments = orig_bsa, orig_seg
    B.xattn_set_attention_events(None, None)
    gpu_ms = e0.elapsed_time(e1)
    step_ms = max(gpu_ms, wall * 1e3) / a.steps

    # then, untimed, the same steps with events around the other calls too, for their part of a step
    run.estimate = timed("estimate", orig_est)
    if not run.fused:
        run.merge = timed("merge", orig_merge)
    run.pack = timed("pack", orig_pack)
    run.reduce = timed("reduce", orig_reduce)
    B.bsa_prefill_packed, B.bsa_prefill_segments = wrap(orig_bsa, "bsa_call"), wrap(orig_seg, "bsa_call")
    for _ in range(a.steps):
        run.run()
    torch.cuda.synchronize()
    run.estimate, run.merge, run.pack, run.reduce = orig_est, orig_merge, orig_pack, orig_reduce
    B.bsa_prefill_packed, B.bsa_prefill_segments = orig_bsa, orig_seg

    parts = {}
    bsa_durs = []
    open_ev = {}
    for tag, e in ev:
        name, kind = tag.split(":")
        if kind == "start":
            open_ev[name] = e
        else:
            dt = open_ev.pop(name).elapsed_time(e)
            parts[name] = parts.get(name, 0.0) + dt
            if name == "bsa_launch":
                bsa_durs.append(dt)
    for kk in parts:
        parts[kk] /= a.steps

    launches, est_flops, _, split = count_flops(run)
    # compute and comm density from the library's counts over one more (untimed) step
    run.reset_density()
    run.track_density = True
    run.run()
    run.track_density = False
    dens_rec = run.density()
    # HBM-bound helpers: algorithmic bytes per call over their event time
    n_merge = sum(1 for b in run.bufs if b.p > 0)
    hbm = {}
    if n_merge and parts.get("merge"):
        c_len = w["chunk"]
        per_merge = 3 * c_len * w["hq"] * w["d"] * q.element_size() + 3 * w["hq"] * c_len * 4
        hbm["merge_gbs"] = round(per_merge * n_merge / (parts["merge"] * 1e-3) / 1e9, 1)
    if n_merge and not parts.get("merge"):
        # the fused step has no merge: the LSE merge is timed alone on two partials of the chunk's shape
        c_len = w["chunk"]
        oa, ob = (torch.randn(c_len, w["hq"], w["d"], device=q.device).to(q.dtype) for _ in range(2))
        la, lb = (torch.randn(w["hq"], c_len, device=q.device) for _ in range(2))
        oo, lo = torch.empty_like(oa), torch.empty_like(la)
        for _ in range(3):
            B.attn_merge(oa, la, ob, lb, o_out=oo, lse_out=lo)
        m0, m1 = timing_event(), timing_event()
        m0.record(stream)
        for _ in range(20):
            B.attn_merge(oa, la, ob, lb, o_out=oo, lse_out=lo)
        m1.record(stream)
        torch.cuda.synchronize()
        per_merge = 3 * c_len * w["hq"] * w["d"] * q.element_size() + 3 * w["hq"] * c_len * 4
        hbm["merge_gbs_standalone"] = round(per_merge * 20 / (m0.elapsed_time(m1) * 1e-3) / 1e9, 1)
    red = [b for b in run.bufs if b.keep_any is not None]
    if red and parts.get("reduce"):
        per_red = sum(b.mask.shape[0] * b.mask.shape[1] * b.keep_any.shape[0] * (w["cache_block"] // 128)
                      + b.keep_per_head.numel() + b.keep_any.numel() + b.keep_any_blocks.numel() for b in red)
        hbm["reducer_gbs"] = round(per_red / (parts["reduce"] * 1e-3) / 1e9, 1)
    bsa_flops_step = sum(launches)
    n_launch = len(launches)
    assert len(bsa_durs) == n_launch * a.steps, (len(bsa_durs), n_launch)
    bsa_avg_ms = sum(bsa_durs) / len(bsa_durs)
    bsa_tflops = (bsa_flops_step * a.steps) / (sum(bsa_durs) * 1e-3) / 1e12
    eff_tflops = (bsa_flops_step + est_flops) / (step_ms * 1e-3) / 1e12
    tokens = len(run.starts) * w["chunk"]
    value = tokens / (step_ms * 1e-3)
    if q.dtype == torch.bfloat16 and w["d"] == 128:
        # the library takes the head-pair form when the query heads per kv head are even (XATTN_PAIR=0 disables it)
        if (w["hq"] // w["hkv"]) % 2 == 0 and os.environ.get("XATTN_PAIR", "1") != "0":
            kernel_name = "bsa_pair_kernel<128, bf16> (block-sparse attention, two query heads per workgroup)"
        else:
            kernel_name = "bsa3_kernel<128, bf16> (block-sparse attention)"
        timed_call = "the attention kernel alone (events the library records around its launch)"
    else:
        kernel_name = f"bsa_kernel<{w['d']}, {'fp32 as bf16 hi/lo' if q.dtype == torch.float32 else 'bf16'}>"
        timed_call = "one attention call per segment: one kernel"
    traffic = None
    for rec in TRAFFIC.get(a.workload, []):
        if rec["bsa_code_sha256"] == source_sha(ATTN_SRC) and (rec["stride"], rec["threshold"], rec["fused"]) == (
                w["stride"], w["threshold"], run.fused):
            traffic = rec["hbm_bytes_per_launch"]

    out = {
        "metric": "sparse prefill tokens/s per layer (estimate+BSA) at 32K/128K; % bf16 MFMA peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w["dtype"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": a.workload, "tokens": w["L"], "chunk": w["chunk"], "q_heads": w["hq"],
                   "kv_heads": w["hkv"], "head_dim": w["d"], "stride": w["stride"], "threshold": w["threshold"],
                   "block": 128, "chunks_timed": len(run.starts), "estimator": a.estimator,
                   "attention": "one causal pass per chunk" if run.fused else "history + chunk segments, LSE merge"},
        "roofline": {"bound": "mfma", "kernel": kernel_name,
                     "achieved": round(bsa_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(bsa_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "avg_launch_ms": round(bsa_avg_ms, 4), "launches_per_step": n_launch,
                     "flop_per_launch_avg": bsa_flops_step / n_launch,
                     "timed_call": timed_call},
        "effective_tflops": round(eff_tflops, 1),
        "effective_frac_of_peak": round(eff_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "density": round(dens_rec["density"], 4),
        "comm_density": None if dens_rec["comm_density"] is None else round(dens_rec["comm_density"], 4),
        "density_counts": {"selected": dens_rec["selected"], "causal": dens_rec["causal"],
                           "kept_cache_blocks": dens_rec["kept_cache_blocks"],
                           "cache_blocks": dens_rec["cache_blocks"], "cache_block_tokens": run.density_cache_block},
        "parts_ms": {k2: round(v2, 3) for k2, v2 in parts.items()},
        "bsa_gflop_split": {k2: round(v2 / 1e9, 1) for k2, v2 in split.items()},
        "estimate_gflop": round(est_flops / 1e9, 1),
        "bsa_gflop": round(bsa_flops_step / 1e9, 1),
        "bsa_useful_tflops": round(split["useful"] * a.steps / (sum(bsa_durs) * 1e-3) / 1e12, 1),
        # each attention launch of a step (in launch order): its computed-block work and mean event time
        "bsa_per_launch": [{"gflop": round(f / 1e9, 2),
                            "ms": round(sum(bsa_durs[i::n_launch]) / a.steps, 4),
                            "tflops": round(f / (sum(bsa_durs[i::n_launch]) / a.steps * 1e-3) / 1e12, 1)}
                           for i, f in enumerate(launches)],
        **hbm,
    }
    if a.estimator == "downsampled":
        out["vs_full_estimator"] = compare_estimators(run, q, k, v, w, starts)
    return out


def measure_offload(a, w, q, k, v):
    """The step with the history in pinned host memory (includes the host <-> device copies)."""
    import torch
    from block_sparse_attention_xattn_amd.offload import OffloadedChunkedPrefill
    cb = w.get("cache_block", 1024)
    starts = [w["q_start_pos"]] if "q_start_pos" in w else None
    # with the history on the host the full estimate streams it through the ring
    est = "downsampled" if a.estimator == "downsampled" else "streamed"
    run = OffloadedChunkedPrefill(q, k, v, chunk=w["chunk"], stride=w["stride"], threshold=w["threshold"],
                                  cache_block=cb, group=a.group, chunk_starts=starts, estimator=est)
    run.prepare()
    torch.cuda.synchronize()
    for _ in range(a.warmup):
        for p in run.starts:
            run.run_chunk(p)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        for p in run.starts:
            run.run_chunk(p)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / a.steps
    d, hq, blk = w["d"], w["hq"], 128
    nqb = w["chunk"] // blk
    per_tile = 4.0 * d * blk * blk
    block_bytes = cb * w["hkv"] * d * 2
    flops = h2d = d2h = kept = avail = 0
    for p in run.starts:
        kp = run.kept.get(p, [])
        kept += len(kp)
        avail += p // cb
        flops += per_tile * hq * nqb * (len(kp) * (cb // blk) + (nqb + 1) / 2)
        h2d += 2 * block_bytes * len(kp) + (block_bytes * (p // cb) if est == "streamed" else 0)
        d2h += 2 * block_bytes * (w["chunk"] // cb)
    tokens = len(run.starts) * w["chunk"]
    return {
        "metric": "sparse prefill tokens/s per layer with the history offloaded to host memory (PCIe-inclusive)",
        "value": round(tokens / (step_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(step_ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": a.workload, "tokens": w["L"], "chunk": w["chunk"], "q_heads": hq, "kv_heads": w["hkv"],
                   "head_dim": d, "stride": w["stride"], "threshold": w["threshold"], "cache_block": cb,
                   "ring_group": a.group, "estimator": est, "offload": True},
        "kept_cache_blocks": kept, "history_cache_blocks": avail,
        "host_to_device_gb_per_step": round(h2d / 1e9, 3), "device_to_host_gb_per_step": round(d2h / 1e9, 3),
        "host_to_device_gbs": round(h2d / (step_ms * 1e-3) / 1e9, 1),
        "attention_tflops": round(flops / (step_ms * 1e-3) / 1e12, 1),
    }


def compare_estimators(run, q, k, v, w, starts):
    """Cache blocks kept by the downsampled estimate against those of the full estimate (untimed)."""
    import torch
    from block_sparse_attention_xattn_amd.prefill import ChunkedPrefill
    full = ChunkedPrefill(q, k, v, chunk=w["chunk"], stride=w["stride"], threshold=w["threshold"],
                          chunk_starts=starts, cache_block=w.get("cache_block"))
    full.run()
    torch.cuda.synchronize()
    both = n_full = n_ds = n_all = 0
    for bd, bf in zip(run.bufs, full.bufs):
        if bd.keep_any is None:
            continue
        kd = bd.keep_any.cpu().numpy().astype(bool)
        kf = bf.keep_any.cpu().numpy().astype(bool)
        both += int((kd & kf).sum())
        n_full += int(kf.sum())
        n_ds += int(kd.sum())
        n_all += kd.size
    diff = (run.out.float() - full.out.float()).abs().max().item()
    return {"cache_blocks": n_all, "kept_full": n_full, "kept_downsampled": n_ds,
            "recall_of_full": round(both / max(n_full, 1), 4), "out_max_abs_diff": round(diff, 4)}


if __name__ == "__main__":
    main()
