"""xattn_estimate_noalloc (no workspace, the library's own device array) against xattn_estimate.

The two entry points run the same kernels, so their block scores and masks must be identical bit for bit.
Two calls in a row on the same array, the second smaller, show that what the first call left there does not
leak into the second.  A request larger than the array is refused before anything is launched.
"""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(*shape, generator=g)).to(torch.bfloat16)


def test_noalloc_matches_workspace_entry_point():
    from block_sparse_attention_xattn_amd import binding as B
    from block_sparse_attention_xattn_amd import synthetic
    cases = [
        # (label, q, k, q_start_pos, stride, threshold)
        ("32K layer, last chunk", *synthetic.long_context(32768, 32, 8, 128, n_needles=16, seed=2)[:2], 28672, 8,
         0.95),
        ("2K, 4/2 heads, stride 16", _rand((2048, 4, 128), 5), _rand((2048, 2, 128), 6), 1024, 16, 0.9),
        ("1K fp32, 2/1 heads, head_dim 64", *synthetic.tiny(0)[:2], 0, 8, 0.9),
    ]
    for label, q, k, p, S, tau in cases:
        print(f"[noalloc] {label}", flush=True)
        qd = q[p:].to(DEV)          # the query chunk: global positions p .. len(q) - 1
        kd = k.to(DEV)              # its keys 0 .. len(q) - 1
        ref_s, ref_m = B.xattn_estimate(qd, kd, p, S, tau)
        got_s = torch.full_like(ref_s, float("nan"))
        got_m = torch.full_like(ref_m, 7)
        B.xattn_estimate_noalloc(qd, kd, p, S, tau, block_scores=got_s, block_mask=got_m)
        torch.cuda.synchronize()
        assert torch.equal(got_s, ref_s), label
        assert torch.equal(got_m, ref_m), label


def test_noalloc_rejects_beyond_its_array():
    from block_sparse_attention_xattn_amd import binding as B
    lib = B.lib()
    cap = lib.xattn_estimate_noalloc_max_bytes()
    assert cap == 64 << 20
    # 64 query heads against 131072 keys at stride 8: 64 * 1024 * 512 * 4 B = 128 MiB of partials
    need = B.xattn_estimate_workspace_size(4096, 131072, 64, 8, 128, 8)
    assert need > cap
    fake = ctypes.c_void_p(0x100000)
    st = lib.xattn_estimate_noalloc(fake, 64 * 128, 128, fake, 8 * 128, 128, B.XA_BF16, 4096, 131072, 64, 8, 128,
                                    126976, 8, 128, 0.9, fake, fake, None)
    assert st == B.XA_EUNSUPPORTED
    assert b"working memory" in lib.xattn_last_error()
