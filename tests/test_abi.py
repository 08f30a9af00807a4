"""The C ABI on the host (no GPU needed): exports, size queries, argument errors.

Every call here fails validation (or is a pure size query), so nothing is
launched; the library only has to load.
"""
import ctypes
import os
import re

import pytest

from block_sparse_attention_xattn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xattn.h")
FAKE = ctypes.c_void_p(0x100000)      # 256-byte aligned, never dereferenced
FAKE2 = ctypes.c_void_p(0x200000)


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail(f"{B.LIB_PATH} not built (run __graft_entry__.build())")
    return B.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"xattn_estimate", "bsa_prefill", "attn_merge", "xattn_mask_to_cache_blocks", "bsa_pack_v",
            "bsa_prefill_packed"} <= set(names)
    raw = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), f"{n} declared in xattn.h but not exported"


def test_version_and_sizes(lib):
    assert lib.xattn_version().startswith(b"xattn-gfx950")
    # estimate workspace: Hq * nKB * (q_len / stride) fp32 log-sum-exp partials (bf16 input)
    assert B.xattn_estimate_workspace_size(4096, 32768, 32, 8, 128, 8, 128, B.XA_BF16) == 32 * 256 * 512 * 4
    assert B.xattn_estimate_workspace_size(4096, 32768, 32, 8, 128, 8, 128, B.XA_F32) > 32 * 256 * 512 * 4
    # packed V: hkv * d * round_up(capacity, 128) bf16, two planes for fp32
    assert B.bsa_packed_v_bytes(1000, 8, 128, B.XA_BF16) == 8 * 128 * 1024 * 2
    assert B.bsa_packed_v_bytes(1000, 8, 128, B.XA_F32) == 2 * 8 * 128 * 1024 * 2
    assert B.bsa_prefill_packed_workspace_size(4096, 32768, 32, 8, 128, B.XA_BF16) == 0
    assert B.bsa_prefill_workspace_size(4096, 32768, 32, 8, 128, B.XA_BF16) == 8 * 128 * 32768 * 2


def _estimate(lib, **over):
    a = dict(q=FAKE, qt=32 * 128, qh=128, k=FAKE2, kt=8 * 128, kh=128, dt=B.XA_BF16, ql=4096, kl=8192, hq=32,
             hkv=8, d=128, p=4096, S=8, blk=128, tau=0.9, sc=FAKE, m=FAKE2, ws=FAKE, wsb=1 << 40, st=None)
    a.update(over)
    return lib.xattn_estimate(a["q"], a["qt"], a["qh"], a["k"], a["kt"], a["kh"], a["dt"], a["ql"], a["kl"], a["hq"],
                              a["hkv"], a["d"], a["p"], a["S"], a["blk"], a["tau"], a["sc"], a["m"], a["ws"],
                              a["wsb"], a["st"])


@pytest.mark.parametrize("over,status", [
    (dict(d=96), B.XA_EUNSUPPORTED),
    (dict(S=3), B.XA_EUNSUPPORTED),
    (dict(blk=64), B.XA_EUNSUPPORTED),
    (dict(hq=30), B.XA_EINVAL),
    (dict(ql=4000), B.XA_EINVAL),
    (dict(p=100), B.XA_EINVAL),
    (dict(kl=8000), B.XA_EINVAL),
    (dict(q=None), B.XA_EINVAL),
    (dict(qt=33), B.XA_EINVAL),
    (dict(tau=-0.5), B.XA_EINVAL),
    (dict(sc=None), B.XA_EINVAL),
    (dict(wsb=16), B.XA_EWORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100010)), B.XA_EWORKSPACE),
    (dict(dt=7), B.XA_EUNSUPPORTED),
])
def test_estimate_rejects(lib, over, status):
    assert _estimate(lib, **over) == status
    assert lib.xattn_last_error()


def _bsa_packed(lib, **over):
    a = dict(q=FAKE, qt=32 * 128, qh=128, k=FAKE2, kt=8 * 128, kh=128, pv=FAKE, cap=8192, voff=0, dt=B.XA_BF16,
             ql=4096, kl=4096, hq=32, hkv=8, d=128, p=4096, ks=0, m=None, mhs=0, mrs=0, moff=0, blk=128, causal=0,
             scale=0.0, out=FAKE2, odt=B.XA_BF16, lse=FAKE, ws=None, wsb=0, st=None)
    a.update(over)
    return lib.bsa_prefill_packed(a["q"], a["qt"], a["qh"], a["k"], a["kt"], a["kh"], a["pv"], a["cap"], a["voff"],
                                  a["dt"], a["ql"], a["kl"], a["hq"], a["hkv"], a["d"], a["p"], a["ks"], a["m"],
                                  a["mhs"], a["mrs"], a["moff"], a["blk"], a["causal"], a["scale"], a["out"],
                                  a["odt"], a["lse"], a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("over,status", [
    (dict(d=256), B.XA_EUNSUPPORTED),
    (dict(blk=256), B.XA_EUNSUPPORTED),
    (dict(hkv=5), B.XA_EINVAL),
    (dict(ql=100), B.XA_EINVAL),
    (dict(kl=0), B.XA_EINVAL),
    (dict(ks=64), B.XA_EINVAL),
    (dict(voff=64), B.XA_EINVAL),
    (dict(voff=4096, kl=8192), B.XA_EINVAL),        # past the packed capacity
    (dict(m=FAKE, moff=40), B.XA_EINVAL),           # mask offset past the first key block
    (dict(m=FAKE, mhs=-1), B.XA_EINVAL),
    (dict(out=None), B.XA_EINVAL),
    (dict(out=ctypes.c_void_p(0x100008)), B.XA_EINVAL),
    (dict(scale=-1.0), B.XA_EINVAL),
    (dict(odt=3), B.XA_EUNSUPPORTED),
    (dict(pv=ctypes.c_void_p(0x100010)), B.XA_EINVAL),
    (dict(dt=B.XA_F32, ws=None, wsb=0), B.XA_EWORKSPACE),   # fp32 needs split-plane workspace
])
def test_bsa_packed_rejects(lib, over, status):
    assert _bsa_packed(lib, **over) == status


def test_attention_events_arguments(lib):
    # exactly one event is an error; both null switches the hook off (no HIP call is made either way)
    assert lib.xattn_set_attention_events(None, FAKE) == B.XA_EINVAL
    assert lib.xattn_set_attention_events(FAKE, None) == B.XA_EINVAL
    assert b"both events or neither" in lib.xattn_last_error()
    assert lib.xattn_set_attention_events(None, None) == B.XA_OK


def test_merge_and_reducer_reject(lib):
    P = ctypes.c_void_p
    assert lib.attn_merge(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B.XA_BF16, 128, 4, 100, None) == B.XA_EINVAL
    assert lib.attn_merge(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 9, 128, 4, 128, None) == B.XA_EUNSUPPORTED
    assert lib.attn_merge(None, FAKE, FAKE, FAKE, FAKE, FAKE, B.XA_BF16, 128, 4, 128, None) == B.XA_EINVAL
    assert lib.attn_merge(FAKE, FAKE, FAKE, FAKE, P(0x100004), FAKE, B.XA_BF16, 128, 4, 128, None) == B.XA_EINVAL
    assert lib.attn_merge(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B.XA_BF16, 0, 4, 128, None) == B.XA_OK  # empty
    assert lib.xattn_mask_to_cache_blocks(FAKE, 0, 4, 64, 0, 0, 0, 8, 8, 1, FAKE, FAKE, FAKE, None) == B.XA_EINVAL
    assert lib.xattn_mask_to_cache_blocks(FAKE, 4, 4, 64, 0, 0, 0, 9, 8, 1, FAKE, FAKE, FAKE, None) == B.XA_EINVAL
    assert lib.xattn_mask_to_cache_blocks(None, 4, 4, 64, 0, 0, 0, 8, 8, 1, FAKE, FAKE, FAKE, None) == B.XA_EINVAL
    assert lib.xattn_mask_to_cache_blocks(FAKE, 4, 4, 64, 0, 0, 0, 0, 8, 1, FAKE, FAKE, FAKE, None) == B.XA_OK


def test_pack_v_rejects(lib):
    assert lib.bsa_pack_v(FAKE, 1024, 128, B.XA_BF16, 256, 8, 128, FAKE2, 100, 0, None) == B.XA_EINVAL  # capacity
    assert lib.bsa_pack_v(FAKE, 1024, 128, B.XA_BF16, 256, 8, 128, FAKE2, 1024, 64, None) == B.XA_EINVAL  # offset
    assert lib.bsa_pack_v(FAKE, 1024, 128, B.XA_BF16, 256, 8, 96, FAKE2, 1024, 0, None) == B.XA_EUNSUPPORTED
    assert lib.bsa_pack_v(FAKE, 1024, 128, B.XA_BF16, 256, 8, 128, ctypes.c_void_p(0x200010), 1024, 0,
                          None) == B.XA_EINVAL


def _plan_bytes(n_items, d):
    a = lambda b: (b + 255) // 256 * 256  # noqa: E731
    ms = min(n_items, 512)
    return (256 + 3 * a(4 * n_items) + a(4 * ms) + a(4 * (n_items + ms)) + a(ms * 2 * 128 * d * 4)
            + a(ms * 2 * 128 * 4))


def test_segments_workspace(lib):
    # ticket/counters, per-item counts, medians, slots; split items; entries; fp32 partials of split items
    assert B.bsa_prefill_segments_workspace_size(4096, 32, 128, 2) == _plan_bytes(2 * 32 * 32, 128)
    assert B.bsa_prefill_segments_workspace_size(4000, 32, 128, 1) == _plan_bytes(32 * 32, 128)  # ragged
    assert B.bsa_prefill_segments_workspace_size(1024, 8, 128, 2) == _plan_bytes(128, 128)      # < 512 items
    assert B.bsa_prefill_segments_workspace_size(4096, 32, 128, 2) < 70 * 2 ** 20
    assert B.bsa_prefill_segments_workspace_size(0, 32, 128, 2) == 0
    assert B.bsa_prefill_segments_workspace_size(4096, 32, 128, 5) == 0
    assert B.bsa_prefill_segments_workspace_size(4096, 32, 0, 2) == 0
    seg = (B.Segment * 1)()
    seg[0] = B.Segment(FAKE.value, 8 * 128, 128, 4096, 0, 0, None, 0, 0, 0, 0, FAKE2.value, FAKE.value)
    need = B.bsa_prefill_segments_workspace_size(4096, 32, 128, 1)

    def call(ws, wsb, n=1, dt=B.XA_BF16):
        return lib.bsa_prefill_segments(FAKE, 32 * 128, 128, FAKE, 8192, dt, 4096, 32, 8, 128, 4096, seg, n, 128,
                                        0.0, B.XA_BF16, ws, wsb, None)
    assert call(None, 0) == B.XA_EWORKSPACE
    assert call(FAKE, need - 1) == B.XA_EWORKSPACE
    assert call(ctypes.c_void_p(0x100010), need) == B.XA_EWORKSPACE
    assert call(FAKE, need, n=0) == B.XA_EINVAL
    assert call(FAKE, need, n=5) == B.XA_EINVAL
    assert call(FAKE, need, dt=B.XA_F32) == B.XA_EUNSUPPORTED


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def test_offload_entry_points_reject(lib):
    I32 = ctypes.c_int32
    keep = (I32 * 2)(0, 9)

    def off(n=4, first=0, n_host=8, d=128, cb=1024, stg=FAKE2, dt=B.XA_BF16):
        return lib.xattn_offload_blocks(FAKE, 1024, 128, FAKE, 1024, 128, dt, n, 8, d, cb, FAKE, FAKE, n_host, first,
                                        stg, None)
    assert off(first=6) == B.XA_EINVAL                       # past the host store
    assert off(n=-1) == B.XA_EINVAL
    assert off(d=96) == B.XA_EUNSUPPORTED
    assert off(cb=1000) == B.XA_EINVAL
    assert off(stg=ctypes.c_void_p(0x200010)) == B.XA_EINVAL
    assert off(dt=B.XA_F32) == B.XA_EUNSUPPORTED

    def hist(ids=keep, n=2, group=2, rvt=FAKE2, dt=B.XA_BF16):
        return lib.bsa_history_offloaded(FAKE, 4096, 128, dt, 1024, 32, 8, 128, 8192, FAKE, FAKE, 8, 1024, ids, n,
                                         group, FAKE, rvt, FAKE, FAKE, FAKE, FAKE, None, None)
    assert hist() == B.XA_EINVAL                             # id 9 outside 8 host blocks
    assert hist(ids=None, n=1) == B.XA_EINVAL
    assert hist(n=1, group=0) == B.XA_EINVAL
    assert hist(n=1, rvt=ctypes.c_void_p(0x200010)) == B.XA_EINVAL
    assert hist(n=1, dt=B.XA_F32) == B.XA_EUNSUPPORTED

    need = B.xattn_estimate_workspace_size(1024, 5120, 32, 8, 128, 8, 128, B.XA_BF16)

    def est(p=4096, n_host=8, S=8, group=2, ring=FAKE2, ws=FAKE, wsb=need, tau=0.9, dt=B.XA_BF16):
        return lib.xattn_estimate_offloaded(FAKE, 4096, 128, FAKE, 1024, 128, dt, 1024, 32, 8, 128, p, FAKE, n_host,
                                            1024, group, ring, S, 128, tau, FAKE, FAKE, ws, wsb, None, None)
    assert est(p=1000) == B.XA_EINVAL                        # not whole cache blocks
    assert est(p=12288) == B.XA_EINVAL                       # more history than the host store holds
    assert est(S=3) == B.XA_EUNSUPPORTED
    assert est(group=0) == B.XA_EINVAL
    assert est(ring=ctypes.c_void_p(0x200008)) == B.XA_EINVAL
    assert est(wsb=need - 1) == B.XA_EWORKSPACE
    assert est(ws=ctypes.c_void_p(0x100010)) == B.XA_EWORKSPACE
    assert est(tau=float("nan")) == B.XA_EINVAL
    assert est(dt=B.XA_F32) == B.XA_EUNSUPPORTED


def test_varlen_sizes_and_rejects(lib):
    C = lambda xs: (ctypes.c_int64 * len(xs))(*xs)  # noqa: E731
    cq, ck = [0, 256, 256, 640], [0, 512, 768, 1664]            # lens (256, 512), (0, 256), (384, 896)
    assert B.xattn_varlen_mask_elems(cq, ck, 4) == 4 * (2 * 4 + 0 + 3 * 7)
    assert B.xattn_varlen_mask_elems([0, 100], [0, 128], 4) == -1            # ragged
    assert B.xattn_varlen_mask_elems([0, 256], [0, 128], 4) == -1            # q_len > k_len
    assert B.xattn_varlen_mask_elems([128, 256], [0, 256], 4) == -1          # not starting at 0
    lse_floats = 4 * (4 * 256 // 8 + 0 + 7 * 384 // 8)
    assert B.xattn_estimate_varlen_workspace_size(cq, ck, 4, 2, 8) == 256 + (lse_floats * 4 + 255) // 256 * 256
    assert B.bsa_prefill_varlen_workspace_size(cq, ck, 4, 128) == 256 + _plan_bytes(4 * (2 + 0 + 3), 128)
    need_e = B.xattn_estimate_varlen_workspace_size(cq, ck, 4, 2, 8)

    def est(cq=cq, ck=ck, b=3, d=128, S=8, ws=FAKE, wsb=need_e, dt=B.XA_BF16):
        return lib.xattn_estimate_varlen(FAKE, 512, 128, FAKE2, 256, 128, dt, C(cq), C(ck), b, 4, 2, d, S, 128, 0.9,
                                         FAKE, FAKE2, ws, wsb, None)
    assert est(d=64) == B.XA_EUNSUPPORTED
    assert est(dt=B.XA_F32) == B.XA_EUNSUPPORTED
    assert est(S=3) == B.XA_EUNSUPPORTED
    assert est(cq=[0, 256, 256, 700]) == B.XA_EINVAL
    assert est(ck=[0, 128, 384, 1280]) == B.XA_EINVAL                     # first sequence: q_len > k_len
    assert est(b=0) == B.XA_EINVAL
    assert est(wsb=need_e - 1) == B.XA_EWORKSPACE
    need_b = B.bsa_prefill_varlen_workspace_size(cq, ck, 4, 128)

    def bsa(cap=1664, out=FAKE, odt=B.XA_BF16, ws=FAKE2, wsb=need_b, d=128):
        return lib.bsa_prefill_varlen(FAKE, 512, 128, FAKE2, 256, 128, FAKE, cap, B.XA_BF16, C(cq), C(ck), 3, 4, 2, d,
                                      None, 128, 0.0, out, odt, FAKE2, ws, wsb, None)
    assert bsa(cap=1536) == B.XA_EINVAL                                    # packed V shorter than the keys
    assert bsa(out=ctypes.c_void_p(0x100008)) == B.XA_EINVAL
    assert bsa(odt=7) == B.XA_EUNSUPPORTED
    assert bsa(d=64) == B.XA_EUNSUPPORTED
    assert bsa(wsb=need_b - 1) == B.XA_EWORKSPACE


def test_density_counts_rejects(lib):
    def dc(mask=FAKE, heads=4, nqb=2, ncols=16, hs=32, rs=16, diag0=14, keep=FAKE2, ncb=3, counts=FAKE):
        return lib.xattn_density_counts(mask, heads, nqb, ncols, hs, rs, diag0, keep, ncb, counts, None)
    assert dc(counts=None) == B.XA_EINVAL
    assert dc(counts=ctypes.c_void_p(0x100004)) == B.XA_EINVAL        # not 8-byte aligned
    assert dc(heads=0) == B.XA_EINVAL
    assert dc(ncols=0) == B.XA_EINVAL
    assert dc(rs=-16) == B.XA_EINVAL
    assert dc(ncb=-1) == B.XA_EINVAL
    assert dc(keep=None, ncb=3) == B.XA_EINVAL                           # cache blocks without a keep list
    assert dc(mask=None, keep=None, ncb=0) == B.XA_OK                     # nothing to count: nothing launched


@pytest.mark.parametrize("qt,qh,ok", [
    (32 * 128, 128, True),          # token-major
    (128, 4096 * 128, True),        # head-major (4096 tokens of a head, then the next head)
    (128, 128, False),              # heads alias tokens
    (32 * 128, 64, False),          # heads overlap inside a row
    (64 * 128, 256, True),          # token-major with gaps (a slice of a wider buffer)
    (128, 128 * 100, False),        # head-major but heads closer than the token extent
])
def test_estimate_rejects_aliasing_layouts(lib, qt, qh, ok):
    # block_scores is null, so even an accepted layout fails validation (after the layout check): nothing launches
    st = _estimate(lib, qt=qt, qh=qh, sc=None)
    assert st == B.XA_EINVAL
    assert (b"overlap" in lib.xattn_last_error()) != ok
