"""Thin ctypes binding of libxattn.so (argument marshalling only).

Every function here has the name of the C entry point it calls, takes torch
tensors that already live on the GPU, passes their device pointers, sizes and
strides, and enqueues on the current torch stream.  No arithmetic of the path
happens in Python; if the library is missing the call raises.

Layouts (batch = 1): q [q_len, Hq, d], k/v [kv_len, Hkv, d] (last dim
contiguous); block masks / scores [Hq, q_len/128, n_key_blocks]; out
[q_len, Hq, d]; lse [Hq, q_len].
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libxattn.so")

XA_OK, XA_EINVAL, XA_EUNSUPPORTED, XA_EWORKSPACE, XA_EHIP = 0, 1, 2, 3, 4
XA_F32, XA_BF16 = 0, 1
STATUS_NAMES = {0: "XA_OK", 1: "XA_EINVAL", 2: "XA_EUNSUPPORTED", 3: "XA_EWORKSPACE", 4: "XA_EHIP"}

_lib = None


class Segment(ctypes.Structure):
    """xa_segment_t (xattn.h)."""
    _fields_ = [("k", ctypes.c_void_p), ("k_tok_stride", ctypes.c_int64), ("k_head_stride", ctypes.c_int64),
                ("kv_len", ctypes.c_int64), ("kv_start", ctypes.c_int64), ("v_token_offset", ctypes.c_int64),
                ("block_mask", ctypes.c_void_p), ("mask_head_stride", ctypes.c_int64),
                ("mask_row_stride", ctypes.c_int64), ("mask_kb_offset", ctypes.c_int64), ("causal", ctypes.c_int32),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


class XattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _declare(lib):
    P, I64, I32, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.xattn_last_error.restype = ctypes.c_char_p
    lib.xattn_last_error.argtypes = []
    lib.xattn_version.restype = ctypes.c_char_p
    lib.xattn_version.argtypes = []
    lib.xattn_set_attention_events.restype = ctypes.c_int
    lib.xattn_set_attention_events.argtypes = [P, P]
    lib.xattn_estimate_workspace_size.restype = SZ
    lib.xattn_estimate_workspace_size.argtypes = [I64, I64, I32, I32, I32, I32, I32, ctypes.c_int]
    lib.xattn_estimate.restype = ctypes.c_int
    lib.xattn_estimate.argtypes = [P, I64, I64, P, I64, I64, ctypes.c_int, I64, I64, I32, I32, I32,
                                   I64, I32, I32, F, P, P, P, SZ, P]
    lib.xattn_estimate_noalloc_max_bytes.restype = SZ
    lib.xattn_estimate_noalloc_max_bytes.argtypes = []
    lib.xattn_estimate_noalloc.restype = ctypes.c_int
    lib.xattn_estimate_noalloc.argtypes = [P, I64, I64, P, I64, I64, ctypes.c_int, I64, I64, I32, I32, I32,
                                           I64, I32, I32, F, P, P, P]
    lib.bsa_prefill_workspace_size.restype = SZ
    lib.bsa_prefill_workspace_size.argtypes = [I64, I64, I32, I32, I32, ctypes.c_int]
    lib.bsa_prefill.restype = ctypes.c_int
    lib.bsa_prefill.argtypes = [P, I64, I64, P, I64, I64, P, I64, I64, ctypes.c_int, I64, I64, I32, I32, I32,
                                I64, I64, P, I64, I64, I64, I32, I32, F, P, ctypes.c_int, P, P, SZ, P]
    lib.bsa_packed_v_bytes.restype = SZ
    lib.bsa_packed_v_bytes.argtypes = [I64, I32, I32, ctypes.c_int]
    lib.bsa_pack_v.restype = ctypes.c_int
    lib.bsa_pack_v.argtypes = [P, I64, I64, ctypes.c_int, I64, I32, I32, P, I64, I64, P]
    lib.bsa_prefill_packed_workspace_size.restype = SZ
    lib.bsa_prefill_packed_workspace_size.argtypes = [I64, I64, I32, I32, I32, ctypes.c_int]
    lib.bsa_prefill_packed.restype = ctypes.c_int
    lib.bsa_prefill_packed.argtypes = [P, I64, I64, P, I64, I64, P, I64, I64, ctypes.c_int, I64, I64, I32, I32, I32,
                                       I64, I64, P, I64, I64, I64, I32, I32, F, P, ctypes.c_int, P, P, SZ, P]
    lib.bsa_prefill_segments.restype = ctypes.c_int
    lib.bsa_prefill_segments.argtypes = [P, I64, I64, P, I64, ctypes.c_int, I64, I32, I32, I32, I64,
                                         ctypes.POINTER(Segment), I32, I32, F, ctypes.c_int, P, SZ, P]
    lib.bsa_prefill_segments_workspace_size.restype = SZ
    lib.bsa_prefill_segments_workspace_size.argtypes = [I64, I32, I32, I32]
    lib.xattn_downsample_keys.restype = ctypes.c_int
    lib.xattn_downsample_keys.argtypes = [P, I64, I64, ctypes.c_int, I64, I32, I32, I32, P, I64, I64, P]
    lib.xattn_estimate_history_ds_workspace_size.restype = SZ
    lib.xattn_estimate_history_ds_workspace_size.argtypes = [I64, I64, I32, I32, I32, I32, I32, ctypes.c_int]
    lib.xattn_estimate_history_ds.restype = ctypes.c_int
    lib.xattn_estimate_history_ds.argtypes = [P, I64, I64, P, I64, I64, ctypes.c_int, I64, I64, I32, I32, I32, I32,
                                              I32, F, P, P, P, SZ, P]
    lib.xattn_offload_blocks.restype = ctypes.c_int
    lib.xattn_offload_blocks.argtypes = [P, I64, I64, P, I64, I64, ctypes.c_int, I32, I32, I32, I32, P, P, I64, I64,
                                         P, P]
    lib.bsa_history_offloaded.restype = ctypes.c_int
    lib.bsa_history_offloaded.argtypes = [P, I64, I64, ctypes.c_int, I64, I32, I32, I32, I64, P, P, I64, I32, P, I32,
                                          I32, P, P, P, P, P, P, P, P]
    lib.xattn_estimate_offloaded.argtypes = [P, I64, I64, P, I64, I64, ctypes.c_int, I64, I32, I32, I32, I64, P,
                                             I64, I32, I32, P, I32, I32, F, P, P, P, SZ, P, P]
    I64P = ctypes.POINTER(ctypes.c_int64)
    lib.xattn_varlen_mask_elems.restype = I64
    lib.xattn_varlen_mask_elems.argtypes = [I64P, I64P, I32, I32]
    lib.xattn_estimate_varlen_workspace_size.restype = SZ
    lib.xattn_estimate_varlen_workspace_size.argtypes = [I64P, I64P, I32, I32, I32, I32]
    lib.xattn_estimate_varlen.argtypes = [P, I64, I64, P, I64, I64, ctypes.c_int, I64P, I64P, I32, I32, I32, I32, I32,
                                          I32, F, P, P, P, SZ, P]
    lib.bsa_prefill_varlen_workspace_size.restype = SZ
    lib.bsa_prefill_varlen_workspace_size.argtypes = [I64P, I64P, I32, I32, I32]
    lib.bsa_prefill_varlen.argtypes = [P, I64, I64, P, I64, I64, P, I64, ctypes.c_int, I64P, I64P, I32, I32, I32, I32,
                                       P, I32, F, P, ctypes.c_int, P, P, SZ, P]
    lib.attn_merge.restype = ctypes.c_int
    lib.attn_merge.argtypes = [P, P, P, P, P, P, ctypes.c_int, I64, I32, I32, P]
    lib.xattn_mask_to_cache_blocks.restype = ctypes.c_int
    lib.xattn_mask_to_cache_blocks.argtypes = [P, I32, I32, I64, I64, I64, I64, I64, I32, I32, P, P, P, P]
    lib.xattn_density_counts.restype = ctypes.c_int
    lib.xattn_density_counts.argtypes = [P, I32, I32, I64, I64, I64, I64, P, I64, P, P]
    return lib


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_xattn_amd.build`")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _check(st: int):
    if st != XA_OK:
        raise XattnError(st, lib().xattn_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return XA_BF16
    if t.dtype == torch.float32:
        return XA_F32
    raise XattnError(XA_EUNSUPPORTED, f"dtype {t.dtype} (bfloat16 or float32 only)")


def _qkv_check(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise XattnError(XA_EINVAL, f"{name} must be a GPU tensor")
    if t.dim() != 3 or t.stride(2) != 1:
        raise XattnError(XA_EINVAL, f"{name} must be [tokens, heads, head_dim] with a contiguous last dim")


def _dense_check(t, name: str, shape, dtype, device):
    """t must be a contiguous tensor of exactly `shape` and `dtype` on `device` (the kernels write it densely)."""
    if t is None:
        return
    if not t.is_cuda or t.device != torch.device(device):
        raise XattnError(XA_EINVAL, f"{name} must be on {device}")
    if tuple(t.shape) != tuple(shape):
        raise XattnError(XA_EINVAL, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise XattnError(XA_EINVAL, f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise XattnError(XA_EINVAL, f"{name} must be contiguous")


def _flat_check(t, name: str, min_elems: int, dtype, device):
    """t must be a contiguous tensor of `dtype` on `device` holding at least min_elems elements."""
    if not t.is_cuda or t.device != torch.device(device):
        raise XattnError(XA_EINVAL, f"{name} must be on {device}")
    if t.dtype != dtype or not t.is_contiguous():
        raise XattnError(XA_EINVAL, f"{name} must be a contiguous {dtype} tensor")
    if t.numel() < min_elems:
        raise XattnError(XA_EINVAL, f"{name} holds {t.numel()} elements, needs {min_elems}")


def _mask_check(m, name: str, device, heads=None, n_rows=None, col_lo=None, col_hi=None, hs=None, rs=None):
    """A byte mask on `device` with a contiguous last dim; when the rows / columns a call reads are given,
    every byte h*hs + qb*rs + col (h < heads, qb < n_rows, col_lo <= col <= col_hi) must lie inside the
    tensor's storage."""
    if not m.is_cuda or m.device != torch.device(device):
        raise XattnError(XA_EINVAL, f"{name} must be on {device}")
    if m.dtype not in (torch.uint8, torch.bool) or m.stride(-1) not in (0, 1):
        raise XattnError(XA_EINVAL, f"{name} must be uint8/bool with a contiguous last dim")
    if heads is None or n_rows is None or col_hi is None or col_hi < col_lo:
        return
    hs = m.stride(0) if hs is None else hs
    rs = m.stride(1) if rs is None else rs
    if col_lo < 0 or hs < 0 or rs < 0:
        raise XattnError(XA_EINVAL, f"{name}: negative column or stride")
    last = (heads - 1) * hs + (n_rows - 1) * rs + col_hi
    avail = m.untyped_storage().nbytes() - m.storage_offset() * m.element_size()
    if last >= avail:
        raise XattnError(XA_EINVAL, f"{name}: the call reads byte {last} but only {avail} are reachable")


def _out_dtype(out, out_dtype, default):
    """The output dtype: out_dtype if given, else out's, else default; out must agree with it."""
    odt = out_dtype if out_dtype is not None else (out.dtype if out is not None else default)
    if out is not None and out.dtype != odt:
        raise XattnError(XA_EINVAL, f"out has dtype {out.dtype} but out_dtype is {odt}")
    return odt


def _attn_mask_strides(m, q, hq, q_len, kv_start, kv_len, mask_kb_offset, block, mask_head_stride,
                       mask_row_stride):
    """(head stride, row stride) of an attention call's mask after checking that every byte the call reads
    (heads 0..hq-1, query blocks 0..q_len/block-1, the key blocks of [kv_start, kv_start+kv_len) shifted by
    mask_kb_offset) lies inside it; (0, 0) without a mask."""
    if m is None:
        return 0, 0
    if m.dim() != 3:
        raise XattnError(XA_EINVAL, "block_mask must be [heads, query blocks, key blocks] (or a broadcast view)")
    hs = m.stride(0) if mask_head_stride is None else mask_head_stride
    rs = m.stride(1) if mask_row_stride is None else mask_row_stride
    if kv_len > 0 and q_len > 0:
        lo = kv_start // block - mask_kb_offset
        hi = (kv_start + kv_len - 1) // block - mask_kb_offset
        _mask_check(m, "block_mask", q.device, hq, max(q_len // block, 1), lo, hi, hs, rs)
    else:
        _mask_check(m, "block_mask", q.device)
    return hs, rs


def xattn_set_attention_events(before=None, after=None, stream=None):
    """Measurement hook: later attention calls on this thread record the torch.cuda.Event objects
    `before` / `after` immediately around each launch of a ping-pong attention kernel (head-pair or single-head
    form); (None, None)
    turns it off.  An event torch has not created yet is recorded once on `stream` here so that its
    handle exists."""
    handles = []
    for ev in (before, after):
        if ev is not None and ev.cuda_event == 0:
            ev.record(torch.cuda.current_stream() if stream is None else stream)
        handles.append(None if ev is None else ctypes.c_void_p(ev.cuda_event))
    _check(lib().xattn_set_attention_events(*handles))


def workspace(nbytes: int, device) -> torch.Tensor:
    """A device byte buffer of at least nbytes (256-byte aligned by the caching allocator)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def xattn_estimate_workspace_size(q_len, k_len, num_q_heads, num_kv_heads, head_dim, stride, block=128,
                                  dtype=XA_BF16) -> int:
    return int(lib().xattn_estimate_workspace_size(q_len, k_len, num_q_heads, num_kv_heads, head_dim, stride,
                                                   block, dtype))


def bsa_prefill_workspace_size(q_len, kv_len, num_q_heads, num_kv_heads, head_dim, dtype=XA_BF16) -> int:
    return int(lib().bsa_prefill_workspace_size(q_len, kv_len, num_q_heads, num_kv_heads, head_dim, dtype))


def xattn_estimate(q, k, q_start_pos: int, stride: int = 8, threshold: float = 0.9, block: int = 128,
                   block_scores=None, block_mask=None, ws=None, stream=None):
    """Block scores and block mask of one query chunk (see xattn.h).  Returns (scores, mask)."""
    _qkv_check(q, "q")
    _qkv_check(k, "k")
    dt = _dtype_code(q)
    if k.dtype != q.dtype:
        raise XattnError(XA_EINVAL, "q and k dtypes differ")
    q_len, hq, d = q.shape
    k_len, hkv, _ = k.shape
    n_qb, nkb = q_len // block, k_len // block
    if block_scores is None:
        block_scores = torch.empty(hq, n_qb, nkb, dtype=torch.float32, device=q.device)
    if block_mask is None:
        block_mask = torch.empty(hq, n_qb, nkb, dtype=torch.uint8, device=q.device)
    _dense_check(block_scores, "block_scores", (hq, n_qb, nkb), torch.float32, q.device)
    _dense_check(block_mask, "block_mask", (hq, n_qb, nkb), block_mask.dtype if block_mask.dtype == torch.bool
                 else torch.uint8, q.device)
    need = xattn_estimate_workspace_size(q_len, k_len, hq, hkv, d, stride, block, dt)
    if ws is None:
        ws = workspace(need, q.device)
    _check(lib().xattn_estimate(_ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1), dt,
                                q_len, k_len, hq, hkv, d, q_start_pos, stride, block, float(threshold),
                                _ptr(block_scores), _ptr(block_mask), _ptr(ws), ws.numel(), _stream(stream)))
    return block_scores, block_mask


def xattn_estimate_noalloc(q, k, q_start_pos: int, stride: int = 8, threshold: float = 0.9, block: int = 128,
                           block_scores=None, block_mask=None, stream=None):
    """xattn_estimate with the library's own working memory (no workspace; see xattn.h).  Returns (scores, mask);
    pass preallocated block_scores / block_mask to allocate nothing here either."""
    _qkv_check(q, "q")
    _qkv_check(k, "k")
    dt = _dtype_code(q)
    if k.dtype != q.dtype:
        raise XattnError(XA_EINVAL, "q and k dtypes differ")
    q_len, hq, d = q.shape
    k_len, hkv, _ = k.shape
    n_qb, nkb = q_len // block, k_len // block
    if block_scores is None:
        block_scores = torch.empty(hq, n_qb, nkb, dtype=torch.float32, device=q.device)
    if block_mask is None:
        block_mask = torch.empty(hq, n_qb, nkb, dtype=torch.uint8, device=q.device)
    _dense_check(block_scores, "block_scores", (hq, n_qb, nkb), torch.float32, q.device)
    _dense_check(block_mask, "block_mask", (hq, n_qb, nkb), block_mask.dtype if block_mask.dtype == torch.bool
                 else torch.uint8, q.device)
    _check(lib().xattn_estimate_noalloc(_ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1), dt,
                                        q_len, k_len, hq, hkv, d, q_start_pos, stride, block, float(threshold),
                                        _ptr(block_scores), _ptr(block_mask), _stream(stream)))
    return block_scores, block_mask


def bsa_prefill(q, k, v, q_start_pos: int, kv_start: int, block_mask=None, mask_kb_offset: int = 0,
                causal: bool = True, softmax_scale: float = 0.0, out_dtype=None, block: int = 128,
                out=None, lse=None, ws=None, mask_head_stride=None, mask_row_stride=None, stream=None):
    """Block-sparse attention with LSE (see xattn.h).  Returns (out, lse).

    block_mask: uint8 [Hq, n_qb, n_cols] (or a broadcast view with zero strides), or None for dense.
    """
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _qkv_check(t, nm)
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise XattnError(XA_EINVAL, "q, k, v dtypes differ")
    q_len, hq, d = q.shape
    kv_len, hkv, _ = k.shape
    out_dtype = _out_dtype(out, out_dtype, q.dtype)
    odt = _dtype_code(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty(q_len, hq, d, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty(hq, q_len, dtype=torch.float32, device=q.device)
    _dense_check(out, "out", (q_len, hq, d), out_dtype, q.device)
    _dense_check(lse, "lse", (hq, q_len), torch.float32, q.device)
    hs, rs = _attn_mask_strides(block_mask, q, hq, q_len, kv_start, kv_len, mask_kb_offset, block,
                                mask_head_stride, mask_row_stride)
    need = bsa_prefill_workspace_size(q_len, kv_len, hq, hkv, d, dt)
    if ws is None:
        ws = workspace(need, q.device)
    _check(lib().bsa_prefill(_ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1),
                             _ptr(v), v.stride(0), v.stride(1), dt, q_len, kv_len, hq, hkv, d,
                             q_start_pos, kv_start, _ptr(block_mask), hs, rs, mask_kb_offset, block,
                             1 if causal else 0, float(softmax_scale), _ptr(out), odt, _ptr(lse),
                             _ptr(ws), ws.numel(), _stream(stream)))
    return out, lse


def bsa_packed_v_bytes(capacity, num_kv_heads, head_dim, dtype=XA_BF16) -> int:
    return int(lib().bsa_packed_v_bytes(capacity, num_kv_heads, head_dim, dtype))


def bsa_prefill_packed_workspace_size(q_len, kv_len, num_q_heads, num_kv_heads, head_dim, dtype=XA_BF16) -> int:
    return int(lib().bsa_prefill_packed_workspace_size(q_len, kv_len, num_q_heads, num_kv_heads, head_dim, dtype))


class PackedV:
    """A packed-V buffer of ``capacity`` tokens (see bsa_pack_v in xattn.h)."""

    def __init__(self, capacity: int, num_kv_heads: int, head_dim: int, dtype, device):
        self.capacity, self.hkv, self.d = capacity, num_kv_heads, head_dim
        self.dtype = dtype
        self.code = _dtype_code(torch.empty(0, dtype=dtype))
        self.buf = workspace(bsa_packed_v_bytes(capacity, num_kv_heads, head_dim, self.code), device)


def bsa_pack_v(v, packed: PackedV, token_offset: int, stream=None):
    """Pack V rows [n, Hkv, d] as packed tokens token_offset .. token_offset+n-1."""
    _qkv_check(v, "v")
    if v.dtype != packed.dtype:
        raise XattnError(XA_EINVAL, "v dtype differs from the packed buffer")
    n, hkv, d = v.shape
    _check(lib().bsa_pack_v(_ptr(v), v.stride(0), v.stride(1), packed.code, n, hkv, d, _ptr(packed.buf),
                            packed.capacity, token_offset, _stream(stream)))


def bsa_prefill_packed(q, k, packed: PackedV, v_token_offset: int, q_start_pos: int, kv_start: int,
                       block_mask=None, mask_kb_offset: int = 0, causal: bool = True, softmax_scale: float = 0.0,
                       out_dtype=None, block: int = 128, out=None, lse=None, ws=None, mask_head_stride=None,
                       mask_row_stride=None, stream=None):
    """bsa_prefill with V read from packed tokens v_token_offset .. +kv_len.  Returns (out, lse)."""
    for t, nm in ((q, "q"), (k, "k")):
        _qkv_check(t, nm)
    dt = _dtype_code(q)
    q_len, hq, d = q.shape
    kv_len, hkv, _ = k.shape
    out_dtype = _out_dtype(out, out_dtype, q.dtype)
    odt = _dtype_code(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty(q_len, hq, d, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty(hq, q_len, dtype=torch.float32, device=q.device)
    _dense_check(out, "out", (q_len, hq, d), out_dtype, q.device)
    _dense_check(lse, "lse", (hq, q_len), torch.float32, q.device)
    hs, rs = _attn_mask_strides(block_mask, q, hq, q_len, kv_start, kv_len, mask_kb_offset, block,
                                mask_head_stride, mask_row_stride)
    need = bsa_prefill_packed_workspace_size(q_len, kv_len, hq, hkv, d, dt)
    if ws is None and need > 0:
        ws = workspace(need, q.device)
    _check(lib().bsa_prefill_packed(_ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1),
                                    _ptr(packed.buf), packed.capacity, v_token_offset, dt, q_len, kv_len, hq, hkv,
                                    d, q_start_pos, kv_start, _ptr(block_mask), hs, rs, mask_kb_offset, block,
                                    1 if causal else 0, float(softmax_scale), _ptr(out), odt, _ptr(lse), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(stream)))
    return out, lse


def bsa_prefill_segments_workspace_size(q_len: int, num_q_heads: int, head_dim: int, n_segments: int) -> int:
    return int(lib().bsa_prefill_segments_workspace_size(q_len, num_q_heads, head_dim, n_segments))


def bsa_prefill_segments(q, packed: PackedV, q_start_pos: int, segments, softmax_scale: float = 0.0, block: int = 128,
                         ws=None, stream=None):
    """Several attention problems over one query chunk in one launch (see xattn.h).

    segments: list of dicts with keys k, kv_start, v_token_offset, block_mask (or None), causal, out, lse and
    optionally mask_kb_offset, mask_head_stride, mask_row_stride.  ws: the work-order buffer
    (bsa_prefill_segments_workspace_size bytes; allocated here when None).  Returns [(out, lse), ...].
    """
    _qkv_check(q, "q")
    dt = _dtype_code(q)
    q_len, hq, d = q.shape
    arr = (Segment * len(segments))()
    keep = []
    if not segments:
        raise XattnError(XA_EINVAL, "bsa_prefill_segments: no segments")
    out_dtype = segments[0]["out"].dtype
    for i, g in enumerate(segments):
        k = g["k"]
        _qkv_check(k, "k")
        if k.device != q.device or k.dtype != q.dtype:
            raise XattnError(XA_EINVAL, f"segment {i}: k must be on q's device with q's dtype")
        _dense_check(g["out"], f"segment {i} out", (q_len, hq, d), out_dtype, q.device)
        _dense_check(g["lse"], f"segment {i} lse", (hq, q_len), torch.float32, q.device)
        m = g.get("block_mask")
        hs, rs = _attn_mask_strides(m, q, hq, q_len, g["kv_start"], k.shape[0], g.get("mask_kb_offset", 0), block,
                                    g.get("mask_head_stride"), g.get("mask_row_stride"))
        arr[i] = Segment(k.data_ptr(), k.stride(0), k.stride(1), k.shape[0], g["kv_start"], g["v_token_offset"],
                         None if m is None else m.data_ptr(), hs, rs, g.get("mask_kb_offset", 0),
                         1 if g["causal"] else 0, g["out"].data_ptr(), g["lse"].data_ptr())
        keep.append((g["out"], g["lse"]))
    odt = _dtype_code(segments[0]["out"])
    if ws is None:
        ws = workspace(bsa_prefill_segments_workspace_size(q_len, hq, d, len(segments)), q.device)
    _check(lib().bsa_prefill_segments(_ptr(q), q.stride(0), q.stride(1), _ptr(packed.buf), packed.capacity, dt,
                                      q_len, hq, packed.hkv, d, q_start_pos, arr, len(segments), block,
                                      float(softmax_scale), odt, _ptr(ws), ws.numel(), _stream(stream)))
    return keep


def xattn_downsample_keys(k, stride: int, k_ds, ds_offset: int = 0, stream=None):
    """Rows ds_offset .. ds_offset + len(k)/stride - 1 of k_ds [capacity, Hkv, d] become K[::stride]."""
    _qkv_check(k, "k")
    n, hkv, d = k.shape
    if not k_ds.is_cuda or not k_ds.is_contiguous() or k_ds.dim() != 3 or k_ds.dtype != k.dtype:
        raise XattnError(XA_EINVAL, "k_ds must be a contiguous GPU tensor [capacity, Hkv, d] of k's dtype")
    _check(lib().xattn_downsample_keys(_ptr(k), k.stride(0), k.stride(1), _dtype_code(k), n, hkv, d, stride,
                                       _ptr(k_ds), k_ds.shape[0], ds_offset, _stream(stream)))
    return k_ds


def xattn_estimate_history_ds_workspace_size(q_len, n_ds, num_q_heads, num_kv_heads, head_dim, stride, block=128,
                                             dtype=XA_BF16) -> int:
    return int(lib().xattn_estimate_history_ds_workspace_size(q_len, n_ds, num_q_heads, num_kv_heads, head_dim,
                                                              stride, block, dtype))


def xattn_estimate_history_ds(q, k_ds, stride: int, threshold: float, block: int = 128, block_scores=None,
                              block_mask=None, ws=None, stream=None):
    """Estimate of a query chunk against downsampled history keys (see xattn.h).  Returns (scores, mask)."""
    _qkv_check(q, "q")
    _qkv_check(k_ds, "k_ds")
    q_len, hq, d = q.shape
    n_ds, hkv, _ = k_ds.shape
    b = block // stride
    dt = _dtype_code(q)
    if block_scores is None:
        block_scores = torch.empty(hq, q_len // b, n_ds // b, dtype=torch.float32, device=q.device)
    if block_mask is None:
        block_mask = torch.empty(hq, q_len // b, n_ds // b, dtype=torch.uint8, device=q.device)
    _dense_check(block_scores, "block_scores", (hq, q_len // b, n_ds // b), torch.float32, q.device)
    _dense_check(block_mask, "block_mask", (hq, q_len // b, n_ds // b), torch.uint8, q.device)
    if ws is None:
        ws = workspace(xattn_estimate_history_ds_workspace_size(q_len, n_ds, hq, hkv, d, stride, block, dt),
                       q.device)
    _check(lib().xattn_estimate_history_ds(_ptr(q), q.stride(0), q.stride(1), _ptr(k_ds), k_ds.stride(0),
                                           k_ds.stride(1), dt, q_len, n_ds, hq, hkv, d, stride, block,
                                           float(threshold), _ptr(block_scores), _ptr(block_mask), _ptr(ws),
                                           ws.numel(), _stream(stream)))
    return block_scores, block_mask


class OffloadedKV:
    """Host store of K / packed-V cache blocks (pinned) and the device ring (see xattn.h).

    n_blocks cache blocks of cache_block tokens; the ring holds 2 * group blocks; staging holds the packed V of
    up to max_offload_blocks blocks per xattn_offload_blocks call.
    """

    def __init__(self, n_blocks: int, num_kv_heads: int, head_dim: int, device, cache_block: int = 1024,
                 group: int = 8, max_offload_blocks: int = 8):
        self.n_blocks, self.hkv, self.d = n_blocks, num_kv_heads, head_dim
        self.cache_block, self.group, self.max_offload = cache_block, group, max_offload_blocks
        elems = cache_block * num_kv_heads * head_dim
        self.host_k = torch.empty(n_blocks * elems, dtype=torch.bfloat16, pin_memory=True)
        self.host_vt = torch.empty(n_blocks * elems, dtype=torch.bfloat16, pin_memory=True)
        self.ring_k = torch.empty(2 * group * cache_block, num_kv_heads, head_dim, dtype=torch.bfloat16,
                                  device=device)
        self.ring_vt = workspace(2 * group * elems * 2, device)
        self.staging = workspace(max_offload_blocks * elems * 2, device)
        self.copy_stream = torch.cuda.Stream(device)


def xattn_offload_blocks(store: OffloadedKV, k, v, first_block: int, stream=None):
    """Store the cache blocks of k / v (device, len a multiple of cache_block) as host blocks first_block ..."""
    _qkv_check(k, "k")
    _qkv_check(v, "v")
    n = k.shape[0] // store.cache_block
    if n * store.cache_block != k.shape[0] or n > store.max_offload or first_block + n > store.n_blocks:
        raise XattnError(XA_EINVAL, "offload: whole cache blocks, at most max_offload_blocks, within the store")
    _check(lib().xattn_offload_blocks(_ptr(k), k.stride(0), k.stride(1), _ptr(v), v.stride(0), v.stride(1),
                                      _dtype_code(k), n, store.hkv, store.d, store.cache_block,
                                      ctypes.c_void_p(store.host_k.data_ptr()),
                                      ctypes.c_void_p(store.host_vt.data_ptr()), store.n_blocks, first_block,
                                      _ptr(store.staging), _stream(stream)))


def bsa_history_offloaded(q, q_start_pos: int, store: OffloadedKV, keep, out, lse, part_out, part_lse,
                          stream=None):
    """Attention of q over the host cache blocks `keep` (ids, no causal rule) through the ring (see xattn.h)."""
    _qkv_check(q, "q")
    q_len, hq, d = q.shape
    for t, nm in ((out, "out"), (part_out, "part_out")):
        _dense_check(t, nm, (q_len, hq, d), torch.bfloat16, q.device)
    for t, nm in ((lse, "lse"), (part_lse, "part_lse")):
        _dense_check(t, nm, (hq, q_len), torch.float32, q.device)
    if any(int(i) < 0 or int(i) >= store.n_blocks for i in keep):
        raise XattnError(XA_EINVAL, "keep ids must lie in the host store")
    ids = (ctypes.c_int32 * max(len(keep), 1))(*[int(i) for i in keep])
    _check(lib().bsa_history_offloaded(_ptr(q), q.stride(0), q.stride(1), _dtype_code(q), q_len, hq, store.hkv, d,
                                       q_start_pos, ctypes.c_void_p(store.host_k.data_ptr()),
                                       ctypes.c_void_p(store.host_vt.data_ptr()), store.n_blocks,
                                       store.cache_block, ids, len(keep), store.group, _ptr(store.ring_k),
                                       _ptr(store.ring_vt), _ptr(out), _ptr(lse), _ptr(part_out), _ptr(part_lse),
                                       _stream(stream), store.copy_stream.cuda_stream))
    return out, lse


def xattn_estimate_offloaded(q, k_cur, q_start_pos: int, store: OffloadedKV, stride: int = 8,
                             threshold: float = 0.9, block: int = 128, block_scores=None, block_mask=None, ws=None,
                             stream=None):
    """xattn_estimate of q against host cache blocks 0 .. q_start_pos/cache_block - 1 of store and the chunk's
    own keys k_cur, the history streamed through the store's ring (see xattn.h).  Returns (scores, mask)."""
    _qkv_check(q, "q")
    _qkv_check(k_cur, "k_cur")
    q_len, hq, d = q.shape
    k_len = q_start_pos + q_len
    n_qb, nkb = q_len // block, k_len // block
    if block_scores is None:
        block_scores = torch.empty(hq, n_qb, nkb, dtype=torch.float32, device=q.device)
    if block_mask is None:
        block_mask = torch.empty(hq, n_qb, nkb, dtype=torch.uint8, device=q.device)
    if ws is None:
        ws = workspace(xattn_estimate_workspace_size(q_len, k_len, hq, store.hkv, d, stride, block, XA_BF16),
                       q.device)
    _check(lib().xattn_estimate_offloaded(_ptr(q), q.stride(0), q.stride(1), _ptr(k_cur), k_cur.stride(0),
                                          k_cur.stride(1), _dtype_code(q), q_len, hq, store.hkv, d, q_start_pos,
                                          ctypes.c_void_p(store.host_k.data_ptr()), store.n_blocks,
                                          store.cache_block, store.group, _ptr(store.ring_k), stride, block,
                                          float(threshold), _ptr(block_scores), _ptr(block_mask), _ptr(ws),
                                          ws.numel(), _stream(stream), store.copy_stream.cuda_stream))
    return block_scores, block_mask


def _cu(cu):
    vals = [int(x) for x in (cu.tolist() if hasattr(cu, "tolist") else cu)]
    return (ctypes.c_int64 * len(vals))(*vals), len(vals) - 1


def xattn_varlen_mask_elems(cu_seqlens_q, cu_seqlens_k, num_q_heads: int) -> int:
    cq, b = _cu(cu_seqlens_q)
    ck, _ = _cu(cu_seqlens_k)
    return int(lib().xattn_varlen_mask_elems(cq, ck, b, num_q_heads))


def xattn_estimate_varlen_workspace_size(cu_seqlens_q, cu_seqlens_k, num_q_heads, num_kv_heads, stride) -> int:
    cq, b = _cu(cu_seqlens_q)
    ck, _ = _cu(cu_seqlens_k)
    return int(lib().xattn_estimate_varlen_workspace_size(cq, ck, b, num_q_heads, num_kv_heads, stride))


def bsa_prefill_varlen_workspace_size(cu_seqlens_q, cu_seqlens_k, num_q_heads, head_dim) -> int:
    cq, b = _cu(cu_seqlens_q)
    ck, _ = _cu(cu_seqlens_k)
    return int(lib().bsa_prefill_varlen_workspace_size(cq, ck, b, num_q_heads, head_dim))


def varlen_blocks(flat, cu_seqlens_q, cu_seqlens_k, num_q_heads: int, block: int = 128):
    """Per-sequence [Hq, q_len/block, k_len/block] views of a packed-batch scores or mask buffer."""
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    out, off = [], 0
    for b in range(len(cq) - 1):
        nq, nk = (cq[b + 1] - cq[b]) // block, (ck[b + 1] - ck[b]) // block
        n = num_q_heads * nq * nk
        out.append(flat[off:off + n].view(num_q_heads, nq, nk))
        off += n
    return out


def varlen_lse(flat, cu_seqlens_q, num_q_heads: int):
    """Per-sequence [Hq, q_len] views of a packed-batch LSE buffer."""
    cq = [int(x) for x in cu_seqlens_q]
    return [flat[num_q_heads * cq[b]:num_q_heads * cq[b + 1]].view(num_q_heads, cq[b + 1] - cq[b])
            for b in range(len(cq) - 1)]


def xattn_estimate_varlen(q, k, cu_seqlens_q, cu_seqlens_k, stride: int = 8, threshold: float = 0.9,
                          block: int = 128, block_scores=None, block_mask=None, ws=None, stream=None):
    """Estimate of every sequence of a packed batch (see xattn.h).  Returns flat (scores, mask)."""
    _qkv_check(q, "q")
    _qkv_check(k, "k")
    _, hq, d = q.shape
    hkv = k.shape[1]
    cq, b = _cu(cu_seqlens_q)
    ck, _ = _cu(cu_seqlens_k)
    n = int(lib().xattn_varlen_mask_elems(cq, ck, b, hq))
    if n < 0:
        raise XattnError(XA_EINVAL, "invalid packed-batch lengths")
    if block_scores is None:
        block_scores = torch.empty(max(n, 1), dtype=torch.float32, device=q.device)
    if block_mask is None:
        block_mask = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _flat_check(block_scores, "block_scores", n, torch.float32, q.device)
    _flat_check(block_mask, "block_mask", n, torch.uint8, q.device)
    if ws is None:
        ws = workspace(lib().xattn_estimate_varlen_workspace_size(cq, ck, b, hq, hkv, stride), q.device)
    _check(lib().xattn_estimate_varlen(_ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1),
                                       _dtype_code(q), cq, ck, b, hq, hkv, d, stride, block, float(threshold),
                                       _ptr(block_scores), _ptr(block_mask), _ptr(ws), ws.numel(), _stream(stream)))
    return block_scores, block_mask


def bsa_prefill_varlen(q, k, packed: PackedV, cu_seqlens_q, cu_seqlens_k, block_mask=None, softmax_scale=0.0,
                       out_dtype=None, block: int = 128, out=None, lse=None, ws=None, stream=None):
    """Causal block-sparse attention of every sequence of a packed batch (see xattn.h).  Returns (out, flat lse)."""
    _qkv_check(q, "q")
    _qkv_check(k, "k")
    total_q, hq, d = q.shape
    hkv = k.shape[1]
    cq, b = _cu(cu_seqlens_q)
    ck, _ = _cu(cu_seqlens_k)
    odt = _out_dtype(out, out_dtype, q.dtype)
    if out is None:
        out = torch.empty(total_q, hq, d, dtype=odt, device=q.device)
    if lse is None:
        lse = torch.empty(max(hq * total_q, 1), dtype=torch.float32, device=q.device)
    _dense_check(out, "out", (total_q, hq, d), odt, q.device)
    _flat_check(lse, "lse", hq * total_q, torch.float32, q.device)
    if block_mask is not None:
        _flat_check(block_mask, "block_mask", int(lib().xattn_varlen_mask_elems(cq, ck, b, hq)),
                    block_mask.dtype if block_mask.dtype == torch.bool else torch.uint8, q.device)
    if ws is None:
        ws = workspace(lib().bsa_prefill_varlen_workspace_size(cq, ck, b, hq, d), q.device)
    _check(lib().bsa_prefill_varlen(_ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1),
                                    _ptr(packed.buf), packed.capacity, _dtype_code(q), cq, ck, b, hq, hkv, d,
                                    _ptr(block_mask) if block_mask is not None else None, block,
                                    float(softmax_scale), _ptr(out), _dtype_code(out), _ptr(lse), _ptr(ws),
                                    ws.numel(), _stream(stream)))
    return out, lse


def attn_merge(o_a, lse_a, o_b, lse_b, o_out=None, lse_out=None, stream=None):
    """LSE merge (see xattn.h); o_out / lse_out may alias the inputs.  Returns (o, lse)."""
    if o_a.dim() != 3:
        raise XattnError(XA_EINVAL, "attn_merge: o_a must be [q_len, heads, head_dim]")
    q_len, heads, d = o_a.shape
    if o_out is None:
        o_out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    for t, nm in ((o_a, "o_a"), (o_b, "o_b"), (o_out, "o_out")):
        _dense_check(t, nm, (q_len, heads, d), o_a.dtype, o_a.device)
    for t, nm in ((lse_a, "lse_a"), (lse_b, "lse_b"), (lse_out, "lse_out")):
        _dense_check(t, nm, (heads, q_len), torch.float32, o_a.device)
    _check(lib().attn_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o_out), _ptr(lse_out),
                            _dtype_code(o_a), q_len, heads, d, _stream(stream)))
    return o_out, lse_out


def xattn_mask_to_cache_blocks(block_mask, kb_begin: int, n_cache_blocks: int, sub_blocks: int = 8,
                               force_first_last: bool = True, keep_per_head=None, keep_any=None,
                               keep_any_blocks=None, want=("per_head", "any", "any_blocks"), stream=None):
    """Reduce a [H, n_qb, n_cols] block mask to cache blocks.  Returns (per_head, any, any_blocks)."""
    H, n_qb, n_cols = block_mask.shape
    dev = block_mask.device
    _mask_check(block_mask, "block_mask", dev, H, n_qb, 0, n_cols - 1)
    if keep_per_head is None and "per_head" in want:
        keep_per_head = torch.empty(H, n_qb, n_cache_blocks, dtype=torch.uint8, device=dev)
    if keep_any is None and "any" in want:
        keep_any = torch.empty(n_cache_blocks, dtype=torch.uint8, device=dev)
    if keep_any_blocks is None and "any_blocks" in want:
        keep_any_blocks = torch.empty(n_cache_blocks * sub_blocks, dtype=torch.uint8, device=dev)
    _dense_check(keep_per_head, "keep_per_head", (H, n_qb, n_cache_blocks), torch.uint8, dev)
    _dense_check(keep_any, "keep_any", (n_cache_blocks,), torch.uint8, dev)
    _dense_check(keep_any_blocks, "keep_any_blocks", (n_cache_blocks * sub_blocks,), torch.uint8, dev)
    _check(lib().xattn_mask_to_cache_blocks(_ptr(block_mask), H, n_qb, n_cols, block_mask.stride(0),
                                            block_mask.stride(1), kb_begin, n_cache_blocks, sub_blocks,
                                            1 if force_first_last else 0, _ptr(keep_per_head), _ptr(keep_any),
                                            _ptr(keep_any_blocks), _stream(stream)))
    return keep_per_head, keep_any, keep_any_blocks


def xattn_density_counts(counts, block_mask=None, diag0: int = 0, keep_any=None, stream=None):
    """Add a chunk's density counts to `counts` (int64 [4] on the GPU; see xattn.h):
    [kept causal pairs, causal pairs, kept cache blocks, cache blocks].

    block_mask: [H, n_qb, n_cols] uint8 (query block qb's causal columns are 0 .. diag0 + qb), or None;
    keep_any: [n_cache_blocks] uint8, or None.  Returns counts.
    """
    if not counts.is_cuda or counts.dtype != torch.int64 or counts.numel() < 4 or not counts.is_contiguous():
        raise XattnError(XA_EINVAL, "counts must be a contiguous int64 GPU tensor of at least 4 elements")
    H = n_qb = n_cols = hs = rs = 0
    if block_mask is not None:
        _mask_check(block_mask, "block_mask", counts.device)
        H, n_qb, n_cols = block_mask.shape
        hs, rs = block_mask.stride(0), block_mask.stride(1)
    ncb = 0
    if keep_any is not None:
        if not keep_any.is_cuda or keep_any.dtype not in (torch.uint8, torch.bool) or not keep_any.is_contiguous():
            raise XattnError(XA_EINVAL, "keep_any must be a contiguous uint8/bool GPU tensor")
        ncb = keep_any.numel()
    _check(lib().xattn_density_counts(_ptr(block_mask), H, n_qb, n_cols, hs, rs, diag0, _ptr(keep_any), ncb,
                                      _ptr(counts), _stream(stream)))
    return counts

