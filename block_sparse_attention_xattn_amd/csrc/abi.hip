// C ABI layer: argument validation, workspace carving and kernel launches for
// xattn_estimate and bsa_prefill, plus the error/version helpers.  Every check
// runs before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "launchers.h"

namespace xa_host {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

xa_status_t fail(xa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

xa_status_t check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(XA_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return XA_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace xa_host

using namespace xa;
using xa_host::align256;
using xa_host::fail;

extern "C" const char* xattn_last_error(void) { return xa_host::g_err; }
extern "C" const char* xattn_version(void) { return "xattn-gfx950 0.1"; }

// ---------------------------------------------------------------------------
// shared validation
// ---------------------------------------------------------------------------
static xa_status_t check_heads(const char* fn, int32_t hq, int32_t hkv, int32_t d) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
    return fail(XA_EINVAL, "%s: num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", fn, hq, hkv);
  if (d != 64 && d != 128) return fail(XA_EUNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn, d);
  return XA_OK;
}

static xa_status_t check_tensor(const char* fn, const char* name, const void* p, int64_t tok, int64_t head,
                                int64_t len, int32_t heads, int32_t d, xa_dtype_t dt) {
  if (!p) return fail(XA_EINVAL, "%s: %s is null", fn, name);
  if (tok < 0 || head < 0) return fail(XA_EINVAL, "%s: %s has a negative stride", fn, name);
  if (tok % 8 != 0 || head % 8 != 0 || (uintptr_t)p % 16 != 0)
    return fail(XA_EINVAL, "%s: %s must be 16-byte aligned with strides that are multiples of 8 elements", fn,
                name);
  if (len > 1 && tok < (int64_t)heads * d && head < d)
    return fail(XA_EINVAL, "%s: %s strides overlap rows", fn, name);
  (void)dt;
  return XA_OK;
}

// ---------------------------------------------------------------------------
// xattn_estimate
// ---------------------------------------------------------------------------
namespace {
struct EstLayout {
  size_t lse_off, lse_bytes, qh_off, ql_off, kh_off, kl_off, plane_q, plane_k, total;
};

EstLayout est_layout(int64_t q_len, int64_t k_len, int32_t hq, int32_t hkv, int32_t d, int32_t stride,
                     int32_t block, xa_dtype_t dt) {
  EstLayout L{};
  const int64_t R = q_len / stride;
  const int64_t nkb = k_len / block;
  L.lse_off = 0;
  L.lse_bytes = align256((size_t)hq * nkb * R * sizeof(float));
  size_t off = L.lse_bytes;
  if (dt == XA_F32) {
    L.plane_q = align256((size_t)q_len * hq * d * 2);
    L.plane_k = align256((size_t)k_len * hkv * d * 2);
    L.qh_off = off;
    off += L.plane_q;
    L.ql_off = off;
    off += L.plane_q;
    L.kh_off = off;
    off += L.plane_k;
    L.kl_off = off;
    off += L.plane_k;
  }
  L.total = off;
  return L;
}
}  // namespace

extern "C" size_t xattn_estimate_workspace_size(int64_t q_len, int64_t k_len, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim, int32_t stride,
                                                int32_t block, xa_dtype_t dtype) {
  if (q_len <= 0 || k_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || stride <= 0 ||
      block <= 0)
    return 0;
  return est_layout(q_len, k_len, num_q_heads, num_kv_heads, head_dim, stride, block, dtype).total;
}

extern "C" xa_status_t xattn_estimate(const void* q, int64_t q_tok, int64_t q_head, const void* k, int64_t k_tok,
                                      int64_t k_head, xa_dtype_t dtype, int64_t q_len, int64_t k_len,
                                      int32_t hq, int32_t hkv, int32_t d, int64_t q_start, int32_t stride,
                                      int32_t block, float threshold, float* block_scores, uint8_t* block_mask,
                                      void* workspace, size_t ws_bytes, xa_stream_t stream) {
  const char* fn = "xattn_estimate";
  xa_status_t st;
  if ((st = check_heads(fn, hq, hkv, d)) != XA_OK) return st;
  if (dtype != XA_F32 && dtype != XA_BF16) return fail(XA_EUNSUPPORTED, "%s: dtype must be XA_F32 or XA_BF16", fn);
  if (block != 128) return fail(XA_EUNSUPPORTED, "%s: block must be 128 (got %d)", fn, block);
  if (stride != 2 && stride != 4 && stride != 8 && stride != 16)
    return fail(XA_EUNSUPPORTED, "%s: stride %d not in {2, 4, 8, 16}", fn, stride);
  if (q_len <= 0 || q_len % block != 0) return fail(XA_EINVAL, "%s: q_len %lld must be a positive multiple of %d", fn, (long long)q_len, block);
  if (q_start < 0 || q_start % block != 0) return fail(XA_EINVAL, "%s: q_start_pos %lld must be a non-negative multiple of %d", fn, (long long)q_start, block);
  if (k_len != q_start + q_len) return fail(XA_EINVAL, "%s: k_len %lld != q_start_pos + q_len = %lld", fn, (long long)k_len, (long long)(q_start + q_len));
  if (k_len / block > 8192) return fail(XA_EUNSUPPORTED, "%s: k_len / block = %lld exceeds 8192 key blocks", fn, (long long)(k_len / block));
  if (!(threshold >= 0.f) || isnan(threshold)) return fail(XA_EINVAL, "%s: threshold must be >= 0", fn);
  if ((st = check_tensor(fn, "q", q, q_tok, q_head, q_len, hq, d, dtype)) != XA_OK) return st;
  if ((st = check_tensor(fn, "k", k, k_tok, k_head, k_len, hkv, d, dtype)) != XA_OK) return st;
  if (!block_scores || !block_mask) return fail(XA_EINVAL, "%s: block_scores and block_mask are required", fn);
  const EstLayout L = est_layout(q_len, k_len, hq, hkv, d, stride, block, dtype);
  if (!workspace || ws_bytes < L.total || (uintptr_t)workspace % 256 != 0)
    return fail(XA_EWORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, L.total,
                ws_bytes);
  const int64_t R = q_len / stride, N = k_len / stride, nkb = k_len / block;
  if ((int64_t)hq * nkb * R > ((int64_t)1 << 40)) return fail(XA_EUNSUPPORTED, "%s: problem too large", fn);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  EstParams p{};
  p.q_len = q_len;
  p.k_len = k_len;
  p.q_start = q_start;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.S = stride;
  p.b = block / stride;
  p.R = (int)R;
  p.N = (int)N;
  p.nkb = (int)nkb;
  p.n_rt = (int)((R + 127) / 128);
  p.n_ct = (int)((N + 127) / 128);
  p.scale_log2 = kLog2e / ((float)stride * sqrtf((float)d));
  p.lse_part = reinterpret_cast<float*>(ws + L.lse_off);
  hipError_t e;
  if (dtype == XA_BF16) {
    p.q_hi = static_cast<const bf16*>(q);
    p.k_hi = static_cast<const bf16*>(k);
    p.q_tok = q_tok;
    p.q_head = q_head;
    p.k_tok = k_tok;
    p.k_head = k_head;
  } else {
    bf16* qh = reinterpret_cast<bf16*>(ws + L.qh_off);
    bf16* ql = reinterpret_cast<bf16*>(ws + L.ql_off);
    bf16* kh = reinterpret_cast<bf16*>(ws + L.kh_off);
    bf16* kl = reinterpret_cast<bf16*>(ws + L.kl_off);
    if ((e = launch_split((const float*)q, q_tok, q_head, q_len, hq, d, qh, ql, s)) != hipSuccess ||
        (e = launch_split((const float*)k, k_tok, k_head, k_len, hkv, d, kh, kl, s)) != hipSuccess)
      return fail(XA_EHIP, "%s: split launch failed: %s", fn, hipGetErrorString(e));
    p.q_hi = qh;
    p.q_lo = ql;
    p.k_hi = kh;
    p.k_lo = kl;
    p.q_tok = (int64_t)hq * d;
    p.q_head = d;
    p.k_tok = (int64_t)hkv * d;
    p.k_head = d;
  }
  const int64_t grid = (int64_t)hkv * p.n_ct * p.n_rt * p.group;
  if (grid > 0x7fffffff) return fail(XA_EUNSUPPORTED, "%s: grid too large", fn);
  if (d == 128)
    e = dtype == XA_BF16 ? launch_est_gemm<128, false>(p, s) : launch_est_gemm<128, true>(p, s);
  else
    e = dtype == XA_BF16 ? launch_est_gemm<64, false>(p, s) : launch_est_gemm<64, true>(p, s);
  if (e != hipSuccess) return fail(XA_EHIP, "%s: estimate GEMM launch failed: %s", fn, hipGetErrorString(e));
  SelParams sp{};
  sp.lse_part = p.lse_part;
  sp.R = p.R;
  sp.nkb = p.nkb;
  sp.b = p.b;
  sp.hq = hq;
  sp.n_qb = (int)(q_len / block);
  sp.cur = q_start / block;
  sp.threshold = threshold;
  sp.scores = block_scores;
  sp.mask = block_mask;
  if ((e = launch_est_select(sp, s)) != hipSuccess)
    return fail(XA_EHIP, "%s: selection launch failed: %s", fn, hipGetErrorString(e));
  return XA_OK;
}

// ---------------------------------------------------------------------------
// bsa_prefill
// ---------------------------------------------------------------------------
namespace {
struct BsaLayout {
  size_t vh_off, vl_off, qh_off, ql_off, kh_off, kl_off, total;
  int64_t pitch;
};

BsaLayout bsa_layout(int64_t q_len, int64_t kv_len, int32_t hq, int32_t hkv, int32_t d, xa_dtype_t dt) {
  BsaLayout L{};
  L.pitch = (kv_len + 127) / 128 * 128;
  const size_t vt = align256((size_t)hkv * d * L.pitch * 2);
  size_t off = 0;
  L.vh_off = off;
  off += vt;
  if (dt == XA_F32) {
    L.vl_off = off;
    off += vt;
    const size_t pq = align256((size_t)q_len * hq * d * 2);
    const size_t pk = align256((size_t)kv_len * hkv * d * 2);
    L.qh_off = off;
    off += pq;
    L.ql_off = off;
    off += pq;
    L.kh_off = off;
    off += pk;
    L.kl_off = off;
    off += pk;
  }
  L.total = off;
  return L;
}
}  // namespace

extern "C" size_t bsa_prefill_workspace_size(int64_t q_len, int64_t kv_len, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, xa_dtype_t dtype) {
  if (q_len <= 0 || kv_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  return bsa_layout(q_len, kv_len, num_q_heads, num_kv_heads, head_dim, dtype).total;
}

extern "C" xa_status_t bsa_prefill(const void* q, int64_t q_tok, int64_t q_head, const void* k, int64_t k_tok,
                                   int64_t k_head, const void* v, int64_t v_tok, int64_t v_head, xa_dtype_t dtype,
                                   int64_t q_len, int64_t kv_len, int32_t hq, int32_t hkv, int32_t d,
                                   int64_t q_start, int64_t kv_start, const uint8_t* block_mask,
                                   int64_t mask_hs, int64_t mask_rs, int64_t mask_off, int32_t block,
                                   int32_t causal, float softmax_scale, void* out, xa_dtype_t out_dtype,
                                   float* lse, void* workspace, size_t ws_bytes, xa_stream_t stream) {
  const char* fn = "bsa_prefill";
  xa_status_t st;
  if ((st = check_heads(fn, hq, hkv, d)) != XA_OK) return st;
  if (dtype != XA_F32 && dtype != XA_BF16) return fail(XA_EUNSUPPORTED, "%s: dtype must be XA_F32 or XA_BF16", fn);
  if (out_dtype != XA_F32 && out_dtype != XA_BF16)
    return fail(XA_EUNSUPPORTED, "%s: out_dtype must be XA_F32 or XA_BF16", fn);
  if (block != 128) return fail(XA_EUNSUPPORTED, "%s: block must be 128 (got %d)", fn, block);
  if (q_len <= 0 || q_len % block != 0) return fail(XA_EINVAL, "%s: q_len %lld must be a positive multiple of %d", fn, (long long)q_len, block);
  if (kv_len <= 0) return fail(XA_EINVAL, "%s: kv_len must be positive", fn);
  if (q_start < 0 || q_start % block != 0 || kv_start < 0 || kv_start % block != 0)
    return fail(XA_EINVAL, "%s: q_start_pos and kv_start must be non-negative multiples of %d", fn, block);
  if ((st = check_tensor(fn, "q", q, q_tok, q_head, q_len, hq, d, dtype)) != XA_OK) return st;
  if ((st = check_tensor(fn, "k", k, k_tok, k_head, kv_len, hkv, d, dtype)) != XA_OK) return st;
  if ((st = check_tensor(fn, "v", v, v_tok, v_head, kv_len, hkv, d, dtype)) != XA_OK) return st;
  if (block_mask && (mask_hs < 0 || mask_rs < 0)) return fail(XA_EINVAL, "%s: negative mask stride", fn);
  if (block_mask && kv_start / block - mask_off < 0)
    return fail(XA_EINVAL, "%s: mask_kb_offset %lld is past the first key block %lld", fn, (long long)mask_off,
                (long long)(kv_start / block));
  if (!out || !lse) return fail(XA_EINVAL, "%s: out and lse are required", fn);
  if ((uintptr_t)out % 16 != 0) return fail(XA_EINVAL, "%s: out must be 16-byte aligned", fn);
  if (!(softmax_scale >= 0.f)) return fail(XA_EINVAL, "%s: softmax_scale must be >= 0 (0 = 1/sqrt(d))", fn);
  const BsaLayout L = bsa_layout(q_len, kv_len, hq, hkv, d, dtype);
  if (!workspace || ws_bytes < L.total || (uintptr_t)workspace % 256 != 0)
    return fail(XA_EWORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, L.total,
                ws_bytes);
  const int64_t n_qb = q_len / block;
  if ((int64_t)hq * n_qb > 0x7fffffff) return fail(XA_EUNSUPPORTED, "%s: grid too large", fn);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d);
  BsaParams p{};
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.n_qb = (int)n_qb;
  p.q_start = q_start;
  p.kv_start = kv_start;
  p.mask = block_mask;
  p.mask_hs = mask_hs;
  p.mask_rs = mask_rs;
  p.mask_off = mask_off;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * kLog2e;
  p.out = out;
  p.lse = lse;
  p.vt_pitch = L.pitch;
  p.vt_head = (int64_t)d * L.pitch;
  bf16* vh = reinterpret_cast<bf16*>(ws + L.vh_off);
  bf16* vl = dtype == XA_F32 ? reinterpret_cast<bf16*>(ws + L.vl_off) : nullptr;
  hipError_t e = launch_vt(v, dtype, v_tok, v_head, kv_len, hkv, d, vh, vl, L.pitch, s);
  if (e != hipSuccess) return fail(XA_EHIP, "%s: V transpose launch failed: %s", fn, hipGetErrorString(e));
  p.vt_hi = vh;
  p.vt_lo = vl;
  if (dtype == XA_BF16) {
    p.q_hi = static_cast<const bf16*>(q);
    p.k_hi = static_cast<const bf16*>(k);
    p.q_tok = q_tok;
    p.q_head = q_head;
    p.k_tok = k_tok;
    p.k_head = k_head;
  } else {
    bf16* qh = reinterpret_cast<bf16*>(ws + L.qh_off);
    bf16* ql = reinterpret_cast<bf16*>(ws + L.ql_off);
    bf16* kh = reinterpret_cast<bf16*>(ws + L.kh_off);
    bf16* kl = reinterpret_cast<bf16*>(ws + L.kl_off);
    if ((e = launch_split((const float*)q, q_tok, q_head, q_len, hq, d, qh, ql, s)) != hipSuccess ||
        (e = launch_split((const float*)k, k_tok, k_head, kv_len, hkv, d, kh, kl, s)) != hipSuccess)
      return fail(XA_EHIP, "%s: split launch failed: %s", fn, hipGetErrorString(e));
    p.q_hi = qh;
    p.q_lo = ql;
    p.k_hi = kh;
    p.k_lo = kl;
    p.q_tok = (int64_t)hq * d;
    p.q_head = d;
    p.k_tok = (int64_t)hkv * d;
    p.k_head = d;
  }
  const bool split = dtype == XA_F32;
  const bool obf = out_dtype == XA_BF16;
  if (d == 128) {
    if (split) e = obf ? launch_bsa<128, true, bf16>(p, s) : launch_bsa<128, true, float>(p, s);
    else e = obf ? launch_bsa<128, false, bf16>(p, s) : launch_bsa<128, false, float>(p, s);
  } else {
    if (split) e = obf ? launch_bsa<64, true, bf16>(p, s) : launch_bsa<64, true, float>(p, s);
    else e = obf ? launch_bsa<64, false, bf16>(p, s) : launch_bsa<64, false, float>(p, s);
  }
  if (e != hipSuccess) return fail(XA_EHIP, "%s: attention launch failed: %s", fn, hipGetErrorString(e));
  return XA_OK;
}
