// C ABI layer: argument validation, workspace carving and kernel launches for
// xattn_estimate and bsa_prefill, plus the error/version helpers.  Every check
// runs before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <vector>

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

extern "C" xa_status_t xattn_set_attention_events(xa_event_t before, xa_event_t after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(XA_EINVAL, "xattn_set_attention_events: pass both events or neither");
  set_attention_events(reinterpret_cast<hipEvent_t>(before), reinterpret_cast<hipEvent_t>(after));
  return XA_OK;
}

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
  // rows must not alias: token-major (heads of a token side by side, tokens after them) or head-major
  // (tokens of a head side by side, heads after them); a stride along an axis of length 1 is never used
  const bool one_tok = len <= 1, one_head = heads <= 1;
  bool disjoint;
  if (one_tok && one_head) disjoint = true;
  else if (one_tok) disjoint = head >= d;
  else if (one_head) disjoint = tok >= d;
  else disjoint = (head >= d && tok >= (int64_t)heads * head) || (tok >= d && head >= len * tok);
  if (!disjoint) return fail(XA_EINVAL, "%s: %s strides overlap rows", fn, name);
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

namespace {
// Estimate GEMM (reshaped by stride S, b rows per query block) + selection.
// q_start_eff fixes the causal limit of reshaped column c for row r:
// c <= q_start_eff / S + r.  hist_only: all key blocks visible, block 0 the
// only forced block.
xa_status_t estimate_core(const char* fn, const void* q, int64_t q_tok, int64_t q_head, const void* k, int64_t k_tok,
                          int64_t k_head, xa_dtype_t dtype, int64_t q_len, int64_t k_len, int32_t hq, int32_t hkv,
                          int32_t d, int32_t stride, int32_t b, int64_t q_start_eff, int64_t n_qb, int64_t cur,
                          bool hist_only, float threshold, float* block_scores, uint8_t* block_mask, char* ws,
                          const EstLayout& L, hipStream_t s) {
  const int64_t R = q_len / stride, N = k_len / stride, nkb = N / b;
  EstParams p{};
  p.q_len = q_len;
  p.k_len = k_len;
  p.q_start = q_start_eff;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.S = stride;
  p.b = b;
  p.R = (int)R;
  p.N = (int)N;
  p.nkb = (int)nkb;
  p.nkb_ld = (int)nkb;
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
  sp.npow_cap = 1;
  while (sp.npow_cap < p.nkb) sp.npow_cap <<= 1;
  sp.b = p.b;
  sp.hq = hq;
  sp.n_qb = (int)n_qb;
  sp.hist_only = hist_only ? 1 : 0;
  sp.cur = cur;
  sp.threshold = threshold;
  sp.scores = block_scores;
  sp.mask = block_mask;
  if ((e = launch_est_select(sp, s)) != hipSuccess)
    return fail(XA_EHIP, "%s: selection launch failed: %s", fn, hipGetErrorString(e));
  return XA_OK;
}
}  // namespace

namespace {
// Argument checks of xattn_estimate (everything but the workspace); fills the workspace layout.
xa_status_t validate_estimate(const char* fn, const void* q, int64_t q_tok, int64_t q_head, const void* k,
                              int64_t k_tok, int64_t k_head, xa_dtype_t dtype, int64_t q_len, int64_t k_len,
                              int32_t hq, int32_t hkv, int32_t d, int64_t q_start, int32_t stride, int32_t block,
                              float threshold, float* block_scores, uint8_t* block_mask, EstLayout& L) {
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
  const int64_t R = q_len / stride, nkb = k_len / block;
  if ((int64_t)hq * nkb * R > ((int64_t)1 << 40)) return fail(XA_EUNSUPPORTED, "%s: problem too large", fn);
  L = est_layout(q_len, k_len, hq, hkv, d, stride, block, dtype);
  return XA_OK;
}
}  // namespace

extern "C" xa_status_t xattn_estimate(const void* q, int64_t q_tok, int64_t q_head, const void* k, int64_t k_tok,
                                      int64_t k_head, xa_dtype_t dtype, int64_t q_len, int64_t k_len,
                                      int32_t hq, int32_t hkv, int32_t d, int64_t q_start, int32_t stride,
                                      int32_t block, float threshold, float* block_scores, uint8_t* block_mask,
                                      void* workspace, size_t ws_bytes, xa_stream_t stream) {
  const char* fn = "xattn_estimate";
  EstLayout L{};
  xa_status_t st = validate_estimate(fn, q, q_tok, q_head, k, k_tok, k_head, dtype, q_len, k_len, hq, hkv, d,
                                     q_start, stride, block, threshold, block_scores, block_mask, L);
  if (st != XA_OK) return st;
  if (!workspace || ws_bytes < L.total || (uintptr_t)workspace % 256 != 0)
    return fail(XA_EWORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, L.total,
                ws_bytes);
  return estimate_core(fn, q, q_tok, q_head, k, k_tok, k_head, dtype, q_len, k_len, hq, hkv, d, stride,
                       block / stride, q_start, q_len / block, q_start / block, false, threshold, block_scores,
                       block_mask, static_cast<char*>(workspace), L, reinterpret_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// xattn_estimate_noalloc: xattn_estimate with its working memory (the per-(row, key block) log-sum-exp
// partials, plus the bf16 hi / lo planes of fp32 inputs) in `scratch`, a device array of the library, so the
// caller passes no workspace and nothing is allocated.  Each device holds its own copy of the array; its
// address on a device comes from hipGetSymbolAddress, taken once per device (with that device current) and
// kept.  The array's name in host code is only a host-side handle: kernels get the kept device address.
// Nothing in the array has to start at zero (the GEMM writes every partial the selection reads), so calls
// clear nothing; calls that overlap on one device share the array and race.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices];  // device address of `scratch` on device i (null until first use)

xa_status_t device_scratch(const char* fn, hipStream_t s, char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(XA_EHIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(XA_EUNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  if (s != nullptr) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(s, &sd);
    if (e != hipSuccess) return fail(XA_EHIP, "%s: hipStreamGetDevice failed: %s", fn, hipGetErrorString(e));
    if (sd != dev)
      return fail(XA_EINVAL, "%s: the stream belongs to device %d but device %d is current", fn, (int)sd, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(XA_EHIP, "%s: hipGetSymbolAddress(scratch) failed: %s", fn, hipGetErrorString(e));
    g_scratch_dev[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_dev[dev];
  return XA_OK;
}
}  // namespace

extern "C" size_t xattn_estimate_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" xa_status_t xattn_estimate_noalloc(const void* q, int64_t q_tok, int64_t q_head, const void* k,
                                              int64_t k_tok, int64_t k_head, xa_dtype_t dtype, int64_t q_len,
                                              int64_t k_len, int32_t hq, int32_t hkv, int32_t d, int64_t q_start,
                                              int32_t stride, int32_t block, float threshold, float* block_scores,
                                              uint8_t* block_mask, xa_stream_t stream) {
  const char* fn = "xattn_estimate_noalloc";
  EstLayout L{};
  xa_status_t st = validate_estimate(fn, q, q_tok, q_head, k, k_tok, k_head, dtype, q_len, k_len, hq, hkv, d,
                                     q_start, stride, block, threshold, block_scores, block_mask, L);
  if (st != XA_OK) return st;
  if (L.total > kScratchBytes)
    return fail(XA_EUNSUPPORTED, "%s: needs %zu bytes of working memory, the library's array holds %zu", fn,
                L.total, kScratchBytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = nullptr;
  if ((st = device_scratch(fn, s, &ws)) != XA_OK) return st;
  return estimate_core(fn, q, q_tok, q_head, k, k_tok, k_head, dtype, q_len, k_len, hq, hkv, d, stride,
                       block / stride, q_start, q_len / block, q_start / block, false, threshold, block_scores,
                       block_mask, ws, L, s);
}

// ---------------------------------------------------------------------------
// Downsampled history keys and the estimate against them
// ---------------------------------------------------------------------------
extern "C" xa_status_t xattn_downsample_keys(const void* k, int64_t k_tok, int64_t k_head, xa_dtype_t dtype,
                                             int64_t n_tokens, int32_t hkv, int32_t d, int32_t stride, void* k_ds,
                                             int64_t ds_capacity, int64_t ds_offset, xa_stream_t stream) {
  const char* fn = "xattn_downsample_keys";
  xa_status_t st;
  if ((st = check_heads(fn, hkv, hkv, d)) != XA_OK) return st;
  if (dtype != XA_F32 && dtype != XA_BF16) return fail(XA_EUNSUPPORTED, "%s: dtype must be XA_F32 or XA_BF16", fn);
  if (stride < 1) return fail(XA_EINVAL, "%s: stride must be positive (got %d)", fn, stride);
  if (n_tokens <= 0 || n_tokens % stride != 0)
    return fail(XA_EINVAL, "%s: n_tokens %lld must be a positive multiple of the stride %d", fn, (long long)n_tokens,
                stride);
  const int64_t n_out = n_tokens / stride;
  if (ds_offset < 0 || ds_capacity <= 0 || ds_offset + n_out > ds_capacity)
    return fail(XA_EINVAL, "%s: rows [%lld, %lld) outside the capacity %lld", fn, (long long)ds_offset,
                (long long)(ds_offset + n_out), (long long)ds_capacity);
  if ((st = check_tensor(fn, "k", k, k_tok, k_head, n_tokens, hkv, d, dtype)) != XA_OK) return st;
  if (!k_ds || (uintptr_t)k_ds % 16 != 0) return fail(XA_EINVAL, "%s: k_ds must be 16-byte aligned", fn);
  const hipError_t e = launch_downsample_keys(k, dtype, k_tok, k_head, n_out, hkv, d, stride, k_ds, ds_offset,
                                              reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(XA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return XA_OK;
}

extern "C" size_t xattn_estimate_history_ds_workspace_size(int64_t q_len, int64_t n_ds, int32_t num_q_heads,
                                                           int32_t num_kv_heads, int32_t head_dim, int32_t stride,
                                                           int32_t block, xa_dtype_t dtype) {
  if (q_len <= 0 || n_ds <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || stride <= 0 ||
      block <= 0 || block % stride != 0)
    return 0;
  return est_layout(q_len, n_ds, num_q_heads, num_kv_heads, head_dim, 1, block / stride, dtype).total;
}

extern "C" xa_status_t xattn_estimate_history_ds(const void* q, int64_t q_tok, int64_t q_head, const void* k_ds,
                                                 int64_t kds_tok, int64_t kds_head, xa_dtype_t dtype, int64_t q_len,
                                                 int64_t n_ds, int32_t hq, int32_t hkv, int32_t d, int32_t stride,
                                                 int32_t block, float threshold, float* block_scores,
                                                 uint8_t* block_mask, void* workspace, size_t ws_bytes,
                                                 xa_stream_t stream) {
  const char* fn = "xattn_estimate_history_ds";
  xa_status_t st;
  if ((st = check_heads(fn, hq, hkv, d)) != XA_OK) return st;
  if (dtype != XA_F32 && dtype != XA_BF16) return fail(XA_EUNSUPPORTED, "%s: dtype must be XA_F32 or XA_BF16", fn);
  if (block != 128) return fail(XA_EUNSUPPORTED, "%s: block must be 128 (got %d)", fn, block);
  if (stride != 2 && stride != 4 && stride != 8 && stride != 16)
    return fail(XA_EUNSUPPORTED, "%s: stride %d not in {2, 4, 8, 16}", fn, stride);
  const int b = block / stride;
  if (q_len <= 0 || q_len % b != 0)
    return fail(XA_EINVAL, "%s: q_len %lld must be a positive multiple of block / stride = %d", fn, (long long)q_len, b);
  if (n_ds <= 0 || n_ds % b != 0)
    return fail(XA_EINVAL, "%s: n_ds %lld must be a positive multiple of block / stride = %d", fn, (long long)n_ds, b);
  if (n_ds / b > 8192) return fail(XA_EUNSUPPORTED, "%s: n_ds / (block / stride) exceeds 8192 key blocks", fn);
  if (!(threshold >= 0.f) || isnan(threshold)) return fail(XA_EINVAL, "%s: threshold must be >= 0", fn);
  if ((st = check_tensor(fn, "q", q, q_tok, q_head, q_len, hq, d, dtype)) != XA_OK) return st;
  if ((st = check_tensor(fn, "k_ds", k_ds, kds_tok, kds_head, n_ds, hkv, d, dtype)) != XA_OK) return st;
  if (!block_scores || !block_mask) return fail(XA_EINVAL, "%s: block_scores and block_mask are required", fn);
  const EstLayout L = est_layout(q_len, n_ds, hq, hkv, d, 1, b, dtype);
  if (!workspace || ws_bytes < L.total || (uintptr_t)workspace % 256 != 0)
    return fail(XA_EWORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, L.total,
                ws_bytes);
  if ((int64_t)hq * (n_ds / b) * q_len > ((int64_t)1 << 40)) return fail(XA_EUNSUPPORTED, "%s: problem too large", fn);
  // stride 1 over the downsampled keys; the causal limit c <= n_ds + r never binds (history only)
  return estimate_core(fn, q, q_tok, q_head, k_ds, kds_tok, kds_head, dtype, q_len, n_ds, hq, hkv, d, 1, b, n_ds,
                       q_len / b, 0, true, threshold, block_scores, block_mask, static_cast<char*>(workspace), L,
                       reinterpret_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// packed V and bsa_prefill / bsa_prefill_packed
// ---------------------------------------------------------------------------
namespace {
int64_t packed_pitch(int64_t capacity) { return (capacity + 127) / 128 * 128; }

size_t packed_bytes(int64_t capacity, int32_t hkv, int32_t d, xa_dtype_t dt) {
  const size_t planes = dt == XA_F32 ? 2 : 1;
  return align256(planes * (size_t)hkv * d * packed_pitch(capacity) * 2);
}

// fp32 query/key planes (bf16 hi + lo) needed by the split path.
size_t split_qk_bytes(int64_t q_len, int64_t kv_len, int32_t hq, int32_t hkv, int32_t d, xa_dtype_t dt) {
  if (dt != XA_F32) return 0;
  return 2 * align256((size_t)q_len * hq * d * 2) + 2 * align256((size_t)kv_len * hkv * d * 2);
}

xa_status_t validate_bsa_common(const char* fn, const void* q, int64_t q_tok, int64_t q_head, const void* k,
                                int64_t k_tok, int64_t k_head, xa_dtype_t dtype, int64_t q_len, int64_t kv_len,
                                int32_t hq, int32_t hkv, int32_t d, int64_t q_start, int64_t kv_start,
                                const uint8_t* block_mask, int64_t mask_hs, int64_t mask_rs, int64_t mask_off,
                                int32_t block, float softmax_scale, void* out, xa_dtype_t out_dtype, float* lse) {
  xa_status_t st;
  if ((st = check_heads(fn, hq, hkv, d)) != XA_OK) return st;
  if (dtype != XA_F32 && dtype != XA_BF16) return fail(XA_EUNSUPPORTED, "%s: dtype must be XA_F32 or XA_BF16", fn);
  if (out_dtype != XA_F32 && out_dtype != XA_BF16)
    return fail(XA_EUNSUPPORTED, "%s: out_dtype must be XA_F32 or XA_BF16", fn);
  if (block != 128) return fail(XA_EUNSUPPORTED, "%s: block must be 128 (got %d)", fn, block);
  if (q_len <= 0 || q_len % block != 0)
    return fail(XA_EINVAL, "%s: q_len %lld must be a positive multiple of %d", fn, (long long)q_len, block);
  if (kv_len <= 0) return fail(XA_EINVAL, "%s: kv_len must be positive", fn);
  if (q_start < 0 || q_start % block != 0 || kv_start < 0 || kv_start % block != 0)
    return fail(XA_EINVAL, "%s: q_start_pos and kv_start must be non-negative multiples of %d", fn, block);
  if ((st = check_tensor(fn, "q", q, q_tok, q_head, q_len, hq, d, dtype)) != XA_OK) return st;
  if ((st = check_tensor(fn, "k", k, k_tok, k_head, kv_len, hkv, d, dtype)) != XA_OK) return st;
  if (block_mask && (mask_hs < 0 || mask_rs < 0)) return fail(XA_EINVAL, "%s: negative mask stride", fn);
  if (block_mask && kv_start / block - mask_off < 0)
    return fail(XA_EINVAL, "%s: mask_kb_offset %lld is past the first key block %lld", fn, (long long)mask_off,
                (long long)(kv_start / block));
  if (!out || !lse) return fail(XA_EINVAL, "%s: out and lse are required", fn);
  if ((uintptr_t)out % 16 != 0) return fail(XA_EINVAL, "%s: out must be 16-byte aligned", fn);
  if (!(softmax_scale >= 0.f)) return fail(XA_EINVAL, "%s: softmax_scale must be >= 0 (0 = 1/sqrt(d))", fn);
  if ((int64_t)hq * (q_len / block) > 0x7fffffff) return fail(XA_EUNSUPPORTED, "%s: grid too large", fn);
  return XA_OK;
}

// Fill the kernel parameters of one attention problem (V already packed).
BsaParams bsa_params(const bf16* q, int64_t q_tok, int64_t q_head, const bf16* q_lo, const bf16* k, int64_t k_tok,
                     int64_t k_head, const bf16* k_lo, const bf16* vt_hi, const bf16* vt_lo, int64_t pitch,
                     int64_t q_len, int64_t kv_len, int32_t hq, int32_t hkv, int32_t d, int64_t q_start,
                     int64_t kv_start, const uint8_t* block_mask, int64_t mask_hs, int64_t mask_rs, int64_t mask_off,
                     int32_t block, int32_t causal, float softmax_scale, void* out, float* lse) {
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d);
  BsaParams p{};
  p.q_hi = q;
  p.q_lo = q_lo;
  p.q_tok = q_tok;
  p.q_head = q_head;
  p.k_hi = k;
  p.k_lo = k_lo;
  p.k_tok = k_tok;
  p.k_head = k_head;
  p.vt_hi = vt_hi;
  p.vt_lo = vt_lo;
  p.vt_pitch = pitch;
  p.vt_head = (int64_t)d * pitch;
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.n_qb = (int)(q_len / block);
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
  return p;
}

// Split fp32 Q and K into bf16 hi/lo planes in split_ws (fp32 inputs only).
xa_status_t split_qk(const char* fn, const void* q, int64_t& q_tok, int64_t& q_head, const void* k, int64_t& k_tok,
                     int64_t& k_head, int64_t q_len, int64_t kv_len, int32_t hq, int32_t hkv, int32_t d,
                     char* split_ws, const bf16** qh, const bf16** ql, const bf16** kh, const bf16** kl,
                     hipStream_t s) {
  const size_t pq = align256((size_t)q_len * hq * d * 2);
  const size_t pk = align256((size_t)kv_len * hkv * d * 2);
  bf16* qh_ = reinterpret_cast<bf16*>(split_ws);
  bf16* ql_ = reinterpret_cast<bf16*>(split_ws + pq);
  bf16* kh_ = reinterpret_cast<bf16*>(split_ws + 2 * pq);
  bf16* kl_ = reinterpret_cast<bf16*>(split_ws + 2 * pq + pk);
  hipError_t e;
  if ((e = launch_split((const float*)q, q_tok, q_head, q_len, hq, d, qh_, ql_, s)) != hipSuccess ||
      (e = launch_split((const float*)k, k_tok, k_head, kv_len, hkv, d, kh_, kl_, s)) != hipSuccess)
    return fail(XA_EHIP, "%s: split launch failed: %s", fn, hipGetErrorString(e));
  *qh = qh_;
  *ql = ql_;
  *kh = kh_;
  *kl = kl_;
  q_tok = (int64_t)hq * d;
  q_head = d;
  k_tok = (int64_t)hkv * d;
  k_head = d;
  return XA_OK;
}

}  // namespace

namespace xa {
int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}
}  // namespace xa

namespace {
// Attention workgroups resident at once on the current device.
int resident_workgroups() { return bsa_workgroups_per_cu() * device_cus(); }

xa_status_t run_bsa(const char* fn, const BsaParams* segs, int n, int32_t d, xa_dtype_t dtype, xa_dtype_t out_dtype,
                    hipStream_t s, const BsaPlan* plan = nullptr) {
  const bool split = dtype == XA_F32;
  const bool obf = out_dtype == XA_BF16;
  hipError_t e;
  if (d == 128) {
    if (split) e = obf ? launch_bsa<128, true, bf16>(segs, n, plan, s) : launch_bsa<128, true, float>(segs, n, plan, s);
    else e = obf ? launch_bsa<128, false, bf16>(segs, n, plan, s) : launch_bsa<128, false, float>(segs, n, plan, s);
  } else {
    if (split) e = obf ? launch_bsa<64, true, bf16>(segs, n, plan, s) : launch_bsa<64, true, float>(segs, n, plan, s);
    else e = obf ? launch_bsa<64, false, bf16>(segs, n, plan, s) : launch_bsa<64, false, float>(segs, n, plan, s);
  }
  if (e != hipSuccess) return fail(XA_EHIP, "%s: attention launch failed: %s", fn, hipGetErrorString(e));
  return XA_OK;
}

// Launch the attention kernel once the packed V (hi/lo planes) is in place.
xa_status_t bsa_launch(const char* fn, const void* q, int64_t q_tok, int64_t q_head, const void* k, int64_t k_tok,
                       int64_t k_head, const bf16* vt_hi, const bf16* vt_lo, int64_t pitch, xa_dtype_t dtype,
                       int64_t q_len, int64_t kv_len, int32_t hq, int32_t hkv, int32_t d, int64_t q_start,
                       int64_t kv_start, const uint8_t* block_mask, int64_t mask_hs, int64_t mask_rs,
                       int64_t mask_off, int32_t block, int32_t causal, float softmax_scale, void* out,
                       xa_dtype_t out_dtype, float* lse, char* split_ws, hipStream_t s) {
  const bf16 *qh = static_cast<const bf16*>(q), *ql = nullptr, *kh = static_cast<const bf16*>(k), *kl = nullptr;
  if (dtype == XA_F32) {
    const xa_status_t st = split_qk(fn, q, q_tok, q_head, k, k_tok, k_head, q_len, kv_len, hq, hkv, d, split_ws, &qh,
                                    &ql, &kh, &kl, s);
    if (st != XA_OK) return st;
  }
  const BsaParams p = bsa_params(qh, q_tok, q_head, ql, kh, k_tok, k_head, kl, vt_hi, vt_lo, pitch, q_len, kv_len,
                                 hq, hkv, d, q_start, kv_start, block_mask, mask_hs, mask_rs, mask_off, block, causal,
                                 softmax_scale, out, lse);
  return run_bsa(fn, &p, 1, d, dtype, out_dtype, s);
}
}  // namespace

extern "C" size_t bsa_packed_v_bytes(int64_t capacity, int32_t num_kv_heads, int32_t head_dim, xa_dtype_t dtype) {
  if (capacity <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  return packed_bytes(capacity, num_kv_heads, head_dim, dtype);
}

extern "C" xa_status_t bsa_pack_v(const void* v, int64_t v_tok, int64_t v_head, xa_dtype_t dtype, int64_t n_tokens,
                                  int32_t hkv, int32_t d, void* packed_v, int64_t capacity, int64_t token_offset,
                                  xa_stream_t stream) {
  const char* fn = "bsa_pack_v";
  xa_status_t st;
  if ((st = check_heads(fn, hkv, hkv, d)) != XA_OK) return st;
  if (dtype != XA_F32 && dtype != XA_BF16) return fail(XA_EUNSUPPORTED, "%s: dtype must be XA_F32 or XA_BF16", fn);
  if (n_tokens <= 0 || capacity <= 0) return fail(XA_EINVAL, "%s: n_tokens and capacity must be positive", fn);
  if (token_offset < 0 || token_offset % 128 != 0)
    return fail(XA_EINVAL, "%s: token_offset must be a non-negative multiple of 128", fn);
  const int64_t pitch = packed_pitch(capacity);
  if (token_offset + (n_tokens + 127) / 128 * 128 > pitch)
    return fail(XA_EINVAL, "%s: tokens [%lld, %lld) exceed the packed capacity %lld", fn, (long long)token_offset,
                (long long)(token_offset + n_tokens), (long long)pitch);
  if ((st = check_tensor(fn, "v", v, v_tok, v_head, n_tokens, hkv, d, dtype)) != XA_OK) return st;
  if (!packed_v || (uintptr_t)packed_v % 256 != 0) return fail(XA_EINVAL, "%s: packed_v must be 256-byte aligned", fn);
  bf16* vh = static_cast<bf16*>(packed_v);
  bf16* vl = dtype == XA_F32 ? vh + (size_t)hkv * d * pitch : nullptr;
  const hipError_t e = launch_vt(v, dtype, v_tok, v_head, n_tokens, hkv, d, vh, vl, pitch, token_offset,
                                 reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(XA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return XA_OK;
}

extern "C" size_t bsa_prefill_workspace_size(int64_t q_len, int64_t kv_len, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, xa_dtype_t dtype) {
  if (q_len <= 0 || kv_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  return packed_bytes(kv_len, num_kv_heads, head_dim, dtype) +
         split_qk_bytes(q_len, kv_len, num_q_heads, num_kv_heads, head_dim, dtype);
}

extern "C" size_t bsa_prefill_packed_workspace_size(int64_t q_len, int64_t kv_len, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim, xa_dtype_t dtype) {
  if (q_len <= 0 || kv_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  return split_qk_bytes(q_len, kv_len, num_q_heads, num_kv_heads, head_dim, dtype);
}

extern "C" xa_status_t bsa_prefill(const void* q, int64_t q_tok, int64_t q_head, const void* k, int64_t k_tok,
                                   int64_t k_head, const void* v, int64_t v_tok, int64_t v_head, xa_dtype_t dtype,
                                   int64_t q_len, int64_t kv_len, int32_t hq, int32_t hkv, int32_t d,
                                   int64_t q_start, int64_t kv_start, const uint8_t* block_mask,
                                   int64_t mask_hs, int64_t mask_rs, int64_t mask_off, int32_t block,
                                   int32_t causal, float softmax_scale, void* out, xa_dtype_t out_dtype,
                                   float* lse, void* workspace, size_t ws_bytes, xa_stream_t stream) {
  const char* fn = "bsa_prefill";
  xa_status_t st = validate_bsa_common(fn, q, q_tok, q_head, k, k_tok, k_head, dtype, q_len, kv_len, hq, hkv, d,
                                       q_start, kv_start, block_mask, mask_hs, mask_rs, mask_off, block,
                                       softmax_scale, out, out_dtype, lse);
  if (st != XA_OK) return st;
  if ((st = check_tensor(fn, "v", v, v_tok, v_head, kv_len, hkv, d, dtype)) != XA_OK) return st;
  const size_t need = bsa_prefill_workspace_size(q_len, kv_len, hq, hkv, d, dtype);
  if (!workspace || ws_bytes < need || (uintptr_t)workspace % 256 != 0)
    return fail(XA_EWORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, need,
                ws_bytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int64_t pitch = packed_pitch(kv_len);
  bf16* vh = reinterpret_cast<bf16*>(ws);
  bf16* vl = dtype == XA_F32 ? vh + (size_t)hkv * d * pitch : nullptr;
  const hipError_t e = launch_vt(v, dtype, v_tok, v_head, kv_len, hkv, d, vh, vl, pitch, 0, s);
  if (e != hipSuccess) return fail(XA_EHIP, "%s: V pack launch failed: %s", fn, hipGetErrorString(e));
  return bsa_launch(fn, q, q_tok, q_head, k, k_tok, k_head, vh, vl, pitch, dtype, q_len, kv_len, hq, hkv, d, q_start,
                    kv_start, block_mask, mask_hs, mask_rs, mask_off, block, causal, softmax_scale, out, out_dtype,
                    lse, ws + packed_bytes(kv_len, hkv, d, dtype), s);
}

extern "C" xa_status_t bsa_prefill_packed(const void* q, int64_t q_tok, int64_t q_head, const void* k,
                                          int64_t k_tok, int64_t k_head, const void* packed_v, int64_t capacity,
                                          int64_t v_token_offset, xa_dtype_t dtype, int64_t q_len, int64_t kv_len,
                                          int32_t hq, int32_t hkv, int32_t d, int64_t q_start, int64_t kv_start,
                                          const uint8_t* block_mask, int64_t mask_hs, int64_t mask_rs,
                                          int64_t mask_off, int32_t block, int32_t causal, float softmax_scale,
                                          void* out, xa_dtype_t out_dtype, float* lse, void* workspace,
                                          size_t ws_bytes, xa_stream_t stream) {
  const char* fn = "bsa_prefill_packed";
  xa_status_t st = validate_bsa_common(fn, q, q_tok, q_head, k, k_tok, k_head, dtype, q_len, kv_len, hq, hkv, d,
                                       q_start, kv_start, block_mask, mask_hs, mask_rs, mask_off, block,
                                       softmax_scale, out, out_dtype, lse);
  if (st != XA_OK) return st;
  if (!packed_v || (uintptr_t)packed_v % 256 != 0) return fail(XA_EINVAL, "%s: packed_v must be 256-byte aligned", fn);
  if (capacity <= 0 || v_token_offset < 0 || v_token_offset % 128 != 0)
    return fail(XA_EINVAL, "%s: need capacity > 0 and v_token_offset a non-negative multiple of 128", fn);
  const int64_t pitch = packed_pitch(capacity);
  if (v_token_offset + (kv_len + 127) / 128 * 128 > pitch)
    return fail(XA_EINVAL, "%s: packed tokens [%lld, %lld) exceed the capacity %lld", fn,
                (long long)v_token_offset, (long long)(v_token_offset + kv_len), (long long)pitch);
  const size_t need = bsa_prefill_packed_workspace_size(q_len, kv_len, hq, hkv, d, dtype);
  if (need > 0 && (!workspace || ws_bytes < need || (uintptr_t)workspace % 256 != 0))
    return fail(XA_EWORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, need,
                ws_bytes);
  const bf16* vh = static_cast<const bf16*>(packed_v);
  const bf16* vl = dtype == XA_F32 ? vh + (size_t)hkv * d * pitch : nullptr;
  return bsa_launch(fn, q, q_tok, q_head, k, k_tok, k_head, vh + v_token_offset, vl ? vl + v_token_offset : nullptr,
                    pitch, dtype, q_len, kv_len, hq, hkv, d, q_start, kv_start, block_mask, mask_hs, mask_rs,
                    mask_off, block, causal, softmax_scale, out, out_dtype, lse, static_cast<char*>(workspace),
                    reinterpret_cast<hipStream_t>(stream));
}

extern "C" size_t bsa_prefill_segments_workspace_size(int64_t q_len, int32_t num_q_heads, int32_t head_dim,
                                                      int32_t n_segments) {
  if (q_len <= 0 || num_q_heads <= 0 || head_dim <= 0 || n_segments < 1 || n_segments > kMaxSegments) return 0;
  const int64_t n_items = (int64_t)n_segments * num_q_heads * ((q_len + 127) / 128);
  if (n_items > (int64_t)1 << 28) return 0;
  return bsa_plan_layout(n_items, head_dim).total;
}

extern "C" xa_status_t bsa_prefill_segments(const void* q, int64_t q_tok, int64_t q_head, const void* packed_v,
                                            int64_t capacity, xa_dtype_t dtype, int64_t q_len, int32_t hq,
                                            int32_t hkv, int32_t d, int64_t q_start, const xa_segment_t* segments,
                                            int32_t n_segments, int32_t block, float softmax_scale,
                                            xa_dtype_t out_dtype, void* workspace, size_t ws_bytes,
                                            xa_stream_t stream) {
  const char* fn = "bsa_prefill_segments";
  if (!segments || n_segments < 1 || n_segments > kMaxSegments)
    return fail(XA_EINVAL, "%s: need 1..%d segments (got %d)", fn, kMaxSegments, n_segments);
  if (dtype == XA_F32) return fail(XA_EUNSUPPORTED, "%s: segmented calls take XA_BF16 inputs", fn);
  if (!packed_v || (uintptr_t)packed_v % 256 != 0) return fail(XA_EINVAL, "%s: packed_v must be 256-byte aligned", fn);
  const int64_t pitch = packed_pitch(capacity);
  for (int i = 0; i < n_segments; ++i) {
    const xa_segment_t& g = segments[i];
    xa_status_t st = validate_bsa_common(fn, q, q_tok, q_head, g.k, g.k_tok_stride, g.k_head_stride, dtype, q_len,
                                         g.kv_len, hq, hkv, d, q_start, g.kv_start, g.block_mask, g.mask_head_stride,
                                         g.mask_row_stride, g.mask_kb_offset, block, softmax_scale, g.out, out_dtype,
                                         g.lse);
    if (st != XA_OK) return st;
    if (capacity <= 0 || g.v_token_offset < 0 || g.v_token_offset % 128 != 0 ||
        g.v_token_offset + (g.kv_len + 127) / 128 * 128 > pitch)
      return fail(XA_EINVAL, "%s: segment %d: packed tokens [%lld, %lld) outside the capacity %lld", fn, i,
                  (long long)g.v_token_offset, (long long)(g.v_token_offset + g.kv_len), (long long)pitch);
  }
  const size_t need = bsa_prefill_segments_workspace_size(q_len, hq, d, n_segments);
  if (need == 0) return fail(XA_EINVAL, "%s: too many work items (q_len %lld, %d heads)", fn, (long long)q_len, hq);
  if (!workspace || (uintptr_t)workspace % 256 != 0 || ws_bytes < need)
    return fail(XA_EWORKSPACE, "%s: needs a 256-byte aligned workspace of %zu bytes (got %zu at %p)", fn, need,
                ws_bytes, workspace);
  char* w = static_cast<char*>(workspace);
  const int64_t n_items = (int64_t)n_segments * hq * ((q_len + 127) / 128);
  const BsaPlanLayout L = bsa_plan_layout(n_items, d);
  BsaPlan plan{};
  plan.ctl = reinterpret_cast<int*>(w + L.ctl);
  plan.weights = reinterpret_cast<int*>(w + L.weights);
  plan.mid = reinterpret_cast<int*>(w + L.mid);
  plan.slot = reinterpret_cast<int*>(w + L.slot);
  plan.split_items = reinterpret_cast<int*>(w + L.split_items);
  plan.order = reinterpret_cast<int*>(w + L.order);
  plan.part_o = reinterpret_cast<float*>(w + L.part_o);
  plan.part_lse = reinterpret_cast<float*>(w + L.part_lse);
  plan.max_split = L.max_split;
  plan.slots = resident_workgroups();
  BsaParams segs[kMaxSegments];
  const bf16* vh = static_cast<const bf16*>(packed_v);
  for (int i = 0; i < n_segments; ++i) {
    const xa_segment_t& g = segments[i];
    segs[i] = bsa_params(static_cast<const bf16*>(q), q_tok, q_head, nullptr, static_cast<const bf16*>(g.k),
                         g.k_tok_stride, g.k_head_stride, nullptr, vh + g.v_token_offset, nullptr, pitch, q_len,
                         g.kv_len, hq, hkv, d, q_start, g.kv_start, g.block_mask, g.mask_head_stride,
                         g.mask_row_stride, g.mask_kb_offset, block, g.causal, softmax_scale, g.out, g.lse);
  }
  return run_bsa(fn, segs, n_segments, d, dtype, out_dtype, reinterpret_cast<hipStream_t>(stream), &plan);
}

// ---------------------------------------------------------------------------
// Packed batch of sequences (varlen)
// ---------------------------------------------------------------------------
namespace {
constexpr int32_t kMaxBatch = 1 << 16;

struct VarlenShape {
  std::vector<VarlenSeq> seqs;
  int64_t n_items = 0;    // attention items = selection workgroups
  int64_t est_wg = 0;     // estimate-GEMM workgroups
  int64_t lse_elems = 0;  // estimate partials (floats)
  int64_t out_elems = 0;  // scores / mask elements
  int max_nkb = 0;
  int64_t total_q = 0, total_k = 0;
};

// Lengths from the host prefix arrays; every length a multiple of 128, each sequence's queries at most
// its keys.  stride 0: no estimate sizes.
xa_status_t varlen_shape(const char* fn, const int64_t* cu_q, const int64_t* cu_k, int32_t batch, int32_t hq,
                         int32_t hkv, int32_t stride, VarlenShape& V) {
  if (!cu_q || !cu_k) return fail(XA_EINVAL, "%s: cu_seqlens_q and cu_seqlens_k are required", fn);
  if (batch < 1 || batch > kMaxBatch) return fail(XA_EINVAL, "%s: batch %d outside 1..%d", fn, batch, kMaxBatch);
  if (cu_q[0] != 0 || cu_k[0] != 0) return fail(XA_EINVAL, "%s: cu_seqlens must start at 0", fn);
  V.seqs.resize((size_t)batch);
  const int group = hq / hkv;
  for (int b = 0; b < batch; ++b) {
    const int64_t ql = cu_q[b + 1] - cu_q[b], kl = cu_k[b + 1] - cu_k[b];
    if (ql < 0 || kl < 0 || ql % 128 || kl % 128 || ql > kl)
      return fail(XA_EINVAL, "%s: sequence %d: q_len %lld and k_len %lld must be multiples of 128 with q_len <= k_len",
                  fn, b, (long long)ql, (long long)kl);
    if (kl / 128 > 8192) return fail(XA_EUNSUPPORTED, "%s: sequence %d: more than 8192 key blocks", fn, b);
    if (cu_q[b + 1] > 0x7fffffff || cu_k[b + 1] > 0x7fffffff)
      return fail(XA_EUNSUPPORTED, "%s: more than 2^31 - 1 packed tokens", fn);
    VarlenSeq& s = V.seqs[(size_t)b];
    s.q0 = (int)cu_q[b];
    s.q_len = (int)ql;
    s.k0 = (int)cu_k[b];
    s.k_len = (int)kl;
    s.lse_off = V.lse_elems;
    s.out_off = V.out_elems;
    if (stride > 0 && ql > 0) {
      const int64_t R = ql / stride, N = kl / stride;
      V.est_wg += (int64_t)hkv * ((N + 255) / 256) * ((R + 255) / 256) * group;
      V.lse_elems += (int64_t)hq * (kl / 128) * R;
    }
    V.n_items += (int64_t)hq * (ql / 128);
    V.out_elems += (int64_t)hq * (ql / 128) * (kl / 128);
    if (V.est_wg > 0x7fffffff || V.n_items > ((int64_t)1 << 28))
      return fail(XA_EUNSUPPORTED, "%s: batch too large for one grid", fn);
    s.est_end = (int)V.est_wg;
    s.sel_end = (int)V.n_items;
    if (ql > 0 && kl / 128 > V.max_nkb) V.max_nkb = (int)(kl / 128);
  }
  V.total_q = cu_q[batch];
  V.total_k = cu_k[batch];
  return XA_OK;
}

size_t seqs_bytes(int32_t batch) { return align256((size_t)batch * sizeof(VarlenSeq)); }
}  // namespace

extern "C" int64_t xattn_varlen_mask_elems(const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k, int32_t batch,
                                           int32_t num_q_heads) {
  VarlenShape V;
  if (num_q_heads <= 0 ||
      varlen_shape("xattn_varlen_mask_elems", cu_seqlens_q, cu_seqlens_k, batch, num_q_heads, 1, 0, V) != XA_OK)
    return -1;
  return V.out_elems;
}

extern "C" size_t xattn_estimate_varlen_workspace_size(const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k,
                                                       int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                                       int32_t stride) {
  VarlenShape V;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || stride <= 0 || 128 % stride ||
      varlen_shape("xattn_estimate_varlen_workspace_size", cu_seqlens_q, cu_seqlens_k, batch, num_q_heads,
                   num_kv_heads, stride, V) != XA_OK)
    return 0;
  return seqs_bytes(batch) + align256((size_t)V.lse_elems * sizeof(float));
}

extern "C" xa_status_t xattn_estimate_varlen(const void* q, int64_t q_tok, int64_t q_head, const void* k,
                                             int64_t k_tok, int64_t k_head, xa_dtype_t dtype,
                                             const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k, int32_t batch,
                                             int32_t hq, int32_t hkv, int32_t d, int32_t stride, int32_t block,
                                             float threshold, float* block_scores, uint8_t* block_mask,
                                             void* workspace, size_t ws_bytes, xa_stream_t stream) {
  const char* fn = "xattn_estimate_varlen";
  xa_status_t st;
  if ((st = check_heads(fn, hq, hkv, d)) != XA_OK) return st;
  if (dtype != XA_BF16 || d != 128) return fail(XA_EUNSUPPORTED, "%s: XA_BF16 with head_dim 128 only", fn);
  if (block != 128) return fail(XA_EUNSUPPORTED, "%s: block must be 128 (got %d)", fn, block);
  if (stride != 2 && stride != 4 && stride != 8 && stride != 16)
    return fail(XA_EUNSUPPORTED, "%s: stride %d not in {2, 4, 8, 16}", fn, stride);
  if (!(threshold >= 0.f)) return fail(XA_EINVAL, "%s: threshold must be >= 0", fn);
  VarlenShape V;
  if ((st = varlen_shape(fn, cu_seqlens_q, cu_seqlens_k, batch, hq, hkv, stride, V)) != XA_OK) return st;
  if ((st = check_tensor(fn, "q", q, q_tok, q_head, V.total_q, hq, d, dtype)) != XA_OK) return st;
  if ((st = check_tensor(fn, "k", k, k_tok, k_head, V.total_k, hkv, d, dtype)) != XA_OK) return st;
  if (V.out_elems > 0 && (!block_scores || !block_mask))
    return fail(XA_EINVAL, "%s: block_scores and block_mask are required", fn);
  const size_t need = seqs_bytes(batch) + align256((size_t)V.lse_elems * sizeof(float));
  if (!workspace || ws_bytes < need || (uintptr_t)workspace % 256 != 0)
    return fail(XA_EWORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, need, ws_bytes);
  if (V.n_items == 0) return XA_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  VarlenSeq* seqs = reinterpret_cast<VarlenSeq*>(w);
  hipError_t e = upload_words(V.seqs.data(), sizeof(VarlenSeq) * V.seqs.size(), seqs, s);
  if (e != hipSuccess) return fail(XA_EHIP, "%s: record upload failed: %s", fn, hipGetErrorString(e));
  EstParams p{};
  p.q_hi = static_cast<const bf16*>(q);
  p.q_tok = q_tok;
  p.q_head = q_head;
  p.k_hi = static_cast<const bf16*>(k);
  p.k_tok = k_tok;
  p.k_head = k_head;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.S = stride;
  p.b = block / stride;
  p.scale_log2 = kLog2e / ((float)stride * sqrtf((float)d));
  p.lse_part = reinterpret_cast<float*>(w + seqs_bytes(batch));
  p.seqs = seqs;
  p.n_seqs = batch;
  p.grid_total = (int)V.est_wg;
  if ((e = launch_est_gemm_varlen(p, s)) != hipSuccess)
    return fail(XA_EHIP, "%s: estimate GEMM launch failed: %s", fn, hipGetErrorString(e));
  SelParams sp{};
  sp.lse_part = p.lse_part;
  sp.b = p.b;
  sp.hq = hq;
  sp.nkb = V.max_nkb;
  sp.npow_cap = 1;
  while (sp.npow_cap < sp.nkb) sp.npow_cap <<= 1;
  sp.threshold = threshold;
  sp.scores = block_scores;
  sp.mask = block_mask;
  sp.seqs = seqs;
  sp.n_seqs = batch;
  if ((e = launch_est_select_varlen(sp, (int)V.n_items, s)) != hipSuccess)
    return fail(XA_EHIP, "%s: selection launch failed: %s", fn, hipGetErrorString(e));
  return XA_OK;
}

extern "C" size_t bsa_prefill_varlen_workspace_size(const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k,
                                                    int32_t batch, int32_t num_q_heads, int32_t head_dim) {
  VarlenShape V;
  if (num_q_heads <= 0 || head_dim <= 0 ||
      varlen_shape("bsa_prefill_varlen_workspace_size", cu_seqlens_q, cu_seqlens_k, batch, num_q_heads, 1, 0, V) !=
          XA_OK)
    return 0;
  return seqs_bytes(batch) + bsa_plan_layout(V.n_items, head_dim).total;
}

extern "C" xa_status_t bsa_prefill_varlen(const void* q, int64_t q_tok, int64_t q_head, const void* k, int64_t k_tok,
                                          int64_t k_head, const void* packed_v, int64_t capacity, xa_dtype_t dtype,
                                          const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k, int32_t batch,
                                          int32_t hq, int32_t hkv, int32_t d, const uint8_t* block_mask,
                                          int32_t block, float softmax_scale, void* out, xa_dtype_t out_dtype,
                                          float* lse, void* workspace, size_t ws_bytes, xa_stream_t stream) {
  const char* fn = "bsa_prefill_varlen";
  xa_status_t st;
  if ((st = check_heads(fn, hq, hkv, d)) != XA_OK) return st;
  if (dtype != XA_BF16 || d != 128) return fail(XA_EUNSUPPORTED, "%s: XA_BF16 with head_dim 128 only", fn);
  if (out_dtype != XA_F32 && out_dtype != XA_BF16)
    return fail(XA_EUNSUPPORTED, "%s: out_dtype must be XA_F32 or XA_BF16", fn);
  if (block != 128) return fail(XA_EUNSUPPORTED, "%s: block must be 128 (got %d)", fn, block);
  if (!(softmax_scale >= 0.f)) return fail(XA_EINVAL, "%s: softmax_scale must be >= 0 (0 = 1/sqrt(d))", fn);
  VarlenShape V;
  if ((st = varlen_shape(fn, cu_seqlens_q, cu_seqlens_k, batch, hq, hkv, 0, V)) != XA_OK) return st;
  if ((st = check_tensor(fn, "q", q, q_tok, q_head, V.total_q, hq, d, dtype)) != XA_OK) return st;
  if ((st = check_tensor(fn, "k", k, k_tok, k_head, V.total_k, hkv, d, dtype)) != XA_OK) return st;
  if (!packed_v || (uintptr_t)packed_v % 256 != 0) return fail(XA_EINVAL, "%s: packed_v must be 256-byte aligned", fn);
  const int64_t pitch = packed_pitch(capacity);
  if (capacity <= 0 || V.total_k > pitch)
    return fail(XA_EINVAL, "%s: the %lld packed keys exceed the capacity %lld", fn, (long long)V.total_k,
                (long long)pitch);
  if (V.n_items > 0 && (!out || !lse)) return fail(XA_EINVAL, "%s: out and lse are required", fn);
  if ((uintptr_t)out % 16 != 0) return fail(XA_EINVAL, "%s: out must be 16-byte aligned", fn);
  if ((127 * k_tok + d) * 2 >= ((int64_t)1 << 32) || ((int64_t)(d - 1) * pitch + 128) * 2 >= ((int64_t)1 << 32))
    return fail(XA_EUNSUPPORTED, "%s: k stride or packed capacity too large for 32-bit tile offsets", fn);
  const BsaPlanLayout L = bsa_plan_layout(V.n_items, d);
  const size_t need = seqs_bytes(batch) + L.total;
  if (!workspace || ws_bytes < need || (uintptr_t)workspace % 256 != 0)
    return fail(XA_EWORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, need, ws_bytes);
  if (V.n_items == 0) return XA_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  VarlenSeq* seqs = reinterpret_cast<VarlenSeq*>(w);
  hipError_t e = upload_words(V.seqs.data(), sizeof(VarlenSeq) * V.seqs.size(), seqs, s);
  if (e != hipSuccess) return fail(XA_EHIP, "%s: record upload failed: %s", fn, hipGetErrorString(e));
  char* pw = w + seqs_bytes(batch);
  BsaPlan plan{};
  plan.ctl = reinterpret_cast<int*>(pw + L.ctl);
  plan.weights = reinterpret_cast<int*>(pw + L.weights);
  plan.mid = reinterpret_cast<int*>(pw + L.mid);
  plan.slot = reinterpret_cast<int*>(pw + L.slot);
  plan.split_items = reinterpret_cast<int*>(pw + L.split_items);
  plan.order = reinterpret_cast<int*>(pw + L.order);
  plan.part_o = reinterpret_cast<float*>(pw + L.part_o);
  plan.part_lse = reinterpret_cast<float*>(pw + L.part_lse);
  plan.max_split = L.max_split;
  plan.slots = resident_workgroups();
  // shared fields; each sequence's rows, lengths, mask block and outputs are taken relative to them
  const BsaParams shared = bsa_params(static_cast<const bf16*>(q), q_tok, q_head, nullptr, static_cast<const bf16*>(k),
                                      k_tok, k_head, nullptr, static_cast<const bf16*>(packed_v), nullptr, pitch, 128,
                                      128, hq, hkv, d, 0, 0, block_mask, 0, 0, 0, block, 1, softmax_scale, out, lse);
  e = out_dtype == XA_BF16 ? launch_bsa_varlen<bf16>(shared, seqs, batch, (int)V.n_items, &plan, s)
                           : launch_bsa_varlen<float>(shared, seqs, batch, (int)V.n_items, &plan, s);
  if (e != hipSuccess) return fail(XA_EHIP, "%s: attention launch failed: %s", fn, hipGetErrorString(e));
  return XA_OK;
}
