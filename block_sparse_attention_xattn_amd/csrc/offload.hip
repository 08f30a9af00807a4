// Offloaded history: K and packed V of 1024-token cache blocks kept in pinned
// host memory, brought back into a device ring only for the blocks a chunk
// keeps, while the attention over the blocks already brought back runs.
//
// XAttentionBSAPolicy page, compute_chunked_prefill with the offload engine
// (history blocks come from the CPU cache through a ring of GPU slots) and
// Task plan page, "核心设计理解" (1 CPU block = 8 BSA blocks; selection maps
// BSA blocks to CPU blocks): the attention of a chunk over its kept history
// cache blocks, with the copies of the next group of blocks overlapping the
// attention over the current group; groups are merged by their LSE.
#include <hip/hip_runtime.h>

#include "common.h"
#include "launchers.h"
#include "xattn.h"

namespace {
using xa::bf16;
using xa::launch_vt;
using xa_host::fail;

constexpr int kMaxBlocksPerCall = 1 << 20;

struct Events {
  hipEvent_t e[5] = {};
  int n = 0;
  hipError_t create() {
    for (; n < 5; ++n) {
      const hipError_t r = hipEventCreateWithFlags(&e[n], hipEventDisableTiming);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
  ~Events() {
    for (int i = 0; i < n; ++i) (void)hipEventDestroy(e[i]);  // released once the recorded work completes
  }
};
}  // namespace

extern "C" xa_status_t xattn_offload_blocks(const void* k, int64_t k_tok, int64_t k_head, const void* v,
                                            int64_t v_tok, int64_t v_head, xa_dtype_t dtype, int32_t n_blocks,
                                            int32_t hkv, int32_t d, int32_t cache_block, void* host_k,
                                            void* host_vt, int64_t n_host_blocks, int64_t first_block,
                                            void* staging_vt, xa_stream_t stream) {
  const char* fn = "xattn_offload_blocks";
  if (dtype != XA_BF16) return fail(XA_EUNSUPPORTED, "%s: XA_BF16 only", fn);
  if (hkv <= 0 || (d != 64 && d != 128)) return fail(XA_EUNSUPPORTED, "%s: head_dim must be 64 or 128", fn);
  if (cache_block <= 0 || cache_block % 128 != 0)
    return fail(XA_EINVAL, "%s: cache_block must be a positive multiple of 128 (got %d)", fn, cache_block);
  if (n_blocks < 0 || n_blocks > kMaxBlocksPerCall || first_block < 0 || first_block + n_blocks > n_host_blocks)
    return fail(XA_EINVAL, "%s: blocks [%lld, %lld) outside the %lld host blocks", fn, (long long)first_block,
                (long long)(first_block + n_blocks), (long long)n_host_blocks);
  if (n_blocks == 0) return XA_OK;
  if (!k || !v || !host_k || !host_vt || !staging_vt) return fail(XA_EINVAL, "%s: null pointer", fn);
  if (k_head != d || k_tok < (int64_t)hkv * d || k_tok % 8 != 0 || (uintptr_t)k % 16 != 0)
    return fail(XA_EINVAL, "%s: k must be [tokens][heads][head_dim] with heads contiguous in a token", fn);
  if (v_tok % 8 != 0 || v_head % 8 != 0 || (uintptr_t)v % 16 != 0)
    return fail(XA_EINVAL, "%s: v must be 16-byte aligned with strides that are multiples of 8", fn);
  if ((uintptr_t)staging_vt % 256 != 0) return fail(XA_EINVAL, "%s: staging_vt must be 256-byte aligned", fn);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t cb = cache_block;
  const size_t row_bytes = (size_t)hkv * d * 2;
  const size_t block_bytes = (size_t)cb * row_bytes;
  const int64_t n_tok = (int64_t)n_blocks * cb;
  const int64_t host_cap = n_host_blocks * cb;
  // V of the blocks -> packed [hkv][d][n_tok] in the staging buffer, then into columns
  // first_block * cb .. of the host's packed rows (pitch host_cap)
  hipError_t e = launch_vt(v, XA_BF16, v_tok, v_head, n_tok, hkv, d, static_cast<bf16*>(staging_vt), nullptr, n_tok,
                           0, s);
  if (e != hipSuccess) return fail(XA_EHIP, "%s: V pack launch failed: %s", fn, hipGetErrorString(e));
  char* hk = static_cast<char*>(host_k) + (size_t)first_block * block_bytes;
  char* hv = static_cast<char*>(host_vt) + (size_t)first_block * cb * 2;
  e = hipMemcpy2DAsync(hk, row_bytes, k, (size_t)k_tok * 2, row_bytes, (size_t)n_tok, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpy2DAsync(hv, (size_t)host_cap * 2, staging_vt, (size_t)n_tok * 2, (size_t)n_tok * 2, (size_t)hkv * d,
                         hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return fail(XA_EHIP, "%s: copy to host failed: %s", fn, hipGetErrorString(e));
  return XA_OK;
}

extern "C" xa_status_t bsa_history_offloaded(const void* q, int64_t q_tok, int64_t q_head, xa_dtype_t dtype,
                                             int64_t q_len, int32_t hq, int32_t hkv, int32_t d, int64_t q_start_pos,
                                             const void* host_k, const void* host_vt, int64_t n_host_blocks,
                                             int32_t cache_block, const int32_t* keep, int32_t n_keep,
                                             int32_t group, void* ring_k, void* ring_vt, void* out, float* lse,
                                             void* part_out, float* part_lse, xa_stream_t stream,
                                             xa_stream_t copy_stream) {
  const char* fn = "bsa_history_offloaded";
  if (dtype != XA_BF16) return fail(XA_EUNSUPPORTED, "%s: XA_BF16 only", fn);
  if (cache_block <= 0 || cache_block % 128 != 0)
    return fail(XA_EINVAL, "%s: cache_block must be a positive multiple of 128 (got %d)", fn, cache_block);
  if (group <= 0 || (int64_t)group * cache_block * 2 > ((int64_t)1 << 30))
    return fail(XA_EINVAL, "%s: group must be positive and the ring at most 2^30 tokens", fn);
  if (n_keep < 0 || (n_keep > 0 && !keep)) return fail(XA_EINVAL, "%s: keep list missing", fn);
  for (int i = 0; i < n_keep; ++i)
    if (keep[i] < 0 || keep[i] >= n_host_blocks)
      return fail(XA_EINVAL, "%s: keep[%d] = %d outside the %lld host blocks", fn, i, keep[i],
                  (long long)n_host_blocks);
  if (!q || !out || !lse || !part_out || !part_lse || !ring_k || !ring_vt || (n_keep > 0 && (!host_k || !host_vt)))
    return fail(XA_EINVAL, "%s: null pointer", fn);
  if ((uintptr_t)ring_vt % 256 != 0 || (uintptr_t)ring_k % 16 != 0)
    return fail(XA_EINVAL, "%s: ring_vt must be 256-byte and ring_k 16-byte aligned", fn);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipStream_t cs = reinterpret_cast<hipStream_t>(copy_stream);
  const int64_t cb = cache_block;
  const int64_t ring_cap = 2 * (int64_t)group * cb;
  const int64_t host_cap = n_host_blocks * cb;
  const size_t block_bytes = (size_t)cb * hkv * d * 2;
  hipError_t e;
  if (n_keep == 0) {  // no kept history: out 0, lse -inf
    e = hipMemsetAsync(out, 0, (size_t)q_len * hq * d * 2, s);
    if (e == hipSuccess)
      e = hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(lse), 0xff800000u, (size_t)hq * q_len, s);
    return e == hipSuccess ? XA_OK : fail(XA_EHIP, "%s: fill failed: %s", fn, hipGetErrorString(e));
  }
  Events ev;  // [0] start, [1..2] half copied, [3..4] half consumed
  if ((e = ev.create()) != hipSuccess)
    return fail(XA_EHIP, "%s: event creation failed: %s", fn, hipGetErrorString(e));
  // ring slots may still be read by earlier work on the compute stream
  if ((e = hipEventRecord(ev.e[0], s)) != hipSuccess || (e = hipStreamWaitEvent(cs, ev.e[0], 0)) != hipSuccess)
    return fail(XA_EHIP, "%s: stream ordering failed: %s", fn, hipGetErrorString(e));
  const int n_groups = (n_keep + group - 1) / group;
  for (int g = 0; g < n_groups; ++g) {
    const int half = g & 1;
    const int base = half * group;
    const int n_g = n_keep - g * group < group ? n_keep - g * group : group;
    if (g >= 2 && (e = hipStreamWaitEvent(cs, ev.e[3 + half], 0)) != hipSuccess)
      return fail(XA_EHIP, "%s: stream ordering failed: %s", fn, hipGetErrorString(e));
    // one copy of K rows and one 2-D copy of packed-V columns per run of consecutive block ids
    for (int j = 0; j < n_g;) {
      int r = 1;
      while (j + r < n_g && keep[g * group + j + r] == keep[g * group + j] + r) ++r;
      const int64_t blk = keep[g * group + j];
      const int64_t slot = base + j;
      e = hipMemcpyAsync(static_cast<char*>(ring_k) + (size_t)slot * block_bytes,
                         static_cast<const char*>(host_k) + (size_t)blk * block_bytes, (size_t)r * block_bytes,
                         hipMemcpyHostToDevice, cs);
      if (e == hipSuccess)
        e = hipMemcpy2DAsync(static_cast<char*>(ring_vt) + (size_t)slot * cb * 2, (size_t)ring_cap * 2,
                             static_cast<const char*>(host_vt) + (size_t)blk * cb * 2, (size_t)host_cap * 2,
                             (size_t)r * cb * 2, (size_t)hkv * d, hipMemcpyHostToDevice, cs);
      if (e != hipSuccess) return fail(XA_EHIP, "%s: copy to the ring failed: %s", fn, hipGetErrorString(e));
      j += r;
    }
    if ((e = hipEventRecord(ev.e[1 + half], cs)) != hipSuccess ||
        (e = hipStreamWaitEvent(s, ev.e[1 + half], 0)) != hipSuccess)
      return fail(XA_EHIP, "%s: stream ordering failed: %s", fn, hipGetErrorString(e));
    void* o_g = g == 0 ? out : part_out;
    float* l_g = g == 0 ? lse : part_lse;
    const bf16* kg = static_cast<const bf16*>(ring_k) + (size_t)base * cb * hkv * d;
    xa_status_t st = bsa_prefill_packed(q, q_tok, q_head, kg, (int64_t)hkv * d, d, ring_vt, ring_cap,
                                        (int64_t)base * cb, dtype, q_len, (int64_t)n_g * cb, hq, hkv, d, q_start_pos,
                                        0, nullptr, 0, 0, 0, 128, 0, 0.f, o_g, XA_BF16, l_g, nullptr, 0, stream);
    if (st != XA_OK) return st;
    if ((e = hipEventRecord(ev.e[3 + half], s)) != hipSuccess)
      return fail(XA_EHIP, "%s: event record failed: %s", fn, hipGetErrorString(e));
    if (g > 0 && (st = attn_merge(out, lse, part_out, part_lse, out, lse, XA_BF16, q_len, hq, d, stream)) != XA_OK)
      return st;
  }
  return XA_OK;
}

// ---------------------------------------------------------------------------
// Estimate against host-resident history keys
//
// XAttentionBSAPolicy page, select_blocks (the estimate over K that arrives
// from the CPU cache one chunk of blocks at a time: partial row statistics
// per key chunk, their merge, then block sums).  The estimate GEMM already
// leaves one log-sum-exp per (reshaped row, key block); each group of cache
// blocks copied into the ring fills its key blocks' entries, the chunk's own
// keys fill theirs, and one selection pass merges the row statistics and
// forms the block sums, so every history key crosses PCIe once.
// ---------------------------------------------------------------------------
namespace {
using xa::EstParams;
using xa::SelParams;

EstParams est_params(const bf16* q, int64_t q_tok, int64_t q_head, int64_t q_len, int64_t q_start, int32_t hq,
                     int32_t hkv, int32_t d, int32_t stride, float* lse, int64_t nkb_total) {
  EstParams p{};
  p.q_hi = q;
  p.q_tok = q_tok;
  p.q_head = q_head;
  p.q_len = q_len;
  p.q_start = q_start;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.S = stride;
  p.b = 128 / stride;
  p.R = (int)(q_len / stride);
  p.n_rt = (p.R + 127) / 128;
  p.scale_log2 = xa::kLog2e / ((float)stride * sqrtf((float)d));
  p.nkb_ld = (int)nkb_total;
  p.lse_part = lse;
  return p;
}

// keys [key0, key0 + n_keys) of the layer, rows of k with the given strides
hipError_t est_keys(EstParams p, const bf16* k, int64_t k_tok, int64_t k_head, int64_t key0, int64_t n_keys, int d,
                    hipStream_t s) {
  p.k_hi = k;
  p.k_tok = k_tok;
  p.k_head = k_head;
  p.k_len = n_keys;
  p.N = (int)(n_keys / p.S);
  p.n_ct = (p.N + 127) / 128;
  p.c0 = key0 / p.S;
  p.kb0 = (int)(key0 / 128);
  p.nkb = (int)(n_keys / 128);
  return d == 128 ? xa::launch_est_gemm<128, false>(p, s) : xa::launch_est_gemm<64, false>(p, s);
}
}  // namespace

extern "C" xa_status_t xattn_estimate_offloaded(const void* q, int64_t q_tok, int64_t q_head, const void* k_cur,
                                                int64_t kc_tok, int64_t kc_head, xa_dtype_t dtype, int64_t q_len,
                                                int32_t hq, int32_t hkv, int32_t d, int64_t q_start_pos,
                                                const void* host_k, int64_t n_host_blocks, int32_t cache_block,
                                                int32_t group, void* ring_k, int32_t stride, int32_t block,
                                                float threshold, float* block_scores, uint8_t* block_mask,
                                                void* workspace, size_t ws_bytes, xa_stream_t stream,
                                                xa_stream_t copy_stream) {
  const char* fn = "xattn_estimate_offloaded";
  if (dtype != XA_BF16) return fail(XA_EUNSUPPORTED, "%s: XA_BF16 only", fn);
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
    return fail(XA_EINVAL, "%s: num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", fn, hq, hkv);
  if (d != 64 && d != 128) return fail(XA_EUNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn, d);
  if (block != 128) return fail(XA_EUNSUPPORTED, "%s: block must be 128 (got %d)", fn, block);
  if (stride != 2 && stride != 4 && stride != 8 && stride != 16)
    return fail(XA_EUNSUPPORTED, "%s: stride %d not in {2, 4, 8, 16}", fn, stride);
  if (cache_block <= 0 || cache_block % 128 != 0)
    return fail(XA_EINVAL, "%s: cache_block must be a positive multiple of 128 (got %d)", fn, cache_block);
  if (group <= 0 || (int64_t)group * cache_block * 2 > ((int64_t)1 << 30))
    return fail(XA_EINVAL, "%s: group must be positive and the ring at most 2^30 tokens", fn);
  if (q_len <= 0 || q_len % 128 != 0)
    return fail(XA_EINVAL, "%s: q_len %lld must be a positive multiple of 128", fn, (long long)q_len);
  if (q_start_pos < 0 || q_start_pos % cache_block != 0 || q_start_pos / cache_block > n_host_blocks)
    return fail(XA_EINVAL, "%s: q_start_pos %lld must be whole cache blocks held by the %lld host blocks", fn,
                (long long)q_start_pos, (long long)n_host_blocks);
  const int64_t k_len = q_start_pos + q_len;
  const int64_t nkb = k_len / 128;
  if (nkb > 8192) return fail(XA_EUNSUPPORTED, "%s: k_len / block = %lld exceeds 8192 key blocks", fn, (long long)nkb);
  if (!(threshold >= 0.f)) return fail(XA_EINVAL, "%s: threshold must be >= 0", fn);  // NaN fails too
  if (!q || !k_cur || !ring_k || !block_scores || !block_mask || (q_start_pos > 0 && !host_k))
    return fail(XA_EINVAL, "%s: null pointer", fn);
  if (q_tok % 8 || q_head % 8 || (uintptr_t)q % 16 || kc_tok % 8 || kc_head % 8 || (uintptr_t)k_cur % 16 ||
      (uintptr_t)ring_k % 16)
    return fail(XA_EINVAL, "%s: q, k_cur and ring_k must be 16-byte aligned with strides multiples of 8", fn);
  const size_t need = xattn_estimate_workspace_size(q_len, k_len, hq, hkv, d, stride, block, XA_BF16);
  if (!workspace || ws_bytes < need || (uintptr_t)workspace % 256 != 0)
    return fail(XA_EWORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, need, ws_bytes);
  if ((int64_t)hq * nkb * q_len > ((int64_t)1 << 40)) return fail(XA_EUNSUPPORTED, "%s: problem too large", fn);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipStream_t cs = reinterpret_cast<hipStream_t>(copy_stream);
  float* lse = static_cast<float*>(workspace);
  const EstParams p0 = est_params(static_cast<const bf16*>(q), q_tok, q_head, q_len, q_start_pos, hq, hkv, d, stride,
                                  lse, nkb);
  hipError_t e;
  // the chunk's own keys first: they need no copy
  if ((e = est_keys(p0, static_cast<const bf16*>(k_cur), kc_tok, kc_head, q_start_pos, q_len, d, s)) != hipSuccess)
    return fail(XA_EHIP, "%s: estimate GEMM launch failed: %s", fn, hipGetErrorString(e));
  const int64_t cb = cache_block;
  const int64_t row = (int64_t)hkv * d;
  const size_t block_bytes = (size_t)cb * row * 2;
  const int64_t n_hist = q_start_pos / cb;
  if (n_hist > 0) {
    Events ev;  // [0] start, [1..2] half copied, [3..4] half consumed
    if ((e = ev.create()) != hipSuccess)
      return fail(XA_EHIP, "%s: event creation failed: %s", fn, hipGetErrorString(e));
    if ((e = hipEventRecord(ev.e[0], s)) != hipSuccess || (e = hipStreamWaitEvent(cs, ev.e[0], 0)) != hipSuccess)
      return fail(XA_EHIP, "%s: stream ordering failed: %s", fn, hipGetErrorString(e));
    const int64_t n_groups = (n_hist + group - 1) / group;
    for (int64_t g = 0; g < n_groups; ++g) {
      const int half = (int)(g & 1);
      const int64_t base = (int64_t)half * group;
      const int64_t n_g = n_hist - g * group < group ? n_hist - g * group : group;
      if (g >= 2 && (e = hipStreamWaitEvent(cs, ev.e[3 + half], 0)) != hipSuccess)
        return fail(XA_EHIP, "%s: stream ordering failed: %s", fn, hipGetErrorString(e));
      // blocks g*group .. are consecutive on the host and in the ring half: one copy
      e = hipMemcpyAsync(static_cast<char*>(ring_k) + (size_t)base * block_bytes,
                         static_cast<const char*>(host_k) + (size_t)(g * group) * block_bytes,
                         (size_t)n_g * block_bytes, hipMemcpyHostToDevice, cs);
      if (e != hipSuccess) return fail(XA_EHIP, "%s: copy to the ring failed: %s", fn, hipGetErrorString(e));
      if ((e = hipEventRecord(ev.e[1 + half], cs)) != hipSuccess ||
          (e = hipStreamWaitEvent(s, ev.e[1 + half], 0)) != hipSuccess)
        return fail(XA_EHIP, "%s: stream ordering failed: %s", fn, hipGetErrorString(e));
      if ((e = est_keys(p0, static_cast<const bf16*>(ring_k) + (size_t)base * cb * row, row, d, g * group * cb,
                        n_g * cb, d, s)) != hipSuccess)
        return fail(XA_EHIP, "%s: estimate GEMM launch failed: %s", fn, hipGetErrorString(e));
      if ((e = hipEventRecord(ev.e[3 + half], s)) != hipSuccess)
        return fail(XA_EHIP, "%s: event record failed: %s", fn, hipGetErrorString(e));
    }
  }
  SelParams sp{};
  sp.lse_part = lse;
  sp.R = p0.R;
  sp.nkb = (int)nkb;
  sp.npow_cap = 1;
  while (sp.npow_cap < sp.nkb) sp.npow_cap <<= 1;
  sp.b = p0.b;
  sp.hq = hq;
  sp.n_qb = (int)(q_len / 128);
  sp.hist_only = 0;
  sp.cur = q_start_pos / 128;
  sp.threshold = threshold;
  sp.scores = block_scores;
  sp.mask = block_mask;
  if ((e = xa::launch_est_select(sp, s)) != hipSuccess)
    return fail(XA_EHIP, "%s: selection launch failed: %s", fn, hipGetErrorString(e));
  return XA_OK;
}
