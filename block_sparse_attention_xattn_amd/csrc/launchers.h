// Kernel parameter blocks and launchers shared by the kernels and the C ABI.
#pragma once

#include "common.h"

namespace xa {

// Block-sparse attention (bsa.hip).
// One sequence of a packed batch: rows [q0, q0 + q_len) of q and [k0, k0 + k_len) of k, the query rows
// at the end of their keys (global positions k_len - q_len ..); est_end / sel_end: prefix ends of the
// estimate-GEMM and selection workgroups of this and the earlier sequences; lse_off: float offset of its
// estimate partials [hq][k_len/128][q_len/S]; out_off: element offset of its scores / mask
// [hq][q_len/128][k_len/128].
struct VarlenSeq {
  int q0, q_len, k0, k_len;
  int est_end, sel_end;
  int64_t lse_off, out_off;
};

struct BsaParams {
  const bf16* q_hi;
  const bf16* q_lo;
  int64_t q_tok, q_head;
  const bf16* k_hi;
  const bf16* k_lo;
  int64_t k_tok, k_head;
  const bf16* vt_hi;
  const bf16* vt_lo;
  int64_t vt_head, vt_pitch;  // Vt[hkv][d][vt_pitch], key order permuted per 16-group
  int64_t q_len, kv_len;
  int hq, hkv, group, n_qb;
  int64_t q_start, kv_start;
  const uint8_t* mask;
  int64_t mask_hs, mask_rs, mask_off;
  int causal;
  float scale_log2;
  void* out;
  float* lse;
};

// Reshaped GEMM + per-(row, key block) log-sum-exp (estimate.hip).
struct EstParams {
  const bf16* q_hi;
  const bf16* q_lo;
  int64_t q_tok, q_head;
  const bf16* k_hi;
  const bf16* k_lo;
  int64_t k_tok, k_head;
  int64_t q_len, k_len, q_start;
  int hq, hkv, group, S, b, R, N, nkb, n_rt, n_ct;
  float scale_log2;
  // K row 0 is reshaped column c0 (global) = key block kb0; lse_part rows hold nkb_ld key blocks
  int64_t c0;
  int kb0, nkb_ld;
  float* lse_part;  // [hq][nkb_ld][R], log2 units; this call writes key blocks kb0 .. kb0 + nkb - 1
  // packed batch: workgroup w runs sequence s with seqs[s-1].est_end <= w < seqs[s].est_end, the
  // pointers, lengths and offsets above taken relative to that sequence
  const VarlenSeq* seqs;
  int n_seqs, grid_total;
};

// Block sums + threshold selection (estimate.hip).
struct SelParams {
  const float* lse_part;
  int R, nkb, b, hq, n_qb;
  int npow_cap;   // smallest power of two >= nkb (sort buffer length)
  int hist_only;  // 1: keys are history only (all visible, block 0 the only forced block)
  int64_t cur;    // key blocks before the chunk (q_start / 128)
  float threshold;
  float* scores;  // [hq][n_qb][nkb]
  uint8_t* mask;  // [hq][n_qb][nkb]
  // packed batch, as for EstParams (sel_end: hq * q_len/128 workgroups per sequence)
  const VarlenSeq* seqs;
  int n_seqs;
};

// Up to kMaxSegments attention problems sharing Q, heads and packed V, run as
// one grid.  Work item i (one (head, query block) of one segment) belongs to
// segment s when wg_end[s-1] <= i < wg_end[s].  Without an order, workgroup b
// runs item b whole.  With one, each workgroup takes the next ticket t as it
// starts and runs entry order[t] = item * 4 + part: part 0 is the whole item,
// parts 1 and 2 the key blocks before / from mid[item] of a split item, whose
// normalised partial results go to partial slot slot[item] and are merged
// afterwards.
constexpr int kMaxSegments = 4;
constexpr int kMaxSplit = 512;  // items split in two per call, at most
struct BsaMulti {
  BsaParams seg[kMaxSegments];
  int wg_end[kMaxSegments];
  int n_seg;
  int n_items;             // work items of all segments
  const VarlenSeq* seqs;   // packed batch: n_seg sequences (device memory), seg[0] holds the shared fields
  const int* order;        // entries, longest first (null: no order)
  int* ctl;                // [0] next ticket, [1] entries, [2] split items
  const int* mid;          // [items] first key block (segment-relative) of a split item's second half
  const int* slot;         // [items] partial slot of a split item
  const int* split_items;  // [max_split] item of each partial slot
  float* part_o;           // [max_split][2][heads per item][128][D] normalised partial outputs
  float* part_lse;         // [max_split][2][heads per item][128] their LSE (natural log)
  int pair;                // 1: an item is a pair of query heads (2p, 2p + 1) of one kv head (pair kernel)
  int direct;              // workgroups below this index take order entry blockIdx.x without a ticket
};

// Device buffers of the work order of a segmented launch.
struct BsaPlan {
  int* ctl;
  int* weights;  // [items] kept key blocks
  int* mid;
  int* slot;
  int* split_items;
  int* order;    // [items + max_split]
  float* part_o;
  float* part_lse;
  int max_split;  // min(items, kMaxSplit)
  int slots;      // workgroups resident at once; items above total / slots are split
};

// Byte layout of the work-order workspace for n_items items of head_dim d.
struct BsaPlanLayout {
  size_t ctl, weights, mid, slot, split_items, order, part_o, part_lse, total;
  int max_split;
};
inline BsaPlanLayout bsa_plan_layout(int64_t n_items, int d) {
  auto a = [](size_t bytes) { return (bytes + 255) / 256 * 256; };
  BsaPlanLayout L{};
  L.max_split = (int)(n_items < kMaxSplit ? n_items : kMaxSplit);
  size_t o = 0;
  L.ctl = o;          o += 256;
  L.weights = o;      o += a((size_t)n_items * 4);
  L.mid = o;          o += a((size_t)n_items * 4);
  L.slot = o;         o += a((size_t)n_items * 4);
  L.split_items = o;  o += a((size_t)L.max_split * 4);
  L.order = o;        o += a((size_t)(n_items + L.max_split) * 4);
  L.part_o = o;       o += a((size_t)L.max_split * 2 * 128 * d * 4);
  L.part_lse = o;     o += a((size_t)L.max_split * 2 * 128 * 4);
  L.total = o;
  return L;
}

// Events recorded on the launch stream immediately before / after each launch of the ping-pong attention
// kernel (both null: none); per host thread, the events belong to the caller.
void set_attention_events(hipEvent_t before, hipEvent_t after);

template <int D, bool SPLIT, typename OutT>
hipError_t launch_bsa(const BsaParams* segs, int n_seg, const BsaPlan* plan, hipStream_t s);
// A packed batch of bf16, head_dim 128 sequences (records seqs in device memory, n_items = hq * total
// query blocks) as one grid with a work order; `shared` holds the batch's base pointers, strides, heads,
// scale and the mask base (null: dense causal).  hipErrorInvalidValue when tile offsets do not fit 32 bits.
template <typename OutT>
hipError_t launch_bsa_varlen(const BsaParams& shared, const VarlenSeq* seqs, int n_seqs, int n_items,
                             const BsaPlan* plan, hipStream_t s);
// Attention workgroups resident per compute unit (the work order balances over CUs times this).
int bsa_workgroups_per_cu();
// Compute units of the current device (cached per device).
int device_cus();
// Copy `bytes` (a multiple of 4) of host memory to device memory in stream order through kernel arguments.
hipError_t upload_words(const void* src, size_t bytes, void* dst, hipStream_t s);
hipError_t launch_vt(const void* v, xa_dtype_t dt, int64_t v_tok, int64_t v_head, int64_t n_tok, int hkv, int D,
                     bf16* vt_hi, bf16* vt_lo, int64_t pitch, int64_t token_offset, hipStream_t s);
hipError_t launch_split(const float* x, int64_t tok, int64_t head, int64_t L, int H, int D, bf16* hi, bf16* lo,
                        hipStream_t s);
template <int D, bool SPLIT>
hipError_t launch_est_gemm(const EstParams& p, hipStream_t s);
hipError_t launch_est_select(const SelParams& p, hipStream_t s);
// Packed-batch forms (bf16, head_dim 128): p0 holds the shared fields, seqs / n_seqs (device memory), the
// grid total and, for the selection, the largest npow_cap / nkb over the batch (LDS size).
hipError_t launch_est_gemm_varlen(const EstParams& p0, hipStream_t s);
hipError_t launch_est_select_varlen(const SelParams& p0, int grid, hipStream_t s);
hipError_t launch_downsample_keys(const void* k, xa_dtype_t dt, int64_t k_tok, int64_t k_head, int64_t n_out, int hkv,
                                  int d, int stride, void* out, int64_t out_off, hipStream_t s);

}  // namespace xa
