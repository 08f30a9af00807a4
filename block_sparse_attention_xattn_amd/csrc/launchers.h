// Kernel parameter blocks and launchers shared by the kernels and the C ABI.
#pragma once

#include "common.h"

namespace xa {

// Block-sparse attention (bsa.hip).
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
  float* lse_part;  // [hq][nkb][R], log2 units
};

// Block sums + threshold selection (estimate.hip).
struct SelParams {
  const float* lse_part;
  int R, nkb, b, hq, n_qb;
  int npow_cap;  // smallest power of two >= nkb (sort buffer length)
  int64_t cur;   // key blocks before the chunk (q_start / 128)
  float threshold;
  float* scores;  // [hq][n_qb][nkb]
  uint8_t* mask;  // [hq][n_qb][nkb]
};

// Up to kMaxSegments attention problems sharing Q, heads and packed V, run as
// one grid.  Work item i (one (head, query block) of one segment) belongs to
// segment s when wg_end[s-1] <= i < wg_end[s].  Without an order, workgroup b
// runs item b; with one, each workgroup takes the next ticket t as it starts
// and runs item order[t].
constexpr int kMaxSegments = 4;
struct BsaMulti {
  BsaParams seg[kMaxSegments];
  int wg_end[kMaxSegments];
  int n_seg;
  const int* order;  // item ids, longest kept-tile list first (or null)
  int* ticket;       // start counter, zeroed by the ordering kernel
};

// Device buffers for the longest-first ordering of a segmented launch.
struct BsaPlan {
  int* weights;  // [n_items] kept tiles per item
  int* order;    // [n_items]
  int* ticket;
};
// Bytes of the ordering buffers for n_items work items (ticket, weights, order).
inline size_t bsa_plan_bytes(int64_t n_items) {
  const size_t a = ((size_t)n_items * 4 + 255) / 256 * 256;
  return 256 + 2 * a;
}

template <int D, bool SPLIT, typename OutT>
hipError_t launch_bsa(const BsaParams* segs, int n_seg, const BsaPlan* plan, hipStream_t s);
hipError_t launch_vt(const void* v, xa_dtype_t dt, int64_t v_tok, int64_t v_head, int64_t n_tok, int hkv, int D,
                     bf16* vt_hi, bf16* vt_lo, int64_t pitch, int64_t token_offset, hipStream_t s);
hipError_t launch_split(const float* x, int64_t tok, int64_t head, int64_t L, int H, int D, bf16* hi, bf16* lo,
                        hipStream_t s);
template <int D, bool SPLIT>
hipError_t launch_est_gemm(const EstParams& p, hipStream_t s);
hipError_t launch_est_select(const SelParams& p, hipStream_t s);

}  // namespace xa
