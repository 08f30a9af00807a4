// Block-sparse flash attention with LSE (part 2 of the path).
//
// XAttention algorithm guide, "BSA (Block Sparse Attention)": exact softmax
// attention restricted to the 128x128 (query block, key block) tiles that the
// block mask keeps, with token causality; XAttentionBSAPolicy
// .compute_chunked_prefill: the history segment is attended without the
// causal rule, the chunk's own keys with it, and each part returns (out, lse).
//
// Three kernels (gfx950), each described above its body below.  bf16,
// head_dim 128 (the hot path): bsa_pair_kernel (an even number of query heads
// per kv head) computes two query heads of one kv head per workgroup, its two
// groups of four waves alternating matrix and vector phases on the union of
// the two heads' kept blocks (segments, and the packed batch); bsa3_kernel (odd
// group sizes) has both groups on one (query head, query block), on alternate
// kept blocks.
// The matrix phases run at raised issue priority.
// bsa_kernel (XA_F32 inputs, head_dim 64, and tiles whose offsets exceed 32
// bits):
//   * one workgroup = one (query head, 128-row query block); 8 waves.  Wave w
//     owns query rows 32*(w%4) .. +32 and key half 64*(w/4) .. +64 of every
//     kept key block (split over keys inside the workgroup; the two halves are
//     merged once at the end through LDS);
// All:
//   * scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     a lane then owns one query row and 16 keys, so the row max / row sum are
//     mostly in-lane (one cross-half exchange per block for the max);
//   * the fp32 accumulator of S^T, exponentiated and rounded to bf16, is
//     directly the B operand of the O^T += V^T P^T MFMA; V is stored transposed
//     in the workspace with the matching key order inside each 16-key group,
//     so both operands come from LDS with 16-byte reads;
//   * (bsa_kernel) K and V^T tiles of the next kept block are fetched into
//     registers while the current one is being multiplied (two LDS buffers);
//   * the walk over key blocks touches only kept blocks, in ascending order,
//     from a list built in LDS from the mask row.
// XA_F32 inputs use bf16 hi/lo planes and three MFMAs per product.
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "launchers.h"

namespace xa {


constexpr int kBlk = 128;
constexpr int kThreads = 512;
constexpr int kListMax = 1024;

// Item index -> (query head, query block): clusters of (kv head, query block),
// the last query blocks (the most keys under the causal rule) first, the
// `group` query heads of a cluster at ids b, b+8, b+16, ...  Without a work
// order the ids are dispatch slots (workgroup b runs on XCD b mod 8, so a
// cluster's heads share one L2); with one, the order's tickets decide which
// workgroup runs an item and this map only names the items.
__device__ __forceinline__ void bsa_decode(int bid, int group, int hkv, int n_qb, int& h, int& qb) {
  const int clusters = hkv * n_qb;
  const int full_rounds = clusters / 8;
  const int full_ids = full_rounds * 8 * group;
  int c, j;
  if (bid < full_ids) {
    const int x = bid & 7;
    const int t = bid >> 3;
    j = t % group;
    c = (t / group) * 8 + x;
  } else {
    const int rem = bid - full_ids;
    c = full_rounds * 8 + rem / group;
    j = rem % group;
  }
  qb = n_qb - 1 - c / hkv;
  h = (c % hkv) * group + j;
}

template <int D, bool SPLIT, typename OutT>
__global__ __launch_bounds__(kThreads) void bsa_kernel(BsaParams P) {
  constexpr int PLANES = SPLIT ? 2 : 1;
  constexpr int NBUF = SPLIT ? 1 : 2;
  constexpr int KP = D + 8;       // K tile pitch (elements): rows 16 B apart mod 128 B
  constexpr int VP = kBlk + 8;    // V^T tile pitch
  constexpr int KT = kBlk * KP;   // K tile elements per plane
  constexpr int VT = D * VP;      // V^T tile elements per plane
  constexpr int STAGE = PLANES * (KT + VT);
  constexpr int KCH = D / 32;     // 16-byte chunks per thread per K tile (and per V^T tile)
  constexpr int NKK = D / 16;     // MFMA k-steps over head_dim
  constexpr int NMD = D / 32;     // 32-row tiles of O^T

  __shared__ __attribute__((aligned(16))) bf16 smem[NBUF * STAGE];
  __shared__ int s_list[kListMax];
  __shared__ int s_cnt;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = lane_id();
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int wq = wave & 3;
  const int wk = wave >> 2;

  int h, qb;
  bsa_decode(blockIdx.x, P.group, P.hkv, P.n_qb, h, qb);
  const int kvh = h / P.group;

  const int64_t row = (int64_t)qb * kBlk + wq * 32 + n;  // this lane's query row
  const int64_t q_glob = P.q_start + row;
  const int64_t wave_q_lo = P.q_start + (int64_t)qb * kBlk + wq * 32;
  const int64_t wave_q_hi = wave_q_lo + 31;

  // ---- query fragments (B operand of S^T = K Q^T), kept in registers
  bf16x8 qf[PLANES][NKK];
  {
    const int64_t off = row * P.q_tok + (int64_t)h * P.q_head + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qf[0][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(P.q_hi + off + kk * 16));
      if constexpr (SPLIT) qf[1][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(P.q_lo + off + kk * 16));
    }
  }

  f32x16 o[NMD];
#pragma unroll
  for (int i = 0; i < NMD; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  // ---- key-block range of this call
  const int64_t nkb = (P.kv_len + kBlk - 1) / kBlk;
  const int64_t gb0 = P.kv_start / kBlk;
  int64_t jb_end = nkb;
  if (P.causal) {
    const int64_t lim = P.q_start + (int64_t)qb * kBlk + (kBlk - 1) - P.kv_start;
    jb_end = lim < 0 ? 0 : (lim / kBlk + 1 < nkb ? lim / kBlk + 1 : nkb);
  }
  const uint8_t* mrow = P.mask ? P.mask + (int64_t)h * P.mask_hs + (int64_t)qb * P.mask_rs + (gb0 - P.mask_off) : nullptr;

  const bf16* kpl[2] = {P.k_hi, P.k_lo};
  const bf16* vpl[2] = {P.vt_hi, P.vt_lo};
  const int64_t kbase = (int64_t)kvh * P.k_head;
  const int64_t vbase = (int64_t)kvh * P.vt_head;

  u32x4 rk[PLANES][KCH], rv[PLANES][KCH];

  auto load_regs = [&](int jb) {
    const int64_t j0 = (int64_t)jb * kBlk;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      const int r = c / (D / 8);
      const int c8 = c % (D / 8);
      const bool ok = j0 + r < P.kv_len;
      const int64_t off = kbase + (j0 + r) * P.k_tok + c8 * 8;
#pragma unroll
      for (int pl = 0; pl < PLANES; ++pl)
        rk[pl][i] = ok ? *reinterpret_cast<const u32x4*>(kpl[pl] + off) : u32x4{0, 0, 0, 0};
      const int d = c / (kBlk / 8);
      const int k8 = c % (kBlk / 8);
      const int64_t voff = vbase + (int64_t)d * P.vt_pitch + j0 + k8 * 8;
#pragma unroll
      for (int pl = 0; pl < PLANES; ++pl) rv[pl][i] = *reinterpret_cast<const u32x4*>(vpl[pl] + voff);
    }
  };
  auto store_lds = [&](int buf) {
    bf16* st = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      const int r = c / (D / 8);
      const int c8 = c % (D / 8);
      const int d = c / (kBlk / 8);
      const int k8 = c % (kBlk / 8);
#pragma unroll
      for (int pl = 0; pl < PLANES; ++pl) {
        *reinterpret_cast<u32x4*>(st + pl * (KT + VT) + r * KP + c8 * 8) = rk[pl][i];
        *reinterpret_cast<u32x4*>(st + pl * (KT + VT) + KT + d * VP + k8 * 8) = rv[pl][i];
      }
    }
  };

  auto compute = [&](int buf, int jb) {
    const int64_t key0 = (int64_t)jb * kBlk + wk * 64;      // local index of this wave's first key
    const int64_t gkey0 = P.kv_start + key0;
    if (P.causal && gkey0 > wave_q_hi) return;              // this key half is entirely in the future
    if (key0 >= P.kv_len) return;                           // past the tail
    const bool need_mask = (key0 + 64 > P.kv_len) || (P.causal && gkey0 + 63 > wave_q_lo);
    const bf16* st = smem + buf * STAGE;

    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int key = wk * 64 + mt * 32 + n;
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(st + key * KP + kk * 16 + 8 * hh));
        s[mt] = mfma32(a, qf[0][kk], s[mt]);
        if constexpr (SPLIT) {
          const bf16x8 alo = as_bf16x8(*reinterpret_cast<const u32x4*>(st + (KT + VT) + key * KP + kk * 16 + 8 * hh));
          s[mt] = mfma32(a, qf[1][kk], s[mt]);
          s[mt] = mfma32(alo, qf[0][kk], s[mt]);
        }
      }
    }

    // scale into log2 units, mask, running max
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[mt][i] * P.scale_log2;
        if (need_mask) {
          const int64_t kl = key0 + mt * 32 + 8 * (i / 4) + 4 * hh + (i % 4);
          const bool ok = kl < P.kv_len && (!P.causal || P.kv_start + kl <= q_glob);
          x = ok ? x : -INFINITY;
        }
        s[mt][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - ref);
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(s[mt][i] - ref);
        s[mt][i] = p;
        psum += p;
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int md = 0; md < NMD; ++md) o[md] *= alpha;

    // P^T fragments straight from the accumulator registers
    bf16x8 pf[PLANES][4];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = s[k2 >> 1][8 * (k2 & 1) + j];
        if constexpr (SPLIT) {
          bf16 hi, lo;
          split_bf16(p, hi, lo);
          pf[0][k2][j] = hi;
          pf[1][k2][j] = lo;
        } else {
          pf[0][k2][j] = (bf16)p;
        }
      }
    }
#pragma unroll
    for (int md = 0; md < NMD; ++md) {
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        const int d = md * 32 + n;
        const int col = wk * 64 + k2 * 16 + 8 * hh;
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(st + KT + d * VP + col));
        o[md] = mfma32(a, pf[0][k2], o[md]);
        if constexpr (SPLIT) {
          const bf16x8 alo = as_bf16x8(*reinterpret_cast<const u32x4*>(st + (KT + VT) + KT + d * VP + col));
          o[md] = mfma32(a, pf[1][k2], o[md]);
          o[md] = mfma32(alo, pf[0][k2], o[md]);
        }
      }
    }
  };

  // ---- walk the kept blocks, kListMax at a time
  for (int64_t seg = 0; seg < jb_end; seg += kListMax) {
    const int64_t seg_end = seg + kListMax < jb_end ? seg + kListMax : jb_end;
    if (wave == 0) {
      int cnt = 0;
      for (int64_t base = seg; base < seg_end; base += 64) {
        const int64_t jb = base + lane;
        const bool keep = jb < seg_end && (mrow == nullptr || mrow[jb] != 0);
        const uint64_t bal = __ballot(keep);
        const int pos = cnt + __popcll(bal & ((1ull << lane) - 1));
        if (keep) s_list[pos] = (int)jb;
        cnt += __popcll(bal);
      }
      if (lane == 0) s_cnt = cnt;
    }
    __syncthreads();
    const int cnt = s_cnt;
    if (cnt > 0) {
      load_regs(s_list[0]);
      store_lds(0);
      __syncthreads();
      for (int it = 0; it < cnt; ++it) {
        const int jb = s_list[it];
        if constexpr (NBUF == 2) {
          const int buf = it & 1;
          if (it + 1 < cnt) load_regs(s_list[it + 1]);
          compute(buf, jb);
          if (it + 1 < cnt) store_lds(buf ^ 1);
          __syncthreads();
        } else {
          compute(0, jb);
          __syncthreads();
          if (it + 1 < cnt) {
            load_regs(s_list[it + 1]);
            store_lds(0);
          }
          __syncthreads();
        }
      }
    }
    __syncthreads();  // s_list / s_cnt are rewritten by the next segment
  }

  // ---- merge the two key halves of each query row, normalise, write
  const float l_row = halves_sum(l_run);
  float* xch = reinterpret_cast<float*>(smem);  // [4][NMD*16 + 2][64]
  constexpr int XV = NMD * 16 + 2;
  if (wk == 1) {
    float* dst = xch + wq * XV * 64;
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[(md * 16 + i) * 64 + lane] = o[md][i];
    dst[(NMD * 16) * 64 + lane] = m_run;
    dst[(NMD * 16 + 1) * 64 + lane] = l_row;
  }
  __syncthreads();
  if (wk == 0) {
    const float* src = xch + wq * XV * 64;
    const float m1 = src[(NMD * 16) * 64 + lane];
    const float l1 = src[(NMD * 16 + 1) * 64 + lane];
    const float m = fmaxf(m_run, m1);
    float a0 = 0.f, a1 = 0.f, lse_v = -INFINITY, inv = 0.f;
    if (m != -INFINITY) {
      a0 = fast_exp2(m_run - m);
      a1 = fast_exp2(m1 - m);
      const float l = l_row * a0 + l1 * a1;
      inv = 1.f / l;
      lse_v = (m + log2f(l)) * kLn2;
    }
    OutT* out = reinterpret_cast<OutT*>(P.out);
    const int64_t obase = row * ((int64_t)P.hq * D) + (int64_t)h * D;
#pragma unroll
    for (int md = 0; md < NMD; ++md) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = md * 32 + 8 * g4 + 4 * hh;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = g4 * 4 + e;
          v[e] = (o[md][i] * a0 + src[(md * 16 + i) * 64 + lane] * a1) * inv;
        }
        if constexpr (sizeof(OutT) == 2) {
          bf16x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[e] = (bf16)v[e];
          *reinterpret_cast<u32x2*>(out + obase + d0) = __builtin_bit_cast(u32x2, pk);
        } else {
          *reinterpret_cast<f32x4*>(out + obase + d0) = f32x4{v[0], v[1], v[2], v[3]};
        }
      }
    }
    if (hh == 0) P.lse[(int64_t)h * P.q_len + row] = lse_v;
  }
}

// ---------------------------------------------------------------------------
// Tile layout of the bf16 kernel (bsa3_kernel below).
//
//   * wave w of a group owns query rows 32w .. 32w+31 against all 128 keys of
//     each kept block, so no cross-wave merge is needed inside a group;
//   * K and V^T tiles go global -> LDS with buffer_load_dwordx4 ... lds (no
//     staging registers): lane L of a wave-instruction lands at byte 16*L of a
//     1 KiB run, so the 16-byte chunk a lane fetches is chosen such that LDS
//     slot s of row r holds chunk s ^ (r mod 16) (XOR swizzle: fragment reads
//     of 16 consecutive rows hit 16 distinct bank groups);
//   * the running max is only moved when a row's max grows by more than 2^8
//     (P <= 256 in between), so the O rescale is rare.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ bf16x8 lds_frag(const char* tile, int row, int chunk) {
  constexpr int KCH = D / 8;
  return *reinterpret_cast<const bf16x8*>(tile + row * (KCH * 16) + ((chunk ^ (row & (KCH - 1))) << 4));
}

// Raw buffer descriptor over [base, base + bytes); loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from descriptor offset voff into LDS: lane L lands at lds + 16 L.
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Next work-order entry for this workgroup, longest first (-1: every entry is taken).  Workgroups at or past the
// entry count return before calling this.  The first n = min(M.direct, entries) workgroups (dispatched first, one
// per resident slot) take the entries 0 .. n-1 without a ticket, each XCD a contiguous run of them (workgroup b
// runs on XCD b mod 8), so that neighbouring entries (often the query heads of one kv head, reading the same
// tiles) share an L2; the others take tickets from n on.  A ticket stays below the grid size, which the order
// array holds, so the entry is read without waiting for the comparison with the entry count.
__device__ __forceinline__ int take_entry(const BsaMulti& M) {
  const int total = M.ctl[1];
  const int n = M.direct < total ? M.direct : total;
  const int b = (int)blockIdx.x;
  const int t = b < n ? xcd_remap(b, n) : n + atomicAdd(&M.ctl[0], 1);
  const int e = M.order[t];
  return t < total ? e : -1;
}

// Segment of work item `item` (kernel-argument segments) and the first item of that segment.
__device__ __forceinline__ const BsaParams& find_seg(const BsaMulti& M, int item, int& item0) {
  int sidx = 0;
  while (sidx + 1 < M.n_seg && item >= M.wg_end[sidx]) ++sidx;
  item0 = sidx ? M.wg_end[sidx - 1] : 0;
  return M.seg[sidx];
}

// Packed batch: the sequence of work item `item` (binary search of the records' item prefix ends,
// uniform per workgroup) and its problem, seg[0]'s shared fields taken relative to the sequence: its
// query / key / packed-V rows, causal with the queries at the end of its keys, its compact block mask
// [hq][q_len/128][k_len/128], its output rows and its LSE block [hq][q_len].  The records count items
// per (query head, query block); head-pair items are ceil(group / 2) per kv head and query block.
template <int D, typename OutT>
__device__ __forceinline__ BsaParams varlen_params(const BsaMulti& M, int item, int& item0) {
  const int hq = M.seg[0].hq;
  const int per_qb = M.pair ? M.seg[0].hkv * ((M.seg[0].group + 1) / 2) : hq;  // items per query block
  auto end_of = [&](int s) {
    const int e = __builtin_amdgcn_readfirstlane(M.seqs[s].sel_end);
    return M.pair ? e / hq * per_qb : e;
  };
  int lo = 0, hi = M.n_seg - 1;
  while (lo < hi) {
    const int md = (lo + hi) >> 1;
    if (item < end_of(md)) hi = md;
    else lo = md + 1;
  }
  item0 = lo ? end_of(lo - 1) : 0;
  const VarlenSeq& v = M.seqs[lo];
  const int q0 = __builtin_amdgcn_readfirstlane(v.q0);
  const int ql = __builtin_amdgcn_readfirstlane(v.q_len);
  const int k0 = __builtin_amdgcn_readfirstlane(v.k0);
  const int kl = __builtin_amdgcn_readfirstlane(v.k_len);
  BsaParams P = M.seg[0];
  P.q_hi += (int64_t)q0 * P.q_tok;
  P.k_hi += (int64_t)k0 * P.k_tok;
  P.vt_hi += k0;
  P.q_len = ql;
  P.kv_len = kl;
  P.n_qb = ql / kBlk;
  P.q_start = kl - ql;
  P.kv_start = 0;
  if (P.mask) {
    P.mask += rfl64(v.out_off);
    P.mask_rs = kl / kBlk;
    P.mask_hs = (int64_t)(ql / kBlk) * (kl / kBlk);
    P.mask_off = 0;
  }
  P.out = static_cast<OutT*>(P.out) + (int64_t)q0 * P.hq * D;
  P.lse += (int64_t)P.hq * q0;
  return P;
}

// ---------------------------------------------------------------------------
// Ping-pong form (bf16, head_dim 128): one workgroup of eight waves per CU.
// Waves 0-3 (group 0) and 4-7 (group 1) hold the same 128 query rows (32 per
// wave) and take alternate kept key blocks, each group with
// its own K and V^T tiles in LDS.  A barrier of all eight waves ends every
// tick; in each tick one group is in its matrix phase (P V^T of its previous
// block, then K Q^T of its current block) while the other is in its vector
// phase (loads of its next tiles are issued, then the online softmax of its
// current block), so every SIMD holds one wave of each kind.  The two groups'
// running (max, sum, output) are merged through LDS at the end.
// ---------------------------------------------------------------------------
template <int D, typename OutT>
__device__ __forceinline__ void bsa3_body(const BsaMulti& M, const BsaParams& P, int item, int part, int bid) {
  static_assert(D == 128, "ping-pong form: head_dim 128");
  constexpr int KCH = D / 8;
  constexpr int KTB = 128 * KCH * 16;     // K tile bytes
  constexpr int VTB = D * 256;            // V^T tile bytes
  constexpr int NKK = D / 16;
  constexpr int NMD = D / 32;
  constexpr int KI = KCH / 2;
  constexpr int VI = D / 16;
  constexpr float kRescale = 8.0f;
  __shared__ __attribute__((aligned(1024))) char smem[2 * (KTB + VTB)];
  __shared__ int s_list[kListMax];
  __shared__ int s_cnt;
  __shared__ int s_wcnt[8];

  const int wave8 = wave_id();
  const int grp = wave8 >> 2;
  const int wave = wave8 & 3;
  const int lane = lane_id();
  const int n = lane & 31;
  const int hh = lane >> 5;

  int h, qb;
  bsa_decode(bid, P.group, P.hkv, P.n_qb, h, qb);
  const int kvh = h / P.group;
  // this lane's query row is row0 + n (row0 wave-uniform); no 64-bit per-lane index stays live
  const int64_t row0 = (int64_t)qb * kBlk + wave * 32;
  const int64_t wave_q_lo = P.q_start + row0;
  const float c = P.scale_log2;

  bf16x8 qf[NKK];
  {
    const int64_t off = (row0 + n) * P.q_tok + (int64_t)h * P.q_head + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(P.q_hi + off + kk * 16));
  }
  f32x16 o[NMD];
#pragma unroll
  for (int i = 0; i < NMD; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int64_t nkb = (P.kv_len + kBlk - 1) / kBlk;
  const int64_t gb0 = P.kv_start / kBlk;
  int64_t jb_end = nkb;
  if (P.causal) {
    const int64_t lim = P.q_start + (int64_t)qb * kBlk + (kBlk - 1) - P.kv_start;
    jb_end = lim < 0 ? 0 : (lim / kBlk + 1 < nkb ? lim / kBlk + 1 : nkb);
  }
  int64_t jb_lo = 0;
  if (part == 1) jb_end = M.mid[item];
  if (part == 2) jb_lo = M.mid[item];
  const uint8_t* mrow =
      P.mask ? P.mask + (int64_t)h * P.mask_hs + (int64_t)qb * P.mask_rs + (gb0 - P.mask_off) : nullptr;
  const bf16* kg = P.k_hi + (int64_t)kvh * P.k_head;
  const bf16* vg = P.vt_hi + (int64_t)kvh * P.vt_head;
  char* kt = smem + grp * (KTB + VTB);
  char* vt = kt + KTB;
  // loop-invariant arguments in registers (the tick loop would otherwise reload them from the kernel arguments)
  const int64_t kv_len = P.kv_len, kv_start = P.kv_start, k_tok = P.k_tok, vt_pitch = P.vt_pitch;
  const bool causal = P.causal != 0;

  // Piece i of this wave's share of a K (V^T) tile covers rows r = 32 wave + 4 i + lane / 16 (16 lanes of
  // 16 bytes per 256-byte row), lane chunk (lane % 16) ^ (r % 16).  r % 16 = 4 (i % 4) + lane / 16, so the
  // byte offset is kx[i % 4] + i * 4 rows: four per-lane bases per tile instead of eight offsets.
  static_assert(KCH == 16 && KI == 8 && VI == 8, "tile pieces: 16 chunks per row, 8 pieces per wave");
  uint32_t kx[4], vx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wave * 32 + (lane >> 4);
    const int ch = (lane & 15) ^ (4 * j + (lane >> 4));
    kx[j] = (uint32_t)(((int64_t)r * k_tok + ch * 8) * 2);
    vx[j] = (uint32_t)(((int64_t)r * vt_pitch + ch * 8) * 2);
  }
  const uint32_t kstep = (uint32_t)(8 * k_tok);     // 4 rows of K, bytes
  const uint32_t vstep = (uint32_t)(8 * vt_pitch);  // 4 rows of V^T, bytes
  // The LDS destination of piece i is this wave's first piece + i KiB.  The first piece's offset goes through an
  // empty asm at every call, so the compiler derives the eight destinations from one register each time instead
  // of keeping all sixteen (K and V) in scalar registers across the loop.
  auto issue_k = [&](int jb) {
    const int64_t j0 = (int64_t)jb * kBlk;
    const int64_t rows = kv_len - j0 < kBlk ? kv_len - j0 : kBlk;
    const auto rs = tile_rsrc(kg + j0 * k_tok, (uint32_t)(((rows - 1) * k_tok + D) * 2));
    uint32_t d0 = (uint32_t)(wave * KI * 1024);
    asm volatile("" : "+s"(d0));
#pragma unroll
    for (int i = 0; i < KI; ++i) buf2lds16(rs, kx[i & 3] + i * kstep, kt + d0 + i * 1024);
  };
  auto issue_v = [&](int jb) {
    const auto rs = tile_rsrc(vg + (int64_t)jb * kBlk, (uint32_t)(((int64_t)(D - 1) * vt_pitch + kBlk) * 2));
    uint32_t d0 = (uint32_t)(wave * VI * 1024);
    asm volatile("" : "+s"(d0));
#pragma unroll
    for (int i = 0; i < VI; ++i) buf2lds16(rs, vx[i & 3] + i * vstep, vt + d0 + i * 1024);
  };

  f32x16 sacc[4];
  bf16x8 pf[8];
  for (int64_t seg = jb_lo; seg < jb_end; seg += kListMax) {
    const int64_t seg_end = seg + kListMax < jb_end ? seg + kListMax : jb_end;
    {
      // each of the eight waves scans an eighth of the segment: count, exchange, write
      // a wave's share is at most two rounds of 64 columns: both rounds' bytes are read at once and their
      // ballots kept, so the mask row is read once
      static_assert(kListMax / 8 <= 128, "at most two 64-column rounds per wave");
      const int64_t part8 = ((seg_end - seg + 7) / 8 + 63) / 64 * 64;
      const int64_t w0 = seg + wave8 * part8;
      const int64_t w1 = w0 + part8 < seg_end ? w0 + part8 : seg_end;
      bool hit[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int64_t jb = w0 + 64 * t + lane;
        hit[t] = jb < w1 && (mrow == nullptr || mrow[jb] != 0);
      }
      const uint64_t bal0 = __ballot(hit[0]);
      const uint64_t bal1 = __ballot(hit[1]);
      if (lane == 0) s_wcnt[wave8] = __popcll(bal0) + __popcll(bal1);
      __syncthreads();
      int pos0 = 0;
      for (int w = 0; w < wave8; ++w) pos0 += s_wcnt[w];
      const uint64_t below = (1ull << lane) - 1;
      if (hit[0]) s_list[pos0 + __popcll(bal0 & below)] = (int)(w0 + lane);
      pos0 += __popcll(bal0);
      if (hit[1]) s_list[pos0 + __popcll(bal1 & below)] = (int)(w0 + 64 + lane);
      pos0 += __popcll(bal1);
      if (wave8 == 7 && lane == 0) s_cnt = pos0;
    }
    __syncthreads();
    const int cnt = s_cnt;
    // this group's blocks: list positions grp, grp + 2, ...; both groups pass the same barriers
    const int n_own = grp == 0 ? (cnt + 1) / 2 : cnt / 2;
    const int iters = cnt == 0 ? 0 : (cnt + 1) / 2 + 1;
    if (n_own > 0) issue_k(s_list[grp]);
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
    __syncthreads();
    // matrix phase i: P V^T of block i-1, then K Q^T of block i.  Operand fragments are read one
    // contraction step ahead (a ring of four), so an LDS read has four MFMAs to land.
    static_assert(NMD == 4, "fragment ring: four output / score tiles");
    auto mphase = [&](int i) {
      __builtin_amdgcn_s_setprio(2);  // the matrix phase's MFMAs issue ahead of the other group's softmax
      bf16x8 fr[4];
      if (i >= 1 && i - 1 < n_own) {
#pragma unroll
        for (int md = 0; md < NMD; ++md) fr[md] = lds_frag<128>(vt, md * 32 + n, hh);
#pragma unroll
        for (int k2 = 0; k2 < 8; ++k2)
#pragma unroll
          for (int md = 0; md < NMD; ++md) {
            o[md] = mfma32(fr[md], pf[k2], o[md]);
            if (k2 + 1 < 8) fr[md] = lds_frag<128>(vt, md * 32 + n, 2 * (k2 + 1) + hh);
            __builtin_amdgcn_sched_barrier(0);  // keep the read ahead of the next MFMAs
          }
      }
      if (i < n_own) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) sacc[mt] = f32x16{};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) fr[mt] = lds_frag<D>(kt, mt * 32 + n, hh);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            sacc[mt] = mfma32(fr[mt], qf[kk], sacc[mt]);
            if (kk + 1 < NKK) fr[mt] = lds_frag<D>(kt, mt * 32 + n, 2 * (kk + 1) + hh);
            __builtin_amdgcn_sched_barrier(0);  // keep the read ahead of the next MFMAs
          }
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // vector phase i: loads for matrix phase i+1 (K of block i+1, V of block i), softmax of block i
    auto vphase = [&](int i) {
      if (i + 1 < n_own) issue_k(s_list[grp + 2 * (i + 1)]);
      if (i < n_own) {
        const int jb = __builtin_amdgcn_readfirstlane(s_list[grp + 2 * i]);
        issue_v(jb);
        const int64_t key0 = (int64_t)jb * kBlk;
        if ((key0 + kBlk > kv_len) || (causal && kv_start + key0 + kBlk - 1 > wave_q_lo)) {
          int64_t lim = kv_len - 1 - key0;
          const int64_t qlim = wave_q_lo - kv_start - key0 + n;  // causal limit of this lane's row
          if (causal && qlim < lim) lim = qlim;
          const int lim32 = (int)(lim < -1 ? -1 : (lim > kBlk ? kBlk : lim)) - 4 * hh;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int kl = mt * 32 + 8 * (e / 4) + (e % 4);
              sacc[mt][e] = kl <= lim32 ? sacc[mt][e] : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[mt][e]);
        mx = halves_max(mx);
        const bool upd = mx > m_run && (m_run == -INFINITY || (mx - m_run) * c > kRescale);
        if (__builtin_amdgcn_ballot_w64(upd)) {
          const float m_new = upd ? mx : m_run;
          const float alpha = upd ? fast_exp2((m_run - m_new) * c) : 1.f;
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int md = 0; md < NMD; ++md) o[md] *= alpha;
        }
        const float mref = m_run == -INFINITY ? 0.f : m_run * c;
#pragma unroll
        for (int k2 = 0; k2 < 8; ++k2)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float p = fast_exp2(__builtin_fmaf(sacc[k2 >> 1][8 * (k2 & 1) + j], c, -mref));
            l_run += p;
            pf[k2][j] = (bf16)p;
          }
      }
      __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's loads for the next matrix phase landed
    };
    // Both groups run the same loop; group 1 starts one barrier later and group 0 passes one more barrier
    // at the end (the hardware barrier counts waves, and these branches are uniform per wave), so group
    // 1's matrix phase i meets group 0's vector phase i and the other way round.
    if (grp == 1) __syncthreads();
    for (int i = 0; i < iters; ++i) {
      mphase(i);
      __syncthreads();
      vphase(i);
      __syncthreads();
    }
    if (grp == 0) __syncthreads();
  }

  // merge group 1's running state into group 0's (same lane layout), through LDS
  __syncthreads();
  f32x4* xo = reinterpret_cast<f32x4*>(smem);                              // [4 waves][16][64 lanes]
  float* xm = reinterpret_cast<float*>(smem + 4 * 16 * 64 * sizeof(f32x4));  // [4 waves][64 lanes]
  float* xl = xm + 4 * 64;
  if (grp == 1) {
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        xo[(wave * 16 + md * 4 + g4) * 64 + lane] =
            f32x4{o[md][g4 * 4], o[md][g4 * 4 + 1], o[md][g4 * 4 + 2], o[md][g4 * 4 + 3]};
    xm[wave * 64 + lane] = m_run;
    xl[wave * 64 + lane] = l_run;
  }
  __syncthreads();
  // bf16 rows of a whole item go out through LDS: the eight waves then write whole 256-byte rows (a lane's
  // own row pieces are 8 bytes in rows 8 KiB apart, which the memory system takes as partial-line writes)
  constexpr bool kStageOut = sizeof(OutT) == 2;
  const bool stage = kStageOut && part == 0;
  constexpr int kStgPitch = D * 2 + 16;  // padded row pitch: the 8-byte writes of a column spread over banks
  char* stg = smem + 80 * 1024;          // after group 1's state (64 KiB + 2 KiB)
  static_assert(80 * 1024 + 128 * kStgPitch <= 2 * (KTB + VTB), "staging fits the tile buffers");
  if (grp == 1 && !stage) return;
  if (grp == 0) {
  {
    const float m1 = xm[wave * 64 + lane];
    const float l1 = xl[wave * 64 + lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m) * c);
    const float a1 = m1 == -INFINITY ? 0.f : fast_exp2((m1 - m) * c);
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 y = xo[(wave * 16 + md * 4 + g4) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[md][g4 * 4 + e] = o[md][g4 * 4 + e] * a0 + y[e] * a1;
      }
    l_run = l_run * a0 + l1 * a1;
    m_run = m;
  }

  const float l_row = halves_sum(l_run);
  float inv = 0.f, lse_v = -INFINITY;
  if (l_row > 0.f) {
    inv = 1.f / l_row;
    lse_v = (m_run * c + log2f(l_row)) * kLn2;
  }
  if (part != 0) {
    const size_t ps = (size_t)(2 * M.slot[item] + part - 1) * kBlk + wave * 32 + n;
    float* po = M.part_o + ps * D;
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = md * 32 + 8 * g4 + 4 * hh;
        *reinterpret_cast<f32x4*>(po + d0) = f32x4{o[md][g4 * 4] * inv, o[md][g4 * 4 + 1] * inv,
                                                   o[md][g4 * 4 + 2] * inv, o[md][g4 * 4 + 3] * inv};
      }
    if (hh == 0) M.part_lse[ps] = lse_v;
    return;
  }
  if (hh == 0) P.lse[(int64_t)h * P.q_len + row0 + n] = lse_v;
  OutT* out = reinterpret_cast<OutT*>(P.out);
  const int64_t obase = (row0 + n) * ((int64_t)P.hq * D) + (int64_t)h * D;
#pragma unroll
  for (int md = 0; md < NMD; ++md)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = md * 32 + 8 * g4 + 4 * hh;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = o[md][g4 * 4 + e] * inv;
      if constexpr (kStageOut) {
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = (bf16)v[e];
        *reinterpret_cast<u32x2*>(stg + (wave * 32 + n) * kStgPitch + d0 * 2) = __builtin_bit_cast(u32x2, pk);
      } else {
        *reinterpret_cast<f32x4*>(out + obase + d0) = f32x4{v[0], v[1], v[2], v[3]};
      }
    }
  if (!stage) return;
  }
  __syncthreads();
  // 128 rows x 16 pieces of 16 bytes over 512 lanes: lanes 16 j .. 16 j + 15 write one row
  {
    OutT* out = reinterpret_cast<OutT*>(P.out);
    const int64_t rbase = (int64_t)qb * kBlk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = j * 512 + (int)threadIdx.x;
      const int r = q >> 4, ch = q & 15;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stg + r * kStgPitch + ch * 16);
      *reinterpret_cast<u32x4*>(out + (rbase + r) * ((int64_t)P.hq * D) + (int64_t)h * D + ch * 8) = val;
    }
  }
}

template <int D, typename OutT, bool VARLEN>
__global__ __launch_bounds__(512, 1) void bsa3_kernel(BsaMulti M) {
  __shared__ int s_item;
  int item = (int)blockIdx.x, part = 0;
  if (M.order) {
    const int n_items = M.n_items;
    if ((int)blockIdx.x >= n_items && (int)blockIdx.x >= n_items + M.ctl[2]) return;
    if (threadIdx.x == 0) s_item = take_entry(M);
    __syncthreads();
    const int e = __builtin_amdgcn_readfirstlane(s_item);
    if (e < 0) return;
    item = e >> 2;
    part = e & 3;
  }
  int item0;
  if constexpr (VARLEN) {
    const BsaParams P = varlen_params<D, OutT>(M, item, item0);
    bsa3_body<D, OutT>(M, P, item, part, item - item0);
  } else {
    const BsaParams& P = find_seg(M, item, item0);
    bsa3_body<D, OutT>(M, P, item, part, item - item0);
  }
}

// ---------------------------------------------------------------------------
// Pair form (bf16, head_dim 128, an even number of query heads per kv head):
// one workgroup of eight waves per CU computes two query heads of one kv head
// for one 128-row query block.  The query heads of a kv head keep nearly the
// same key blocks, so each K / V^T tile is brought into LDS once for both:
// group g (waves 4g .. 4g+3, 32 rows each) computes head 2p + g over the union
// of the two heads' kept lists, skipping (no MFMA, no softmax) the blocks its
// own head did not keep, so each head's result is exactly its own.  The groups
// stay one phase apart as in the ping-pong form (group 0's matrix phase of
// block i meets group 1's vector phase of block i-1), and the tiles are double
// buffered: K of block i in K slot i % 2, V^T of block i in V slot i % 2.
// Group 1 brings K of block i + 2 and V^T of block i + 1 during its vector
// phase of block i, two phases before group 0 reads them (it waits for them at
// the end of its next matrix phase); group 0's vector phase is softmax only.
// A head-block thus costs half the tile loads of the single-head form.
// ---------------------------------------------------------------------------
// Pair items take the query heads of kv head v two at a time: (v g, v g + 1), (v g + 2, v g + 3), ...; with an
// odd group size g the last item of each kv head holds one head (its second group only helps bring the tiles).
// Item hp (over ceil(g / 2) items per kv head) -> its first query head and its head count.
__device__ __forceinline__ void pair_heads(int hp, int group, int& h0, int& nh) {
  const int per = (group + 1) / 2;
  const int kvh = hp / per, j = hp % per;
  h0 = kvh * group + 2 * j;
  nh = 2 * j + 1 < group ? 2 : 1;
}

template <int D, typename OutT>
__device__ __forceinline__ void bsa_pair_body(const BsaMulti& M, const BsaParams& P, int item, int part, int bid) {
  static_assert(D == 128, "pair form: head_dim 128");
  constexpr int KCH = D / 8;
  constexpr int KTB = 128 * KCH * 16;     // K tile bytes
  constexpr int VTB = D * 256;            // V^T tile bytes
  constexpr int NKK = D / 16;
  constexpr int NMD = D / 32;
  constexpr int KI = KCH / 2;
  constexpr int VI = D / 16;
  constexpr float kRescale = 8.0f;
  constexpr int kOwnShift = 29;           // list entry: key block | (kept by head 2p) << 29 | (by 2p + 1) << 30
  constexpr int kBlockBits = (1 << kOwnShift) - 1;
  __shared__ __attribute__((aligned(1024))) char smem[2 * (KTB + VTB)];  // K slots 0, 1, then V^T slots 0, 1
  __shared__ int s_list[kListMax];
  __shared__ int s_cnt;
  __shared__ int s_wcnt[8];

  const int wave8 = wave_id();
  const int grp = wave8 >> 2;
  const int wave = wave8 & 3;
  const int lane = lane_id();
  const int n = lane & 31;
  const int hh = lane >> 5;

  int hp, qb, h0, nh;
  bsa_decode(bid, (P.group + 1) / 2, P.hkv, P.n_qb, hp, qb);
  pair_heads(hp, P.group, h0, nh);
  const bool active = grp < nh;           // group 1 of a one-head item computes nothing
  const int h = h0 + (active ? grp : 0);  // this group's query head
  const int kvh = h / P.group;
  const int64_t row0 = (int64_t)qb * kBlk + wave * 32;
  const int64_t wave_q_lo = P.q_start + row0;
  const float c = P.scale_log2;

  bf16x8 qf[NKK];
  {
    const int64_t off = (row0 + n) * P.q_tok + (int64_t)h * P.q_head + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(P.q_hi + off + kk * 16));
  }
  f32x16 o[NMD];
#pragma unroll
  for (int i = 0; i < NMD; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int64_t nkb = (P.kv_len + kBlk - 1) / kBlk;
  const int64_t gb0 = P.kv_start / kBlk;
  int64_t jb_end = nkb;
  if (P.causal) {
    const int64_t lim = P.q_start + (int64_t)qb * kBlk + (kBlk - 1) - P.kv_start;
    jb_end = lim < 0 ? 0 : (lim / kBlk + 1 < nkb ? lim / kBlk + 1 : nkb);
  }
  int64_t jb_lo = 0;
  if (part == 1) jb_end = M.mid[item];
  if (part == 2) jb_lo = M.mid[item];
  const uint8_t* mrow0 =
      P.mask ? P.mask + (int64_t)h0 * P.mask_hs + (int64_t)qb * P.mask_rs + (gb0 - P.mask_off) : nullptr;
  const uint8_t* mrow1 = P.mask ? mrow0 + P.mask_hs : nullptr;  // read only when the item has a second head
  const bf16* kg = P.k_hi + (int64_t)kvh * P.k_head;
  const bf16* vg = P.vt_hi + (int64_t)kvh * P.vt_head;
  const int64_t kv_len = P.kv_len, kv_start = P.kv_start, k_tok = P.k_tok, vt_pitch = P.vt_pitch;
  const bool causal = P.causal != 0;
  const int own_bit = active ? 1 << (kOwnShift + grp) : 0;

  // Piece i of this wave's share of a tile covers rows r = 32 wave + 4 i + lane / 16, lane chunk
  // (lane % 16) ^ (r % 16): byte offset kx[i % 4] + i * 4 rows (as in the ping-pong form).
  static_assert(KCH == 16 && KI == 8 && VI == 8, "tile pieces: 16 chunks per row, 8 pieces per wave");
  uint32_t kx[4], vx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wave * 32 + (lane >> 4);
    const int ch = (lane & 15) ^ (4 * j + (lane >> 4));
    kx[j] = (uint32_t)(((int64_t)r * k_tok + ch * 8) * 2);
    vx[j] = (uint32_t)(((int64_t)r * vt_pitch + ch * 8) * 2);
  }
  const uint32_t kstep = (uint32_t)(8 * k_tok);
  const uint32_t vstep = (uint32_t)(8 * vt_pitch);
  // K of block jb into K slot sl; the four waves of the calling group bring the whole tile
  auto issue_k = [&](int jb, int sl) {
    const int64_t j0 = (int64_t)jb * kBlk;
    const int64_t rows = kv_len - j0 < kBlk ? kv_len - j0 : kBlk;
    const auto rs = tile_rsrc(kg + j0 * k_tok, (uint32_t)(((rows - 1) * k_tok + D) * 2));
    uint32_t d0 = (uint32_t)(sl * KTB + wave * KI * 1024);
    asm volatile("" : "+s"(d0));
#pragma unroll
    for (int i = 0; i < KI; ++i) buf2lds16(rs, kx[i & 3] + i * kstep, smem + d0 + i * 1024);
  };
  auto issue_v = [&](int jb, int sl) {
    const auto rs = tile_rsrc(vg + (int64_t)jb * kBlk, (uint32_t)(((int64_t)(D - 1) * vt_pitch + kBlk) * 2));
    uint32_t d0 = (uint32_t)(2 * KTB + sl * VTB + wave * VI * 1024);
    asm volatile("" : "+s"(d0));
#pragma unroll
    for (int i = 0; i < VI; ++i) buf2lds16(rs, vx[i & 3] + i * vstep, smem + d0 + i * 1024);
  };
  auto entry = [&](int i) { return __builtin_amdgcn_readfirstlane(s_list[i]); };

  f32x16 sacc[4];
  bf16x8 pf[8];
  for (int64_t seg = jb_lo; seg < jb_end; seg += kListMax) {
    const int64_t seg_end = seg + kListMax < jb_end ? seg + kListMax : jb_end;
    {
      // union list of the two heads' kept blocks, each entry tagged with the heads that kept it: each of the
      // eight waves reads at most two rounds of 64 columns of both mask rows at once
      static_assert(kListMax / 8 <= 128, "at most two 64-column rounds per wave");
      const int64_t part8 = ((seg_end - seg + 7) / 8 + 63) / 64 * 64;
      const int64_t w0 = seg + wave8 * part8;
      const int64_t w1 = w0 + part8 < seg_end ? w0 + part8 : seg_end;
      int tag[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int64_t jb = w0 + 64 * t + lane;
        const bool in = jb < w1;
        const bool a = in && (mrow0 == nullptr || mrow0[jb] != 0);
        const bool b = nh == 2 && in && (mrow1 == nullptr || mrow1[jb] != 0);
        tag[t] = (a ? 1 << kOwnShift : 0) | (b ? 2 << kOwnShift : 0);
      }
      const uint64_t bal0 = __ballot(tag[0] != 0);
      const uint64_t bal1 = __ballot(tag[1] != 0);
      if (lane == 0) s_wcnt[wave8] = __popcll(bal0) + __popcll(bal1);
      __syncthreads();
      int pos0 = 0;
      for (int w = 0; w < wave8; ++w) pos0 += s_wcnt[w];
      const uint64_t below = (1ull << lane) - 1;
      if (tag[0]) s_list[pos0 + __popcll(bal0 & below)] = (int)(w0 + lane) | tag[0];
      pos0 += __popcll(bal0);
      if (tag[1]) s_list[pos0 + __popcll(bal1 & below)] = (int)(w0 + 64 + lane) | tag[1];
      pos0 += __popcll(bal1);
      if (wave8 == 7 && lane == 0) s_cnt = pos0;
    }
    __syncthreads();
    const int cnt = s_cnt;
    const int iters = cnt == 0 ? 0 : cnt + 1;
    // K of the first two blocks (group 0 the first, group 1 the second) and V^T of the first (group 1)
    if (grp < cnt) issue_k(entry(grp) & kBlockBits, grp);
    if (grp == 1 && cnt > 0) issue_v(entry(0) & kBlockBits, 0);
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
    __syncthreads();
    static_assert(NMD == 4, "fragment ring: four output / score tiles");
    // matrix phase i: P V^T of block i-1 (V slot (i-1) % 2), then K Q^T of block i (K slot i % 2), each only if
    // this group's head kept the block
    auto mphase = [&](int i) {
      // Raised issue priority for the matrix phase: the SIMD otherwise favours the older wave, so group 1's MFMAs
      // waited behind group 0's softmax instructions (its matrix phase ran a quarter longer than group 0's).
      __builtin_amdgcn_s_setprio(2);
      bf16x8 fr[4];
      if (i >= 1 && (entry(i - 1) & own_bit)) {
        const char* vt = smem + 2 * KTB + ((i - 1) & 1) * VTB;
#pragma unroll
        for (int md = 0; md < NMD; ++md) fr[md] = lds_frag<128>(vt, md * 32 + n, hh);
#pragma unroll
        for (int k2 = 0; k2 < 8; ++k2)
#pragma unroll
          for (int md = 0; md < NMD; ++md) {
            o[md] = mfma32(fr[md], pf[k2], o[md]);
            if (k2 + 1 < 8) fr[md] = lds_frag<128>(vt, md * 32 + n, 2 * (k2 + 1) + hh);
            __builtin_amdgcn_sched_barrier(0);
          }
      }
      if (i < cnt && (entry(i) & own_bit)) {
        const char* kt = smem + (i & 1) * KTB;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) sacc[mt] = f32x16{};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) fr[mt] = lds_frag<D>(kt, mt * 32 + n, hh);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            sacc[mt] = mfma32(fr[mt], qf[kk], sacc[mt]);
            if (kk + 1 < NKK) fr[mt] = lds_frag<D>(kt, mt * 32 + n, 2 * (kk + 1) + hh);
            __builtin_amdgcn_sched_barrier(0);
          }
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // vector phase i: group 1 brings V^T of block i + 1 and K of block i + 2; then the softmax of block i
    auto vphase = [&](int i) {
      if (grp == 1 && i + 1 < cnt) issue_v(entry(i + 1) & kBlockBits, (i + 1) & 1);
      if (grp == 1 && i + 2 < cnt) issue_k(entry(i + 2) & kBlockBits, i & 1);
      if (i < cnt) {
        const int e = entry(i);
        if (e & own_bit) {
          const int64_t key0 = (int64_t)(e & kBlockBits) * kBlk;
          if ((key0 + kBlk > kv_len) || (causal && kv_start + key0 + kBlk - 1 > wave_q_lo)) {
            int64_t lim = kv_len - 1 - key0;
            const int64_t qlim = wave_q_lo - kv_start - key0 + n;
            if (causal && qlim < lim) lim = qlim;
            const int lim32 = (int)(lim < -1 ? -1 : (lim > kBlk ? kBlk : lim)) - 4 * hh;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
              for (int q = 0; q < 16; ++q) {
                const int kl = mt * 32 + 8 * (q / 4) + (q % 4);
                sacc[mt][q] = kl <= lim32 ? sacc[mt][q] : -INFINITY;
              }
          }
          float mx = -INFINITY;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int q = 0; q < 16; ++q) mx = fmaxf(mx, sacc[mt][q]);
          mx = halves_max(mx);
          const bool upd = mx > m_run && (m_run == -INFINITY || (mx - m_run) * c > kRescale);
          if (__builtin_amdgcn_ballot_w64(upd)) {
            const float m_new = upd ? mx : m_run;
            const float alpha = upd ? fast_exp2((m_run - m_new) * c) : 1.f;
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int md = 0; md < NMD; ++md) o[md] *= alpha;
          }
          const float mref = m_run == -INFINITY ? 0.f : m_run * c;
#pragma unroll
          for (int k2 = 0; k2 < 8; ++k2)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float p = fast_exp2(__builtin_fmaf(sacc[k2 >> 1][8 * (k2 & 1) + j], c, -mref));
              l_run += p;
              pf[k2][j] = (bf16)p;
            }
        }
      }
    };
    // group 1 starts one barrier later (its matrix phase i meets group 0's vector phase i) and group 0 passes
    // one more barrier at the end; group 1 waits for its tile loads at the end of each matrix phase
    if (grp == 1) __syncthreads();
    for (int i = 0; i < iters; ++i) {
      mphase(i);
      if (grp == 1) __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): K of block i + 1, V^T of block i landed
      __syncthreads();
      vphase(i);
      __syncthreads();
    }
    if (grp == 0) __syncthreads();
  }

  // each group finalises its own head
  const float l_row = halves_sum(l_run);
  float inv = 0.f, lse_v = -INFINITY;
  if (l_row > 0.f) {
    inv = 1.f / l_row;
    lse_v = (m_run * c + log2f(l_row)) * kLn2;
  }
  if (part != 0) {
    if (!active) return;
    const size_t ps = ((size_t)(2 * M.slot[item] + part - 1) * 2 + grp) * kBlk + wave * 32 + n;
    float* po = M.part_o + ps * D;
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = md * 32 + 8 * g4 + 4 * hh;
        *reinterpret_cast<f32x4*>(po + d0) = f32x4{o[md][g4 * 4] * inv, o[md][g4 * 4 + 1] * inv,
                                                   o[md][g4 * 4 + 2] * inv, o[md][g4 * 4 + 3] * inv};
      }
    if (hh == 0) M.part_lse[ps] = lse_v;
    return;
  }
  if (hh == 0 && active) P.lse[(int64_t)h * P.q_len + row0 + n] = lse_v;
  OutT* out = reinterpret_cast<OutT*>(P.out);
  if constexpr (sizeof(OutT) == 2) {
    // both heads' rows through LDS (the tile slots are free: every wave passed the loop's last barrier and
    // no tile load is outstanding), then all eight waves write whole 256-byte rows
    constexpr int kStgPitch = D * 2 + 16;
    static_assert(2 * 128 * kStgPitch <= 2 * (KTB + VTB), "staging fits the tile slots");
    __syncthreads();
    char* stg = smem + grp * 128 * kStgPitch;
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = md * 32 + 8 * g4 + 4 * hh;
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = (bf16)(o[md][g4 * 4 + e] * inv);
        *reinterpret_cast<u32x2*>(stg + (wave * 32 + n) * kStgPitch + d0 * 2) = __builtin_bit_cast(u32x2, pk);
      }
    __syncthreads();
    // 2 heads x 128 rows x 16 pieces of 16 bytes over 512 lanes: lanes 16 j .. 16 j + 15 write one row
    const int64_t rbase = (int64_t)qb * kBlk;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = j * 512 + (int)threadIdx.x;
      const int g = q >> 11, r = (q >> 4) & 127, ch = q & 15;
      if (g >= nh) continue;
      const u32x4 val = *reinterpret_cast<const u32x4*>(smem + (g * 128 + r) * kStgPitch + ch * 16);
      *reinterpret_cast<u32x4*>(out + (rbase + r) * ((int64_t)P.hq * D) + (int64_t)(h0 + g) * D + ch * 8) = val;
    }
  } else {
    if (!active) return;
    const int64_t obase = (row0 + n) * ((int64_t)P.hq * D) + (int64_t)h * D;
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = md * 32 + 8 * g4 + 4 * hh;
        *reinterpret_cast<f32x4*>(out + obase + d0) = f32x4{o[md][g4 * 4] * inv, o[md][g4 * 4 + 1] * inv,
                                                            o[md][g4 * 4 + 2] * inv, o[md][g4 * 4 + 3] * inv};
      }
  }
}

template <int D, typename OutT, bool VARLEN>
__global__ __launch_bounds__(512, 1) void bsa_pair_kernel(BsaMulti M) {
  __shared__ int s_item;
  const int n_items = M.n_items;
  if ((int)blockIdx.x >= n_items && (int)blockIdx.x >= n_items + M.ctl[2]) return;
  if (threadIdx.x == 0) s_item = take_entry(M);
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_item);
  if (e < 0) return;
  const int item = e >> 2, part = e & 3;
  int item0;
  if constexpr (VARLEN) {
    const BsaParams P = varlen_params<D, OutT>(M, item, item0);
    bsa_pair_body<D, OutT>(M, P, item, part, item - item0);
  } else {
    const BsaParams& P = find_seg(M, item, item0);
    bsa_pair_body<D, OutT>(M, P, item, part, item - item0);
  }
}

// ---------------------------------------------------------------------------
// Workspace preparation
// ---------------------------------------------------------------------------

// V [n][hkv][D] (token-major, strided) -> packed V^T: per plane [hkv][D][pitch]
// bf16 (hi plane, then the lo plane for fp32 input), tokens written at columns
// token_offset .. token_offset + round_up(n, 128), keys permuted by kSigma
// inside each group of 16, zero past n.  64x64 tiles through LDS for
// coalesced reads and writes.
template <typename T, bool SPLIT>
__global__ __launch_bounds__(256) void vt_kernel(const T* __restrict__ v, int64_t v_tok, int64_t v_head,
                                                 int64_t n_tok, int D, bf16* vt_hi, bf16* vt_lo,
                                                 int64_t pitch, int64_t token_offset) {
  __shared__ float tile[64][65];
  const int64_t k0 = (int64_t)blockIdx.x * 64;
  const int d0 = blockIdx.y * 64;
  const int kvh = blockIdx.z;
  const int tid = threadIdx.x;
  for (int c = tid; c < 64 * 8; c += 256) {
    const int kr = c / 8, dc = (c % 8) * 8;
    const int64_t key = k0 + kr;
    float vals[8];
    if (key < n_tok) {
      const T* src = v + key * v_tok + (int64_t)kvh * v_head + d0 + dc;
      if constexpr (sizeof(T) == 2) {
        const bf16x8 x = as_bf16x8(*reinterpret_cast<const u32x4*>(src));
#pragma unroll
        for (int j = 0; j < 8; ++j) vals[j] = (float)x[j];
      } else {
        const f32x4 a = reinterpret_cast<const f32x4*>(src)[0];
        const f32x4 b = reinterpret_cast<const f32x4*>(src)[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vals[j] = a[j];
          vals[4 + j] = b[j];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) vals[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[dc + j][kr] = vals[j];
  }
  __syncthreads();
  for (int c = tid; c < 64 * 8; c += 256) {
    const int dr = c / 8, pc = (c % 8) * 8;
    bf16x8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int pos = pc + j;
      const int key = (pos & ~15) | kSigma(pos & 15);
      const float x = tile[dr][key];
      if constexpr (SPLIT) {
        bf16 a, b;
        split_bf16(x, a, b);
        hi[j] = a;
        lo[j] = b;
      } else {
        hi[j] = (bf16)x;
      }
    }
    const int64_t off = ((int64_t)kvh * D + d0 + dr) * pitch + token_offset + k0 + pc;
    *reinterpret_cast<u32x4*>(vt_hi + off) = as_u32x4(hi);
    if constexpr (SPLIT) *reinterpret_cast<u32x4*>(vt_lo + off) = as_u32x4(lo);
  }
}

// fp32 [L][H][D] (strided) -> dense bf16 hi and lo planes [L][H][D].
__global__ __launch_bounds__(256) void split_kernel(const float* __restrict__ x, int64_t tok, int64_t head,
                                                    int64_t L, int H, int D, bf16* hi, bf16* lo) {
  const int64_t chunks = L * H * (D / 8);
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = c / (H * (D / 8));
    const int hd = (int)(c % (H * (D / 8)));
    const int hh = hd / (D / 8);
    const int d = (hd % (D / 8)) * 8;
    const float* src = x + t * tok + (int64_t)hh * head + d;
    const f32x4 a = reinterpret_cast<const f32x4*>(src)[0];
    const f32x4 b = reinterpret_cast<const f32x4*>(src)[1];
    bf16x8 h8, l8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = j < 4 ? a[j] : b[j - 4];
      bf16 p, q;
      split_bf16(v, p, q);
      h8[j] = p;
      l8[j] = q;
    }
    const int64_t off = c * 8;
    *reinterpret_cast<u32x4*>(hi + off) = as_u32x4(h8);
    *reinterpret_cast<u32x4*>(lo + off) = as_u32x4(l8);
  }
}

// ---------------------------------------------------------------------------
// Work order of a segmented launch.  The kept-tile count of a work item's row
// varies several-fold across heads and query blocks; taking items in dispatch
// order leaves long rows for the end of the grid, and a row longer than the
// mean load per workgroup slot bounds the whole launch by itself.  Two small
// kernels count each item's kept tiles, split every item longer than that mean
// into two halves at its median kept block, and sort the entries by
// descending count (counting sort in one workgroup); the attention workgroups
// take entries in that order as they start (greedy longest-processing-time
// list scheduling), and a last kernel merges the two halves of each split item
// by their LSE.  The order decides only which workgroup computes what.
constexpr int kPlanBins = 4096;  // counts >= kPlanBins-1 share the last bin
constexpr int kMinSplit = 20;    // items with fewer kept tiles are never split

template <int D, typename OutT, bool VARLEN>
__device__ __forceinline__ BsaParams item_span(const BsaMulti& M, int item, int& h, int& qb, int64_t& jb_end,
                                               int& nh) {
  int item0;
  BsaParams P;
  if constexpr (VARLEN) P = varlen_params<D, OutT>(M, item, item0);
  else P = find_seg(M, item, item0);
  nh = 1;
  if (M.pair) {
    int hp;
    bsa_decode(item - item0, (P.group + 1) / 2, P.hkv, P.n_qb, hp, qb);
    pair_heads(hp, P.group, h, nh);  // h: the item's first query head
  } else {
    bsa_decode(item - item0, P.group, P.hkv, P.n_qb, h, qb);
  }
  const int64_t nkb = (P.kv_len + kBlk - 1) / kBlk;
  jb_end = nkb;
  if (P.causal) {
    const int64_t lim = P.q_start + (int64_t)qb * kBlk + (kBlk - 1) - P.kv_start;
    jb_end = lim < 0 ? 0 : (lim / kBlk + 1 < nkb ? lim / kBlk + 1 : nkb);
  }
  return P;
}

// One wave per work item: kept key blocks below the causal limit, and the key
// block of its (count / 2)-th kept block (0-based), where a second half starts.
// A pair item counts the blocks either of its two heads kept.
template <bool VARLEN>
__global__ __launch_bounds__(256) void plan_count_kernel(BsaMulti M, int n_items, int* __restrict__ weights,
                                                         int* __restrict__ mid) {
  const int item = (int)blockIdx.x * 4 + wave_id();
  const int lane = lane_id();
  if (item >= n_items) return;
  int h, qb, nh;
  int64_t jb_end;
  const BsaParams P = item_span<128, bf16, VARLEN>(M, item, h, qb, jb_end, nh);
  int cnt;
  int64_t half_at;
  if (P.mask == nullptr) {
    cnt = (int)jb_end;
    half_at = jb_end / 2;
  } else {
    const uint8_t* mrow = P.mask + (int64_t)h * P.mask_hs + (int64_t)qb * P.mask_rs + (P.kv_start / kBlk - P.mask_off);
    const int64_t other = nh == 2 ? P.mask_hs : 0;  // the pair's second head (itself for one-head items)
    auto kept_at = [&](int64_t jb) { return (mrow[jb] | mrow[jb + other]) != 0; };
    cnt = 0;
    for (int64_t jb = lane; jb < jb_end; jb += 64) cnt += kept_at(jb);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    const int target = cnt / 2;
    half_at = jb_end;
    int run = 0;
    for (int64_t base = 0; base < jb_end; base += 64) {
      const int64_t jb = base + lane;
      const bool kept = jb < jb_end && kept_at(jb);
      const uint64_t bal = __ballot(kept);
      const int c = __popcll(bal);
      if (run + c > target) {
        const int before = __popcll(bal & ((1ull << lane) - 1));
        const uint64_t hit = __ballot(kept && run + before == target);
        half_at = base + __ffsll((unsigned long long)hit) - 1;
        break;
      }
      run += c;
    }
  }
  if (lane == 0) {
    weights[item] = cnt;
    mid[item] = (int)half_at;
  }
}

// Exclusive scan of kPlanBins bins from the highest bin down (1024 threads,
// four bins each); bins[b] becomes the number of entries in higher bins.
__device__ __forceinline__ void scan_bins_desc(int* bins, int* wsum) {
  const int t = (int)threadIdx.x;
  const int lane = lane_id();
  const int wave = t >> 6;
  int v[4], own = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = bins[kPlanBins - 1 - 4 * t - j];
    own += v[j];
  }
  int incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int run = incl - own;
  for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bins[kPlanBins - 1 - 4 * t - j] = run;
    run += v[j];
  }
  __syncthreads();
}

// One workgroup: choose the items to split (count above total / slots and at
// least kMinSplit, the longest of them while their whole count bin fits in
// max_split), assign their partial slots, write the entries longest first and
// reset the ticket.
__global__ __launch_bounds__(1024) void plan_sort_kernel(int n_items, const int* __restrict__ weights,
                                                         int* __restrict__ order, int* __restrict__ ctl,
                                                         int* __restrict__ slot, int* __restrict__ split_items,
                                                         int max_split, int slots) {
  __shared__ int cand[kPlanBins];   // split candidates per count bin
  __shared__ int above[kPlanBins];  // candidates in higher bins
  __shared__ int bins[kPlanBins];   // entries per bin, then their write positions
  __shared__ int wsum[16];
  __shared__ long long wtot[16];
  __shared__ int s_nsplit;
  const int t = (int)threadIdx.x;
  const int lane = lane_id();
  const int wave = t >> 6;
  long long tot = 0;
  for (int i = t; i < n_items; i += 1024) tot += weights[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
  if (lane == 0) wtot[wave] = tot;
  for (int b = t; b < kPlanBins; b += 1024) {
    cand[b] = 0;
    bins[b] = 0;
  }
  if (t == 0) s_nsplit = 0;
  __syncthreads();
  long long all = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) all += wtot[w];
  const long long thr = all / (slots > 0 ? slots : 1);
  // halves of fewer than 10 tiles cost more in per-item overhead and merging than they balance
  auto candidate = [&](int w) { return w >= kMinSplit && (long long)w > thr; };
  for (int i = t; i < n_items; i += 1024) {
    const int w = weights[i];
    if (candidate(w)) atomicAdd(&cand[min(w, kPlanBins - 1)], 1);
  }
  __syncthreads();
  for (int b = t; b < kPlanBins; b += 1024) above[b] = cand[b];
  __syncthreads();
  scan_bins_desc(above, wsum);
  auto split = [&](int w) {
    const int b = min(w, kPlanBins - 1);
    return candidate(w) && above[b] + cand[b] <= max_split;
  };
  for (int i = t; i < n_items; i += 1024) {
    const int w = weights[i];
    if (split(w)) {
      atomicAdd(&bins[min(w / 2, kPlanBins - 1)], 1);
      atomicAdd(&bins[min(w - w / 2, kPlanBins - 1)], 1);
    } else {
      atomicAdd(&bins[min(w, kPlanBins - 1)], 1);
    }
  }
  __syncthreads();
  scan_bins_desc(bins, wsum);
  for (int i = t; i < n_items; i += 1024) {
    const int w = weights[i];
    if (split(w)) {
      const int k = atomicAdd(&s_nsplit, 1);
      slot[i] = k;
      split_items[k] = i;
      order[atomicAdd(&bins[min(w / 2, kPlanBins - 1)], 1)] = i * 4 + 1;
      order[atomicAdd(&bins[min(w - w / 2, kPlanBins - 1)], 1)] = i * 4 + 2;
    } else {
      order[atomicAdd(&bins[min(w, kPlanBins - 1)], 1)] = i * 4;
    }
  }
  __syncthreads();
  if (t == 0) {
    ctl[0] = 0;
    ctl[1] = n_items + s_nsplit;
    ctl[2] = s_nsplit;
  }
}

// LSE merge of the two halves of split item k (partial slot k) into its
// segment's out and lse (both -inf: out 0, lse -inf).
template <int D, typename OutT, bool VARLEN>
__device__ void split_merge_one(const BsaMulti& M, int k, int e_head) {
  const int item = M.split_items[k];
  int h, qb, item_nh;
  int64_t jb_end;
  const BsaParams P = item_span<D, OutT, VARLEN>(M, item, h, qb, jb_end, item_nh);
  if (e_head >= item_nh) return;  // the second slot of a one-head pair item
  const int nh = M.pair ? 2 : 1;  // heads per slot; partial (slot k, half p, head e) at ((2 k + p) nh + e) rows
  h += e_head;
  const float* la = M.part_lse + ((size_t)(2 * k) * nh + e_head) * kBlk;
  const float* lb = la + (size_t)nh * kBlk;
  const float* oa = M.part_o + ((size_t)(2 * k) * nh + e_head) * kBlk * D;
  const float* ob = oa + (size_t)nh * kBlk * D;
  OutT* out = reinterpret_cast<OutT*>(P.out);
  for (int e = (int)threadIdx.x; e < kBlk * (D / 4); e += 256) {
    const int r = e / (D / 4);
    const int c = (e % (D / 4)) * 4;
    const float a = la[r], b = lb[r];
    const float m = fmaxf(a, b);
    float wa = 0.f, wb = 0.f, lse = -INFINITY;
    if (m != -INFINITY) {
      wa = expf(a - m);
      wb = expf(b - m);
      lse = m + logf(wa + wb);
      const float inv = 1.f / (wa + wb);
      wa *= inv;
      wb *= inv;
    }
    const f32x4 x = *reinterpret_cast<const f32x4*>(oa + (size_t)r * D + c);
    const f32x4 y = *reinterpret_cast<const f32x4*>(ob + (size_t)r * D + c);
    const int64_t row = (int64_t)qb * kBlk + r;
    OutT* dst = out + row * ((int64_t)P.hq * D) + (int64_t)h * D + c;
    if constexpr (sizeof(OutT) == 2) {
      bf16x4 pk;
#pragma unroll
      for (int j = 0; j < 4; ++j) pk[j] = (bf16)(x[j] * wa + y[j] * wb);
      *reinterpret_cast<u32x2*>(dst) = __builtin_bit_cast(u32x2, pk);
    } else {
      *reinterpret_cast<f32x4*>(dst) = f32x4{x[0] * wa + y[0] * wb, x[1] * wa + y[1] * wb, x[2] * wa + y[2] * wb,
                                            x[3] * wa + y[3] * wb};
    }
    if (c == 0) P.lse[(int64_t)h * P.q_len + row] = lse;
  }
}

// Split halves are merged by a grid of one workgroup per (slot, head) that may be in use (it strides if smaller).
template <int D, typename OutT, bool VARLEN>
__global__ __launch_bounds__(256) void split_merge_kernel(BsaMulti M) {
  const int nh = M.pair ? 2 : 1;
  for (int k = (int)blockIdx.x; k < M.ctl[2] * nh; k += (int)gridDim.x)
    split_merge_one<D, OutT, VARLEN>(M, k / nh, k % nh);
}

// One attention workgroup (eight waves, 132 KiB of LDS) per compute unit.
int bsa_workgroups_per_cu() { return 1; }

// Host tables reach device memory through the arguments of a small kernel, in stream order.
constexpr int kBlobWords = 384;
struct Blob {
  uint32_t w[kBlobWords];
};
__global__ __launch_bounds__(256) void upload_kernel(Blob b, int n_words, uint32_t* __restrict__ dst) {
  for (int i = (int)threadIdx.x; i < n_words; i += 256) dst[i] = b.w[i];
}

hipError_t upload_words(const void* src, size_t bytes, void* dst, hipStream_t s) {
  if (bytes % 4 != 0) return hipErrorInvalidValue;
  const size_t words = bytes / 4;
  for (size_t w0 = 0; w0 < words; w0 += kBlobWords) {
    const int n = (int)(words - w0 < (size_t)kBlobWords ? words - w0 : (size_t)kBlobWords);
    Blob b{};
    memcpy(b.w, static_cast<const uint32_t*>(src) + w0, (size_t)n * 4);
    hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(256), 0, s, b, n, static_cast<uint32_t*>(dst) + w0);
  }
  return hipGetLastError();
}

// Explicit instantiation helpers used by the ABI layer.
// bsa3_kernel addresses a lane's pieces of a K / V^T tile with 32-bit byte offsets.
static bool tile_offsets_fit(const BsaParams* segs, int n_seg, int D) {
  for (int i = 0; i < n_seg; ++i)
    if ((127 * segs[i].k_tok + D) * 2 >= ((int64_t)1 << 32) ||
        ((int64_t)(D - 1) * segs[i].vt_pitch + 128) * 2 >= ((int64_t)1 << 32))
      return false;
  return true;
}

// The pair form is used wherever it applies; XATTN_PAIR=0 in the environment keeps the single-head form (for
// comparisons), read once per process.
static bool pair_form_enabled() {
  static const bool on = [] {
    const char* e = getenv("XATTN_PAIR");
    return !(e && e[0] == '0');
  }();
  return on;
}

static thread_local hipEvent_t t_attn_events[2] = {nullptr, nullptr};
void set_attention_events(hipEvent_t before, hipEvent_t after) {
  t_attn_events[0] = before;
  t_attn_events[1] = after;
}
static hipError_t record_attention_event(int k, hipStream_t s) {
  return t_attn_events[k] ? hipEventRecord(t_attn_events[k], s) : hipSuccess;
}

template <int D, bool SPLIT, typename OutT>
hipError_t launch_bsa(const BsaParams* segs, int n_seg, const BsaPlan* plan, hipStream_t s) {
  if constexpr (!SPLIT && D == 128) {
    if (tile_offsets_fit(segs, n_seg, D)) {
      BsaMulti m{};
      // pair items (two query heads of one kv head per workgroup) when every segment has an even number of
      // query heads per kv head and a work order is available (with an odd group size every kv head would
      // leave a one-head item running at half the rate); the plan's arrays, sized for single-head items, hold
      // the half as many pair items with two heads per split slot
      bool pair = plan != nullptr && pair_form_enabled();
      for (int i = 0; i < n_seg; ++i) pair = pair && segs[i].group % 2 == 0;
      m.pair = pair ? 1 : 0;
      int total = 0;
      for (int i = 0; i < n_seg; ++i) {
        m.seg[i] = segs[i];
        total += (pair ? segs[i].hkv * ((segs[i].group + 1) / 2) : segs[i].hq) * segs[i].n_qb;
        m.wg_end[i] = total;
      }
      m.n_seg = n_seg;
      m.n_items = total;
      if (total > 0) {
        int grid = total;
        int max_split = 0;
        if (plan) {
          max_split = pair ? plan->max_split / 2 : plan->max_split;
          hipLaunchKernelGGL(plan_count_kernel<false>, dim3((total + 3) / 4), dim3(256), 0, s, m, total,
                             plan->weights, plan->mid);
          hipLaunchKernelGGL(plan_sort_kernel, dim3(1), dim3(1024), 0, s, total, (const int*)plan->weights,
                             plan->order, plan->ctl, plan->slot, plan->split_items, max_split, plan->slots);
          m.order = plan->order;
          m.ctl = plan->ctl;
          m.mid = plan->mid;
          m.slot = plan->slot;
          m.split_items = plan->split_items;
          m.part_o = plan->part_o;
          m.part_lse = plan->part_lse;
          m.direct = plan->slots;
          grid = total + max_split;  // entries: items plus halves of split items
        }
        hipError_t ev = record_attention_event(0, s);
        if (ev != hipSuccess) return ev;
        if (pair) hipLaunchKernelGGL((bsa_pair_kernel<D, OutT, false>), dim3(grid), dim3(512), 0, s, m);
        else hipLaunchKernelGGL((bsa3_kernel<D, OutT, false>), dim3(grid), dim3(512), 0, s, m);
        if ((ev = record_attention_event(1, s)) != hipSuccess) return ev;
        // one workgroup per (split slot, head) that may be in use; the ones past the split count exit
        if (max_split > 0)
          hipLaunchKernelGGL((split_merge_kernel<D, OutT, false>), dim3(max_split * (pair ? 2 : 1)), dim3(256), 0,
                             s, m);
      }
      return hipGetLastError();
    }
  }
  for (int i = 0; i < n_seg; ++i)
    hipLaunchKernelGGL((bsa_kernel<D, SPLIT, OutT>), dim3(segs[i].hq * segs[i].n_qb), dim3(kThreads), 0, s, segs[i]);
  return hipGetLastError();
}

template <typename OutT>
hipError_t launch_bsa_varlen(const BsaParams& shared, const VarlenSeq* seqs, int n_seqs, int n_items,
                             const BsaPlan* plan, hipStream_t s) {
  if (n_seqs <= 0 || !plan || !tile_offsets_fit(&shared, 1, 128)) return hipErrorInvalidValue;
  if (n_items == 0) return hipSuccess;
  BsaMulti m{};
  m.seg[0] = shared;
  m.n_seg = n_seqs;
  m.seqs = seqs;
  // head-pair items for an even number of query heads per kv head, as in the segmented form; n_items counts
  // (query head, query block) items, and the plan's arrays hold half as many pair items with two heads per
  // split slot
  const bool pair = pair_form_enabled() && shared.group % 2 == 0;
  m.pair = pair ? 1 : 0;
  const int items = pair ? n_items / 2 : n_items;
  const int max_split = pair ? plan->max_split / 2 : plan->max_split;
  m.n_items = items;
  hipLaunchKernelGGL(plan_count_kernel<true>, dim3((items + 3) / 4), dim3(256), 0, s, m, items, plan->weights,
                     plan->mid);
  hipLaunchKernelGGL(plan_sort_kernel, dim3(1), dim3(1024), 0, s, items, (const int*)plan->weights, plan->order,
                     plan->ctl, plan->slot, plan->split_items, max_split, plan->slots);
  m.order = plan->order;
  m.ctl = plan->ctl;
  m.mid = plan->mid;
  m.slot = plan->slot;
  m.split_items = plan->split_items;
  m.part_o = plan->part_o;
  m.part_lse = plan->part_lse;
  m.direct = plan->slots;
  hipError_t ev = record_attention_event(0, s);
  if (ev != hipSuccess) return ev;
  if (pair) hipLaunchKernelGGL((bsa_pair_kernel<128, OutT, true>), dim3(items + max_split), dim3(512), 0, s, m);
  else hipLaunchKernelGGL((bsa3_kernel<128, OutT, true>), dim3(items + max_split), dim3(512), 0, s, m);
  if ((ev = record_attention_event(1, s)) != hipSuccess) return ev;
  if (max_split > 0)
    hipLaunchKernelGGL((split_merge_kernel<128, OutT, true>), dim3(max_split * (pair ? 2 : 1)), dim3(256), 0, s, m);
  return hipGetLastError();
}
template hipError_t launch_bsa_varlen<bf16>(const BsaParams&, const VarlenSeq*, int, int, const BsaPlan*,
                                            hipStream_t);
template hipError_t launch_bsa_varlen<float>(const BsaParams&, const VarlenSeq*, int, int, const BsaPlan*,
                                             hipStream_t);

template hipError_t launch_bsa<64, false, bf16>(const BsaParams*, int, const BsaPlan*, hipStream_t);
template hipError_t launch_bsa<64, false, float>(const BsaParams*, int, const BsaPlan*, hipStream_t);
template hipError_t launch_bsa<64, true, bf16>(const BsaParams*, int, const BsaPlan*, hipStream_t);
template hipError_t launch_bsa<64, true, float>(const BsaParams*, int, const BsaPlan*, hipStream_t);
template hipError_t launch_bsa<128, false, bf16>(const BsaParams*, int, const BsaPlan*, hipStream_t);
template hipError_t launch_bsa<128, false, float>(const BsaParams*, int, const BsaPlan*, hipStream_t);
template hipError_t launch_bsa<128, true, bf16>(const BsaParams*, int, const BsaPlan*, hipStream_t);
template hipError_t launch_bsa<128, true, float>(const BsaParams*, int, const BsaPlan*, hipStream_t);

hipError_t launch_vt(const void* v, xa_dtype_t dt, int64_t v_tok, int64_t v_head, int64_t n_tok, int hkv,
                     int D, bf16* vt_hi, bf16* vt_lo, int64_t pitch, int64_t token_offset, hipStream_t s) {
  const int64_t ext = (n_tok + 127) / 128 * 128;
  dim3 grid((unsigned)(ext / 64), (unsigned)(D / 64), (unsigned)hkv);
  if (dt == XA_BF16)
    hipLaunchKernelGGL((vt_kernel<bf16, false>), grid, dim3(256), 0, s, (const bf16*)v, v_tok, v_head, n_tok,
                       D, vt_hi, vt_lo, pitch, token_offset);
  else
    hipLaunchKernelGGL((vt_kernel<float, true>), grid, dim3(256), 0, s, (const float*)v, v_tok, v_head, n_tok,
                       D, vt_hi, vt_lo, pitch, token_offset);
  return hipGetLastError();
}

hipError_t launch_split(const float* x, int64_t tok, int64_t head, int64_t L, int H, int D, bf16* hi, bf16* lo,
                        hipStream_t s) {
  const int64_t chunks = L * H * (D / 8);
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(split_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, tok, head, L, H, D, hi, lo);
  return hipGetLastError();
}

}  // namespace xa
