// XAttention importance estimate and block selection (part 1 of the path).
//
// XAttention algorithm guide (nano-vllm docs): "Stride Reshape 详解 / Inverse
// 模式" (row r of the reshaped Q is Q[r*S+S-1-t] concatenated over t, column c
// of the reshaped K is K[c*S+t] over t), "Triton Kernels 详解"
// (flat_group_gemm_fuse_reshape computes the product without materialising the
// reshaped tensors; softmax_fuse_block_sum normalises each row and sums
// block_size/stride x block_size/stride tiles), "块选择算法" (cumulative
// threshold with sink and diagonal kept).  Chunk placement and the
// 1/(S*sqrt(d)) scale follow XAttentionBSAPolicy.select_blocks.
//
// Two kernels instead of the pages' recompute-twice passes:
//   est_gemm_kernel   -- reshaped Q K^T on MFMA (the reshape is pure
//                        addressing: stage t of the contraction stages the
//                        query tokens r*S+S-1-t and key tokens c*S+t), then
//                        per (row, key block) the log-sum-exp of the visible
//                        scores, written once ([Hq][nKB][R], fp32, log2 units);
//                        est_gemm2_kernel is the bf16, d = 128 form: 256 x 256
//                        tiles, one resident workgroup per CU walking every
//                        grid-th tile, the next tile's first slice loaded
//                        while the current tile's scores are reduced;
//   est_select_kernel -- per (head, query block): row normaliser = log-sum-exp
//                        over key blocks, block score = sum over the block's
//                        rows of exp2(lse_part - row lse), then the threshold
//                        selection (bitonic sort in LDS + prefix sums).
// The block scores therefore need one GEMM pass, not two.
#include "launchers.h"

namespace xa {


constexpr int kEThreads = 256;

template <int D, bool SPLIT, int HALF>
__global__ __launch_bounds__(kEThreads) void est_gemm_kernel(EstParams P) {
  constexpr int TP = D + 8;          // LDS tile pitch (elements)
  constexpr int TILE = 128 * TP;
  constexpr int NKK = D / 16;
  constexpr int CH = 128 * (D / 8) / kEThreads;  // 16-B chunks per thread per tile
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * TILE];
  bf16* qs = smem;
  bf16* ks = smem + TILE;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = lane_id();
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int wr = wave & 1;   // 64-row half of the tile
  const int wc = wave >> 1;  // 64-column half of the tile

  // work order: (kv head, column tile, row tile, head-in-group), last fastest
  const int total = P.hkv * P.n_ct * P.n_rt * P.group;
  int w = xcd_remap(blockIdx.x, total);
  const int j = w % P.group;
  w /= P.group;
  const int rt = w % P.n_rt;
  w /= P.n_rt;
  const int ct = w % P.n_ct;
  const int kvh = w / P.n_ct;
  const int h = kvh * P.group + j;

  const int64_t cdiag = P.q_start / P.S - P.c0;  // local column c visible to row r iff c <= cdiag + r
  const int r_hi = min(P.R - 1, rt * 128 + 127);
  if ((int64_t)ct * 128 > cdiag + r_hi) return;  // tile entirely right of the causal limit

  const int w_r0 = rt * 128 + wr * 64;
  const int w_c0 = ct * 128 + wc * 64;
  const bool wave_live = w_r0 < P.R && w_c0 < P.N && (int64_t)w_c0 <= cdiag + min(P.R - 1, w_r0 + 63);

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[a][c] = f32x16{};

  const int combos = SPLIT ? 3 : 1;
  for (int t = 0; t < P.S; ++t) {
    for (int cb = 0; cb < combos; ++cb) {
      const bf16* qsrc = (cb == 2) ? P.q_lo : P.q_hi;
      const bf16* ksrc = (cb == 1) ? P.k_lo : P.k_hi;
      u32x4 rq[CH], rk[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = tid + kEThreads * i;
        const int r = c / (D / 8);
        const int c8 = c % (D / 8);
        const int64_t qr = (int64_t)rt * 128 + r;
        const int64_t qtok = qr * P.S + (P.S - 1 - t);
        rq[i] = qr < P.R ? *reinterpret_cast<const u32x4*>(qsrc + qtok * P.q_tok + (int64_t)h * P.q_head + c8 * 8)
                         : u32x4{0, 0, 0, 0};
        const int64_t kc = (int64_t)ct * 128 + r;
        const int64_t ktok = kc * P.S + t;
        rk[i] = kc < P.N ? *reinterpret_cast<const u32x4*>(ksrc + ktok * P.k_tok + (int64_t)kvh * P.k_head + c8 * 8)
                         : u32x4{0, 0, 0, 0};
      }
      __syncthreads();  // previous stage's reads are done
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = tid + kEThreads * i;
        const int r = c / (D / 8);
        const int c8 = c % (D / 8);
        *reinterpret_cast<u32x4*>(qs + r * TP + c8 * 8) = rq[i];
        *reinterpret_cast<u32x4*>(ks + r * TP + c8 * 8) = rk[i];
      }
      __syncthreads();
      if (wave_live) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          bf16x8 af[2], bfr[2];
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            af[mt] = as_bf16x8(*reinterpret_cast<const u32x4*>(ks + (wc * 64 + mt * 32 + n) * TP + kk * 16 + 8 * hh));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            bfr[nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(qs + (wr * 64 + nt * 32 + n) * TP + kk * 16 + 8 * hh));
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma32(af[mt], bfr[nt], acc[mt][nt]);
        }
      }
    }
  }
  if (!wave_live) return;

  // Epilogue: per (row, key block) log2-sum-exp2 of the visible scores.
  // Lane values v = 16*mt + i sit at column 32*mt + 8*(i/4) + 4*hh + i%4 of the
  // wave's 64 columns, so a key block (b columns) is a run of b/2 values per
  // lane, the other half held by lane ^ 32.
  static_assert(HALF == 4 || HALF == 8 || HALF == 16 || HALF == 32, "key block = 2*HALF reshaped columns");
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = w_r0 + nt * 32 + n;
    float x[32];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t c = (int64_t)w_c0 + mt * 32 + 8 * (i / 4) + 4 * hh + (i % 4);
        const bool ok = c < P.N && c <= cdiag + r;
        x[mt * 16 + i] = ok ? acc[mt][nt][i] * P.scale_log2 : -INFINITY;
      }
#pragma unroll
    for (int g0 = 0; g0 < 32; g0 += HALF) {
      float mx = -INFINITY;
#pragma unroll
      for (int v = g0; v < g0 + HALF; ++v) mx = fmaxf(mx, x[v]);
      mx = halves_max(mx);
      float s = 0.f;
      const float ref = mx == -INFINITY ? 0.f : mx;
#pragma unroll
      for (int v = g0; v < g0 + HALF; ++v) s += fast_exp2(x[v] - ref);
      s = halves_sum(s);
      const int kb = w_c0 / (2 * HALF) + g0 / HALF;
      if (hh == 0 && r < P.R && kb < P.nkb)
        P.lse_part[((int64_t)h * P.nkb_ld + P.kb0 + kb) * P.R + r] = mx == -INFINITY ? -INFINITY : mx + log2f(s);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16, head_dim 128: 256x256 output tile per 16-wave workgroup (4x4 waves of
// 64x64), so every 16-byte fragment read from LDS feeds two MFMAs and each
// byte fetched from L2 feeds twice the MFMA work of a 128x128 tile.  The
// contraction is walked in slices of 64 head-dim columns of one stride step t
// (query tokens r*S+S-1-t, key tokens c*S+t); slices go global -> LDS with
// global_load_lds_dwordx4 into two alternating 64 KiB buffers (128-byte rows,
// 16-byte chunk s of row r stored at slot s ^ ((r >> 1) & 7)), one barrier per
// slice.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void est_g2lds16(const void* g, char* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Sequence of packed-batch workgroup w (binary search of the prefix ends, uniform per workgroup); w
// becomes the workgroup's index inside its sequence.  Record fields go through readfirstlane so they
// stay in scalar registers.
template <bool SEL>
__device__ __forceinline__ const VarlenSeq& varlen_seq(const VarlenSeq* seqs, int n, int& w, int& q0, int& ql,
                                                       int& k0, int& kl) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int md = (lo + hi) >> 1;
    const int end = __builtin_amdgcn_readfirstlane(SEL ? seqs[md].sel_end : seqs[md].est_end);
    if (w < end) hi = md;
    else lo = md + 1;
  }
  if (lo) w -= __builtin_amdgcn_readfirstlane(SEL ? seqs[lo - 1].sel_end : seqs[lo - 1].est_end);
  const VarlenSeq& v = seqs[lo];
  q0 = __builtin_amdgcn_readfirstlane(v.q0);
  ql = __builtin_amdgcn_readfirstlane(v.q_len);
  k0 = __builtin_amdgcn_readfirstlane(v.k0);
  kl = __builtin_amdgcn_readfirstlane(v.k_len);
  return v;
}

// The workgroup computes the tiles v = v0, v0 + vstep, ... below vend (mapped through the XCD grouping when
// remap; the packed batch passes one tile), one after another: the next live tile's first slice is issued into
// the free buffer at the top of the current tile's last slice, so it lands during that slice and the epilogue.
template <int HALF>
__device__ __forceinline__ void est_gemm2_body(const EstParams& P, int v0, int vstep, int vend, bool remap) {
  constexpr int TILE = 256;
  constexpr int SLICE_B = TILE * 128;      // one operand slice: 256 rows x 64 bf16
  constexpr int BUF_B = 2 * SLICE_B;       // Q slice + K slice
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUF_B];

  const int wave = wave_id();
  const int lane = lane_id();
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int wr = wave & 3;
  const int wc = wave >> 2;

  const int n_rt = (P.R + TILE - 1) / TILE;
  const int n_ct = (P.N + TILE - 1) / TILE;
  const int64_t cdiag = P.q_start / P.S - P.c0;

  struct Tile { int rt, ct, h, kvh; };
  // first tile at or after v with unmasked work (uniform); false when none is left
  auto next_live = [&](int& v, Tile& t) -> bool {
    for (; v < vend; v += vstep) {
      int w = remap ? xcd_remap(v, vend) : v;
      const int j = w % P.group;
      w /= P.group;
      t.rt = w % n_rt;
      w /= n_rt;
      t.ct = w % n_ct;
      t.kvh = w / n_ct;
      t.h = t.kvh * P.group + j;
      const int r_hi = min(P.R - 1, t.rt * TILE + TILE - 1);
      if ((int64_t)t.ct * TILE <= cdiag + r_hi) return true;
    }
    return false;
  };

  // this lane's two load chunks per operand per slice (instructions 2*wave, 2*wave+1)
  auto issue = [&](const Tile& T, int slice, int buf) {
    const bf16* qb = P.q_hi + (int64_t)T.h * P.q_head;
    const bf16* kb = P.k_hi + (int64_t)T.kvh * P.k_head;
    const int t = slice >> 1;
    const int dof = (slice & 1) * 64;
    char* dq = smem + buf * BUF_B;
    char* dk = dq + SLICE_B;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int inst = wave * 2 + i;
      const int lin = inst * 64 + lane;
      const int r = lin >> 3;
      const int ch = (lin & 7) ^ ((r >> 1) & 7);
      int qr = T.rt * TILE + r;
      qr = qr < P.R ? qr : P.R - 1;
      int kc = T.ct * TILE + r;
      kc = kc < P.N ? kc : P.N - 1;
      const int64_t qtok = (int64_t)qr * P.S + (P.S - 1 - t);
      const int64_t ktok = (int64_t)kc * P.S + t;
      est_g2lds16(qb + qtok * P.q_tok + dof + ch * 8, dq + inst * 1024);
      est_g2lds16(kb + ktok * P.k_tok + dof + ch * 8, dk + inst * 1024);
    }
  };
  auto frag = [&](const char* base, int r, int ch) {
    return *reinterpret_cast<const bf16x8*>(base + r * 128 + ((ch ^ ((r >> 1) & 7)) << 4));
  };

  const int n_slices = 2 * P.S;  // even: the last slice reads buffer 1, buffer 0 is free during it
  int v = v0;
  Tile cur;
  if (!next_live(v, cur)) return;
  issue(cur, 0, 0);
  while (true) {
    int vn = v + vstep;
    Tile nxt;
    const bool more = next_live(vn, nxt);

    const int w_r0 = cur.rt * TILE + wr * 64;
    const int w_c0 = cur.ct * TILE + wc * 64;
    const bool wave_live = w_r0 < P.R && w_c0 < P.N && (int64_t)w_c0 <= cdiag + min(P.R - 1, w_r0 + 63);

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[a][c] = f32x16{};

    for (int sl = 0; sl < n_slices; ++sl) {
      __builtin_amdgcn_s_waitcnt(0x3f70);  // this wave's loads of slice sl have landed
      __syncthreads();                     // ... and every wave's; the other buffer is free
      if (sl + 1 < n_slices) issue(cur, sl + 1, (sl + 1) & 1);
      else if (more) issue(nxt, 0, 0);
      if (wave_live) {
        const char* qs = smem + (sl & 1) * BUF_B;
        const char* ks = qs + SLICE_B;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          bf16x8 af[2], bfr[2];
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) af[mt] = frag(ks, wc * 64 + mt * 32 + n, 2 * kk + hh);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) bfr[nt] = frag(qs, wr * 64 + nt * 32 + n, 2 * kk + hh);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma32(af[mt], bfr[nt], acc[mt][nt]);
        }
      }
    }

    if (wave_live) {
      // every column of the wave valid for every row of it: no per-element mask
      const bool full = w_c0 + 63 < P.N && (int64_t)w_c0 + 63 <= cdiag + w_r0;
      const float sc = P.scale_log2;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int r = w_r0 + nt * 32 + n;
        float x[32];  // raw scores (the scale is positive, so the maximum is taken before scaling)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) x[mt * 16 + i] = acc[mt][nt][i];
        if (!full) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int64_t c = (int64_t)w_c0 + mt * 32 + 8 * (i / 4) + 4 * hh + (i % 4);
              if (!(c < P.N && c <= cdiag + r)) x[mt * 16 + i] = -INFINITY;
            }
        }
#pragma unroll
        for (int g0 = 0; g0 < 32; g0 += HALF) {
          float mx = -INFINITY;
#pragma unroll
          for (int q = g0; q < g0 + HALF; ++q) mx = fmaxf(mx, x[q]);
          mx = halves_max(mx);
          const float ref = mx == -INFINITY ? 0.f : mx * sc;
          float s = 0.f;
#pragma unroll
          for (int q = g0; q < g0 + HALF; ++q) s += fast_exp2(__builtin_fmaf(x[q], sc, -ref));
          s = halves_sum(s);
          const int kbk = w_c0 / (2 * HALF) + g0 / HALF;
          if (hh == 0 && r < P.R && kbk < P.nkb)
            P.lse_part[((int64_t)cur.h * P.nkb_ld + P.kb0 + kbk) * P.R + r] =
                mx == -INFINITY ? -INFINITY : ref + log2f(s);
        }
      }
    }
    if (!more) break;
    cur = nxt;
    v = vn;
  }
}

template <int HALF, bool VARLEN>
__global__ __launch_bounds__(1024) void est_gemm2_kernel(EstParams P0) {
  if constexpr (VARLEN) {
    int w = xcd_remap(blockIdx.x, P0.grid_total);
    int q0, ql, k0, kl;
    const VarlenSeq& v = varlen_seq<false>(P0.seqs, P0.n_seqs, w, q0, ql, k0, kl);
    EstParams P = P0;
    P.q_hi += (int64_t)q0 * P.q_tok;
    P.k_hi += (int64_t)k0 * P.k_tok;
    P.q_len = ql;
    P.k_len = kl;
    P.q_start = kl - ql;
    P.R = ql / P.S;
    P.N = kl / P.S;
    P.nkb = kl / 128;
    P.nkb_ld = P.nkb;
    P.lse_part += rfl64(v.lse_off);
    est_gemm2_body<HALF>(P, w, 1, w + 1, false);
  } else {
    const int n_rt = (P0.R + 255) / 256, n_ct = (P0.N + 255) / 256;
    est_gemm2_body<HALF>(P0, blockIdx.x, gridDim.x, P0.hkv * n_ct * n_rt * P0.group, true);
  }
}

// ---------------------------------------------------------------------------
// Block sums + cumulative-threshold selection, one workgroup per
// (head, query block).
// ---------------------------------------------------------------------------


// B = rows of a query block in the reshaped score matrix (block / stride); the
// per-row loads are unrolled so that each thread's loads are in flight together.
template <int B>
__device__ __forceinline__ void est_select_body(const SelParams& P, int w) {
  // dynamic LDS: npow_cap sort keys, then nkb mask bytes
  extern __shared__ __attribute__((aligned(16))) unsigned long long sel_dyn[];
  unsigned long long* keys = sel_dyn;
  uint8_t* mrow = reinterpret_cast<uint8_t*>(sel_dyn + P.npow_cap);
  __shared__ float row_lse[64];
  __shared__ float red_m[256];
  __shared__ float red_s[256];
  __shared__ double part[256];
  __shared__ double s_total;
  __shared__ float s_a0, s_ad;

  const int tid = threadIdx.x;
  const int h = w / P.n_qb;
  const int qb = w % P.n_qb;
  constexpr int b = B;
  // always-kept diagonal block; key blocks 0..diag visible (history only: all, no diagonal)
  const int64_t diag = P.hist_only ? -1 : P.cur + qb;
  const int nvis = P.hist_only ? P.nkb : (int)diag + 1;
  const float* base = P.lse_part + (int64_t)h * P.nkb * P.R + (int64_t)qb * b;

  // pass 1: per-row normaliser over key blocks (log2 units)
  {
    constexpr int nstripe = 256 / b;
    constexpr int U = 8;  // loads in flight per thread
    const int r = tid % b;
    const int stripe = tid / b;
    float m = -INFINITY, s = 0.f;
    for (int kb0 = stripe; kb0 < nvis; kb0 += nstripe * U) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kb = kb0 + u * nstripe;
        v[u] = kb < nvis ? base[(int64_t)kb * P.R + r] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (v[u] == -INFINITY) continue;
        if (v[u] > m) {
          s = s * fast_exp2(m - v[u]) + 1.f;
          m = v[u];
        } else {
          s += fast_exp2(v[u] - m);
        }
      }
    }
    red_m[tid] = m;
    red_s[tid] = s;
    __syncthreads();
    if (tid < b) {
      float M = -INFINITY;
      for (int k = 0; k < nstripe; ++k) M = fmaxf(M, red_m[k * b + tid]);
      float S = 0.f;
      for (int k = 0; k < nstripe; ++k) {
        const float mk = red_m[k * b + tid];
        if (mk != -INFINITY) S += red_s[k * b + tid] * fast_exp2(mk - M);
      }
      row_lse[tid] = M + log2f(S);
    }
    __syncthreads();
  }

  // pass 2: block scores, sort keys, row total
  const bool all = P.threshold >= 1.0f;
  int npow = 1;
  while (npow < nvis) npow <<= 1;
  double tsum = 0.0;
  for (int kb = tid; kb < P.nkb; kb += 256) {
    float a = 0.f;
    if (kb < nvis) {
      const float* col = base + (int64_t)kb * P.R;
#pragma unroll
      for (int r0 = 0; r0 < b; r0 += 16) {
        float v[16];
#pragma unroll
        for (int r = 0; r < 16 && r0 + r < b; ++r) v[r] = col[r0 + r];
#pragma unroll
        for (int r = 0; r < 16 && r0 + r < b; ++r)
          if (v[r] != -INFINITY) a += fast_exp2(v[r] - row_lse[r0 + r]);
      }
      tsum += a;
    }
    P.scores[((int64_t)h * P.n_qb + qb) * P.nkb + kb] = a;
    const bool forced = kb == 0 || kb == diag;
    mrow[kb] = (kb < nvis && (all || forced)) ? 1 : 0;
    if (kb < npow) {
      const unsigned bits = __float_as_uint(a);
      keys[kb] = (kb < nvis && !forced) ? (((unsigned long long)(0xffffffffu - bits) << 32) | (unsigned)kb)
                                         : ~0ull;
    }
    if (kb == 0) s_a0 = a;
    if (kb == diag) s_ad = a;
  }
  for (int kb = P.nkb + tid; kb < npow; kb += 256) keys[kb] = ~0ull;
  {
    double t = tsum;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
    if ((tid & 63) == 0) part[tid >> 6] = t;
    __syncthreads();
    if (tid == 0) s_total = part[0] + part[1] + part[2] + part[3];
    __syncthreads();
  }

  const int n_forced = diag > 0 ? 2 : 1;  // block 0, and the diagonal when it is another block
  const int n_other = nvis - n_forced > 0 ? nvis - n_forced : 0;  // sortable blocks
  if (!all && n_other > 0) {
    // bitonic sort, ascending key = descending score, then ascending index
    for (int k = 2; k <= npow; k <<= 1) {
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        for (int i = tid; i < npow; i += 256) {
          const int ixj = i ^ jj;
          if (ixj > i) {
            const unsigned long long x = keys[i], y = keys[ixj];
            const bool up = (i & k) == 0;
            if ((x > y) == up) {
              keys[i] = y;
              keys[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    // prefix mass over the sorted order: contiguous segments per thread
    const int seg = (n_other + 255) / 256;
    const int p0 = tid * seg;
    const int p1 = min(n_other, p0 + seg);
    double loc = 0.0;
    for (int p = p0; p < p1; ++p) loc += (double)__uint_as_float(0xffffffffu - (unsigned)(keys[p] >> 32));
    // exclusive scan of the 256 segment sums: inclusive scan inside each wave, then wave offsets
    const int lane = tid & 63;
    double incl = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double up = __shfl_up(incl, o);
      if (lane >= o) incl += up;
    }
    if (lane == 63) part[tid >> 6] = incl;
    __syncthreads();
    double wave_off = 0.0;
    for (int w = 0; w < (tid >> 6); ++w) wave_off += part[w];
    const double forced_mass = (double)s_a0 + (diag > 0 ? (double)s_ad : 0.0);
    const double need = (double)P.threshold * s_total;
    double run = forced_mass + wave_off + (incl - loc);
    for (int p = p0; p < p1; ++p) {
      const unsigned long long key = keys[p];
      if (run < need) mrow[(unsigned)(key & 0xffffffffu)] = 1;
      run += (double)__uint_as_float(0xffffffffu - (unsigned)(key >> 32));
    }
    __syncthreads();
  } else {
    __syncthreads();
  }
  uint8_t* out = P.mask + ((int64_t)h * P.n_qb + qb) * P.nkb;
  for (int kb = tid; kb < P.nkb; kb += 256) out[kb] = mrow[kb];
}

template <int B, bool VARLEN>
__global__ __launch_bounds__(256) void est_select_kernel(SelParams P0) {
  // each XCD a contiguous range of (head, query block): neighbouring query blocks read the two halves of the
  // same 128-byte lines of the per-block log-sum-exp rows
  int w = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  if constexpr (VARLEN) {
    int q0, ql, k0, kl;
    const VarlenSeq& v = varlen_seq<true>(P0.seqs, P0.n_seqs, w, q0, ql, k0, kl);
    SelParams P = P0;
    P.lse_part += rfl64(v.lse_off);
    const int64_t oo = rfl64(v.out_off);
    P.scores += oo;
    P.mask += oo;
    P.R = ql / (128 / B);
    P.nkb = kl / 128;
    P.n_qb = ql / 128;
    P.cur = (kl - ql) / 128;
    int np = 1;
    while (np < P.nkb) np <<= 1;
    P.npow_cap = np;
    est_select_body<B>(P, w);
  } else {
    est_select_body<B>(P0, w);
  }
}

template <int D, bool SPLIT>
hipError_t launch_est_gemm(const EstParams& p, hipStream_t s) {
  if constexpr (D == 128 && !SPLIT) {
    const int n_rt = (p.R + 255) / 256, n_ct = (p.N + 255) / 256;
    // one resident workgroup per CU (128 KiB of LDS each) walks every grid-th tile
    const int grid = min(p.hkv * n_ct * n_rt * p.group, device_cus());
    switch (p.b) {
      case 8: hipLaunchKernelGGL((est_gemm2_kernel<4, false>), dim3(grid), dim3(1024), 0, s, p); break;
      case 16: hipLaunchKernelGGL((est_gemm2_kernel<8, false>), dim3(grid), dim3(1024), 0, s, p); break;
      case 32: hipLaunchKernelGGL((est_gemm2_kernel<16, false>), dim3(grid), dim3(1024), 0, s, p); break;
      case 64: hipLaunchKernelGGL((est_gemm2_kernel<32, false>), dim3(grid), dim3(1024), 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int grid = p.hkv * p.n_ct * p.n_rt * p.group;
  switch (p.b) {
    case 8: hipLaunchKernelGGL((est_gemm_kernel<D, SPLIT, 4>), dim3(grid), dim3(kEThreads), 0, s, p); break;
    case 16: hipLaunchKernelGGL((est_gemm_kernel<D, SPLIT, 8>), dim3(grid), dim3(kEThreads), 0, s, p); break;
    case 32: hipLaunchKernelGGL((est_gemm_kernel<D, SPLIT, 16>), dim3(grid), dim3(kEThreads), 0, s, p); break;
    case 64: hipLaunchKernelGGL((est_gemm_kernel<D, SPLIT, 32>), dim3(grid), dim3(kEThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template hipError_t launch_est_gemm<64, false>(const EstParams&, hipStream_t);
template hipError_t launch_est_gemm<64, true>(const EstParams&, hipStream_t);
template hipError_t launch_est_gemm<128, false>(const EstParams&, hipStream_t);
template hipError_t launch_est_gemm<128, true>(const EstParams&, hipStream_t);

// K[::stride] of n_out * stride key rows -> dense rows out_off .. out_off + n_out - 1
// of a [capacity][hkv][d] buffer; one 16-byte piece per thread.
template <typename T>
__global__ __launch_bounds__(256) void downsample_keys_kernel(const T* __restrict__ k, int64_t k_tok, int64_t k_head,
                                                              int64_t n_out, int hkv, int d, int stride,
                                                              T* __restrict__ out, int64_t out_off) {
  constexpr int E = 16 / sizeof(T);  // elements per piece
  const int pieces = d / E;
  const int64_t total = n_out * hkv * pieces;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % pieces);
    const int h = (int)((i / pieces) % hkv);
    const int64_t j = i / ((int64_t)pieces * hkv);
    const u32x4 v = *reinterpret_cast<const u32x4*>(k + j * stride * k_tok + (int64_t)h * k_head + c * E);
    *reinterpret_cast<u32x4*>(out + ((out_off + j) * hkv + h) * d + c * E) = v;
  }
}

hipError_t launch_downsample_keys(const void* k, xa_dtype_t dt, int64_t k_tok, int64_t k_head, int64_t n_out, int hkv,
                                  int d, int stride, void* out, int64_t out_off, hipStream_t s) {
  const int64_t pieces = n_out * hkv * (d * (dt == XA_BF16 ? 2 : 4) / 16);
  int64_t blocks = (pieces + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (dt == XA_BF16)
    hipLaunchKernelGGL(downsample_keys_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, s, (const bf16*)k, k_tok,
                       k_head, n_out, hkv, d, stride, (bf16*)out, out_off);
  else
    hipLaunchKernelGGL(downsample_keys_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, (const float*)k,
                       k_tok, k_head, n_out, hkv, d, stride, (float*)out, out_off);
  return hipGetLastError();
}

template <bool VARLEN>
static hipError_t select_launch(const SelParams& p, int grid, hipStream_t s) {
  const size_t lds = (size_t)p.npow_cap * 8 + ((size_t)p.nkb + 15) / 16 * 16;
  auto go = [&](auto kern) {
    if (lds > 65536) (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, s, p);
  };
  switch (p.b) {
    case 8: go(est_select_kernel<8, VARLEN>); break;
    case 16: go(est_select_kernel<16, VARLEN>); break;
    case 32: go(est_select_kernel<32, VARLEN>); break;
    case 64: go(est_select_kernel<64, VARLEN>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_est_select(const SelParams& p, hipStream_t s) { return select_launch<false>(p, p.hq * p.n_qb, s); }

hipError_t launch_est_select_varlen(const SelParams& p0, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  return select_launch<true>(p0, grid, s);
}

hipError_t launch_est_gemm_varlen(const EstParams& p0, hipStream_t s) {
  if (p0.grid_total <= 0) return hipSuccess;
  const dim3 grid(p0.grid_total);
  switch (p0.b) {
    case 8: hipLaunchKernelGGL((est_gemm2_kernel<4, true>), grid, dim3(1024), 0, s, p0); break;
    case 16: hipLaunchKernelGGL((est_gemm2_kernel<8, true>), grid, dim3(1024), 0, s, p0); break;
    case 32: hipLaunchKernelGGL((est_gemm2_kernel<16, true>), grid, dim3(1024), 0, s, p0); break;
    case 64: hipLaunchKernelGGL((est_gemm2_kernel<32, true>), grid, dim3(1024), 0, s, p0); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace xa
