// 128-token block mask -> cache blocks (the reducer feeding block loads).
//
// Task plan page, "select_blocks 设计" step 3: a 1024-token cache block is
// kept if any of its eight 128-token blocks is selected.
// XAttentionBSAPolicy.select_blocks step 6: union over heads and query blocks,
// then the first and last history block are always included.
#include "common.h"

namespace xa {

// One workgroup per cache block, each XCD a contiguous range of them (neighbouring cache blocks read and
// write bytes of the same cache lines).  Threads stride over the (head, query block) rows; each reads its
// row's sub_blocks mask bytes (one 8-byte load where they are 8 and aligned), writes the per-head byte and
// votes into the union.
__global__ __launch_bounds__(256) void cache_block_kernel(
    const uint8_t* __restrict__ mask, int heads, int n_qb, int64_t n_cols, int64_t hs, int64_t rs,
    int64_t kb_begin, int64_t n_cb, int sub, int force_first_last, uint8_t* keep_per_head,
    uint8_t* keep_any, uint8_t* keep_any_blocks) {
  const int64_t cb = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int64_t c0 = kb_begin + cb * sub;
  int64_t c1 = c0 + sub;
  if (c1 > n_cols) c1 = n_cols;
  const bool vec8 = c1 - c0 == 8 && ((reinterpret_cast<uintptr_t>(mask) | (uint64_t)hs | (uint64_t)rs |
                                      (uint64_t)c0) & 7) == 0;
  const int rows = heads * n_qb;
  int any = 0;
  for (int r = threadIdx.x; r < rows; r += blockDim.x) {
    const int h = r / n_qb, qb = r % n_qb;
    const uint8_t* row = mask + h * hs + qb * rs;
    int hit = 0;
    if (vec8) {
      hit = *reinterpret_cast<const uint64_t*>(row + c0) != 0;
    } else {
      for (int64_t c = c0; c < c1; ++c) hit |= row[c];
    }
    hit = hit ? 1 : 0;
    if (keep_per_head) keep_per_head[((int64_t)h * n_qb + qb) * n_cb + cb] = (uint8_t)hit;
    any |= hit;
  }
  any = __syncthreads_or(any);
  if (force_first_last && (cb == 0 || cb == n_cb - 1)) any = 1;
  if (threadIdx.x == 0 && keep_any) keep_any[cb] = (uint8_t)any;
  if (keep_any_blocks)
    for (int s = threadIdx.x; s < sub; s += blockDim.x) keep_any_blocks[cb * sub + s] = (uint8_t)any;
}

// Density counts (XAttentionBSAPolicy.select_blocks step 5 and the comm density after its step 6).
// One wave per (head, query block) row, sixteen rows per workgroup; a row's causal columns are
// 0 .. diag0 + qb (clipped to the mask) and its lanes count the kept bytes among them.  Workgroup 0 also
// counts the kept cache blocks.  One 64-bit atomic per counter and workgroup adds the totals to
// counts[0..3] (few workgroups, so few atomics meet on one address).
constexpr int kDensityWaves = 16;
__global__ __launch_bounds__(64 * kDensityWaves) void density_kernel(const uint8_t* __restrict__ mask, int heads,
                                                                   int n_qb, int64_t n_cols, int64_t hs,
                                                                   int64_t rs, int64_t diag0,
                                                                   const uint8_t* __restrict__ keep_any,
                                                                   int64_t n_cb, unsigned long long* counts) {
  __shared__ unsigned long long s_part[3][kDensityWaves];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  unsigned long long sel = 0, tot = 0, kept = 0;
  if (mask) {
    const int64_t rows = (int64_t)heads * n_qb;
    for (int64_t r = (int64_t)blockIdx.x * kDensityWaves + wave; r < rows; r += (int64_t)gridDim.x * kDensityWaves) {
      const int h = (int)(r / n_qb), qb = (int)(r % n_qb);
      int64_t last = diag0 + qb;
      if (last > n_cols - 1) last = n_cols - 1;
      const uint8_t* row = mask + h * hs + qb * rs;
#pragma unroll 4
      for (int64_t c = lane; c <= last; c += 64) sel += row[c] != 0;
      if (lane == 0 && last >= 0) tot += (unsigned long long)(last + 1);
    }
  }
  if (keep_any && blockIdx.x == 0)
    for (int64_t c = threadIdx.x; c < n_cb; c += blockDim.x) kept += keep_any[c] != 0;
  // wave sums, then the waves' partials through LDS
  for (int off = 32; off > 0; off >>= 1) {
    sel += __shfl_down(sel, off);
    tot += __shfl_down(tot, off);
    kept += __shfl_down(kept, off);
  }
  if (lane == 0) {
    s_part[0][wave] = sel;
    s_part[1][wave] = tot;
    s_part[2][wave] = kept;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long a = 0, b = 0, c = 0;
    for (int i = 0; i < kDensityWaves; ++i) {
      a += s_part[0][i];
      b += s_part[1][i];
      c += s_part[2][i];
    }
    if (a) atomicAdd(&counts[0], a);
    if (b) atomicAdd(&counts[1], b);
    if (blockIdx.x == 0 && keep_any) {
      if (c) atomicAdd(&counts[2], c);
      if (n_cb) atomicAdd(&counts[3], (unsigned long long)n_cb);
    }
  }
}

}  // namespace xa

using namespace xa;

extern "C" xa_status_t xattn_mask_to_cache_blocks(const uint8_t* block_mask, int32_t heads,
                                                  int32_t n_qb, int64_t n_cols, int64_t mask_head_stride,
                                                  int64_t mask_row_stride, int64_t kb_begin,
                                                  int64_t n_cache_blocks, int32_t sub_blocks,
                                                  int32_t force_first_last, uint8_t* keep_per_head,
                                                  uint8_t* keep_any, uint8_t* keep_any_blocks,
                                                  xa_stream_t stream) {
  using xa_host::fail;
  if (heads <= 0 || n_qb <= 0 || sub_blocks <= 0 || n_cols <= 0 || kb_begin < 0 || n_cache_blocks < 0)
    return fail(XA_EINVAL, "xattn_mask_to_cache_blocks: need heads, n_qb, sub_blocks, n_cols > 0 "
                "and kb_begin, n_cache_blocks >= 0");
  if (mask_head_stride < 0 || mask_row_stride < 0)
    return fail(XA_EINVAL, "xattn_mask_to_cache_blocks: negative mask stride");
  if (n_cache_blocks == 0) return XA_OK;
  if (kb_begin + (n_cache_blocks - 1) * (int64_t)sub_blocks >= n_cols)
    return fail(XA_EINVAL, "xattn_mask_to_cache_blocks: cache block %lld starts at column %lld >= n_cols %lld",
                (long long)(n_cache_blocks - 1),
                (long long)(kb_begin + (n_cache_blocks - 1) * (int64_t)sub_blocks), (long long)n_cols);
  if (!block_mask) return fail(XA_EINVAL, "xattn_mask_to_cache_blocks: null block_mask");
  if (!keep_per_head && !keep_any && !keep_any_blocks) return XA_OK;
  if (n_cache_blocks > 0x7fffffff) return fail(XA_EUNSUPPORTED, "xattn_mask_to_cache_blocks: too many cache blocks");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(cache_block_kernel, dim3((unsigned)n_cache_blocks), dim3(256), 0, s, block_mask,
                     heads, n_qb, n_cols, mask_head_stride, mask_row_stride, kb_begin, n_cache_blocks,
                     sub_blocks, force_first_last, keep_per_head, keep_any, keep_any_blocks);
  return xa_host::check_launch("xattn_mask_to_cache_blocks");
}

extern "C" xa_status_t xattn_density_counts(const uint8_t* block_mask, int32_t heads, int32_t n_qb, int64_t n_cols,
                                            int64_t mask_head_stride, int64_t mask_row_stride, int64_t diag0,
                                            const uint8_t* keep_any, int64_t n_cache_blocks, int64_t* counts,
                                            xa_stream_t stream) {
  using xa_host::fail;
  if (!counts) return fail(XA_EINVAL, "xattn_density_counts: null counts");
  if ((uintptr_t)counts % 8 != 0) return fail(XA_EINVAL, "xattn_density_counts: counts must be 8-byte aligned");
  if (block_mask && (heads <= 0 || n_qb <= 0 || n_cols <= 0))
    return fail(XA_EINVAL, "xattn_density_counts: need heads, n_qb, n_cols > 0 with a mask");
  if (block_mask && (mask_head_stride < 0 || mask_row_stride < 0))
    return fail(XA_EINVAL, "xattn_density_counts: negative mask stride");
  if (n_cache_blocks < 0) return fail(XA_EINVAL, "xattn_density_counts: negative n_cache_blocks");
  if (!keep_any && n_cache_blocks > 0)
    return fail(XA_EINVAL, "xattn_density_counts: n_cache_blocks > 0 needs keep_any");
  if (!block_mask && !keep_any) return XA_OK;
  const int64_t rows = block_mask ? (int64_t)heads * n_qb : 0;
  if (rows > 0x7fffffff) return fail(XA_EUNSUPPORTED, "xattn_density_counts: too many mask rows");
  const int64_t wgs = (rows + kDensityWaves - 1) / kDensityWaves;
  const unsigned grid = (unsigned)(wgs < 1 ? 1 : (wgs < 128 ? wgs : 128));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(density_kernel, dim3(grid), dim3(64 * kDensityWaves), 0, s, block_mask, block_mask ? heads : 0,
                     block_mask ? n_qb : 1, n_cols, mask_head_stride, mask_row_stride, diag0, keep_any,
                     n_cache_blocks, reinterpret_cast<unsigned long long*>(counts));
  return xa_host::check_launch("xattn_density_counts");
}
