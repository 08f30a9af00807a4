// LSE merge of two partial attention results (part 3 of the path).
//
// nano-vllm CLAUDE.md, "Online Softmax Merge - Triton Fused Kernel": with
// m = max(lse_a, lse_b) and e_x = exp(lse_x - m), the merged LSE is
// m + ln(e_a + e_b) and the merged output (o_a e_a + o_b e_b) / (e_a + e_b).
// One kernel does both (the pages use two launches).  HBM-bound: every
// element of o_a, o_b and o_out moves once, with 16-byte accesses.
#include "common.h"

namespace xa {

// One group of `lanes` consecutive lanes owns one (token, head) row and walks
// its head_dim in 8-element chunks.  A group never straddles a wave, so every
// lane of the row reads both LSE values before the group's first lane writes
// lse_out (in-place merges are safe).
template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(const T* __restrict__ o_a, const float* lse_a,
                                                    const T* __restrict__ o_b, const float* lse_b,
                                                    T* o_out, float* lse_out, int64_t q_len,
                                                    int heads, int head_dim, int lanes) {
  const int64_t rows = q_len * heads;
  const int rows_per_block = blockDim.x / lanes;
  // each XCD a contiguous range of rows, so the neighbouring tokens' LSE reads share cache lines in its L2
  const int64_t blk = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int64_t row = blk * rows_per_block + threadIdx.x / lanes;
  const int sub = threadIdx.x % lanes;
  if (row >= rows) return;
  const int64_t tok = row / heads;
  const int h = (int)(row % heads);
  const float la = lse_a[(int64_t)h * q_len + tok];
  const float lb = lse_b[(int64_t)h * q_len + tok];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lo = -INFINITY;
  if (m != -INFINITY) {
    const float ea = expf(la - m);
    const float eb = expf(lb - m);
    const float s = ea + eb;
    wa = ea / s;
    wb = eb / s;
    lo = m + logf(s);
  }
  const int64_t base = row * head_dim;
  for (int c = sub * 8; c < head_dim; c += lanes * 8) {
    if constexpr (sizeof(T) == 2) {
      const u32x4 va = *reinterpret_cast<const u32x4*>(o_a + base + c);
      const u32x4 vb = *reinterpret_cast<const u32x4*>(o_b + base + c);
      const bf16x8 a = as_bf16x8(va), b = as_bf16x8(vb);
      bf16x8 r;
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = (bf16)((float)a[j] * wa + (float)b[j] * wb);
      *reinterpret_cast<u32x4*>(o_out + base + c) = as_u32x4(r);
    } else {
      const f32x4* pa = reinterpret_cast<const f32x4*>(o_a + base + c);
      const f32x4* pb = reinterpret_cast<const f32x4*>(o_b + base + c);
      f32x4* po = reinterpret_cast<f32x4*>(o_out + base + c);
      const f32x4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
      po[0] = a0 * wa + b0 * wb;
      po[1] = a1 * wa + b1 * wb;
    }
  }
  if (sub == 0) lse_out[(int64_t)h * q_len + tok] = lo;
}

}  // namespace xa

using namespace xa;

extern "C" xa_status_t attn_merge(const void* o_a, const float* lse_a, const void* o_b,
                                  const float* lse_b, void* o_out, float* lse_out,
                                  xa_dtype_t o_dtype, int64_t q_len, int32_t heads,
                                  int32_t head_dim, xa_stream_t stream) {
  using xa_host::fail;
  if (q_len < 0 || heads <= 0 || head_dim <= 0 || head_dim % 8 != 0)
    return fail(XA_EINVAL, "attn_merge: need q_len >= 0, heads > 0, head_dim > 0 and head_dim %% 8 == 0 "
                "(got q_len=%lld heads=%d head_dim=%d)", (long long)q_len, heads, head_dim);
  if (o_dtype != XA_F32 && o_dtype != XA_BF16)
    return fail(XA_EUNSUPPORTED, "attn_merge: o_dtype must be XA_F32 or XA_BF16");
  if (q_len == 0) return XA_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out)
    return fail(XA_EINVAL, "attn_merge: null pointer");
  const size_t esz = o_dtype == XA_BF16 ? 2 : 4;
  if (((uintptr_t)o_a | (uintptr_t)o_b | (uintptr_t)o_out) % 16 != 0)
    return fail(XA_EINVAL, "attn_merge: o_a, o_b and o_out must be 16-byte aligned");
  (void)esz;
  int chunks = head_dim / 8;
  int lanes = 1;
  while (lanes < chunks && lanes < 64) lanes <<= 1;
  const int threads = 256;
  const int64_t rows = q_len * heads;
  const int64_t rows_per_block = threads / lanes;
  const int64_t grid = (rows + rows_per_block - 1) / rows_per_block;
  if (grid > 0x7fffffff) return fail(XA_EUNSUPPORTED, "attn_merge: problem too large");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (o_dtype == XA_BF16)
    hipLaunchKernelGGL(merge_kernel<bf16>, dim3((unsigned)grid), dim3(threads), 0, s,
                       (const bf16*)o_a, lse_a, (const bf16*)o_b, lse_b, (bf16*)o_out, lse_out,
                       q_len, heads, head_dim, lanes);
  else
    hipLaunchKernelGGL(merge_kernel<float>, dim3((unsigned)grid), dim3(threads), 0, s,
                       (const float*)o_a, lse_a, (const float*)o_b, lse_b, (float*)o_out, lse_out,
                       q_len, heads, head_dim, lanes);
  return xa_host::check_launch("attn_merge");
}
