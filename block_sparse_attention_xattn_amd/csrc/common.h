// Shared device/host helpers for the gfx950 XAttention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "xattn.h"

namespace xa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// MFMA: D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16), one wave.
// Lane l holds A[l%32][8*(l/32) .. +8], B[8*(l/32) .. +8][l%32] and
// D[8*(i/4) + 4*(l/32) + i%4][l%32] for i = 0..15.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combination of lane l's value with lane l^32's (the two 32-lane halves of a wave).  v_permlane32_swap
// exchanges the halves in one VALU instruction, where a shuffle would make a round trip through the LDS
// unit; called with the same register twice it hands every lane the pair {x_l, x_(l^32)}, so both
// halves compute the same result.  All 64 lanes must be active.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// fp32 -> (hi, lo) bf16 pair with hi + lo ~= x to about 16 mantissa bits.
__device__ __forceinline__ void split_bf16(float x, bf16& hi, bf16& lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}

// Key order inside each 16-key group of the transposed V tiles: position s
// holds key kSigma(s).  It matches the key order of the P fragment that a
// 32x32 MFMA accumulator yields when it is re-used as the B operand of the
// next MFMA (an involution: kSigma(kSigma(s)) == s).
__host__ __device__ __forceinline__ int kSigma(int s) {
  // 0..3 -> 0..3, 4..7 -> 8..11, 8..11 -> 4..7, 12..15 -> 12..15
  return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1);
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// A wave-uniform 64-bit value in scalar registers.
__device__ __forceinline__ int64_t rfl64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Spread consecutive work items over the 8 XCDs in contiguous runs: the
// hardware hands workgroup i to XCD i % 8, so item w is placed at slot
// (w % per_xcd) * 8 + w / per_xcd.  Neighbouring items (heads of one GQA group,
// adjacent query blocks) then share an XCD and its L2.
// Ids past the last multiple of 8 map to themselves.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int full = nblocks & ~7;
  if (bid >= full) return bid;
  return (bid & 7) * (full >> 3) + (bid >> 3);
}

}  // namespace xa

// ---------------------------------------------------------------------------
// Host-side error reporting (thread-local message).
// ---------------------------------------------------------------------------
namespace xa_host {
void set_error(const char* fmt, ...);
xa_status_t fail(xa_status_t st, const char* fmt, ...);
xa_status_t check_launch(const char* what);
}  // namespace xa_host
