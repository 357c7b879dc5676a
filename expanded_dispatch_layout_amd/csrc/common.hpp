// Shared device helpers for the gfx950 kernels of libmoe_expand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_expand.h"

namespace moe {

constexpr int kWave = 64;

// Native 16-byte vector.  HIP's uint4 is a class wrapping a union, and arrays
// of it tend to be kept in scratch memory instead of registers.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kGroup = 128;  // quantisation group / block edge

__device__ __forceinline__ int64_t valid_rows(const int32_t* psum_recv_per_rank,
                                              int num_src_ranks, int64_t rows) {
  if (psum_recv_per_rank == nullptr || num_src_ranks <= 0) return rows;
  int64_t v = psum_recv_per_rank[num_src_ranks - 1];
  return v < 0 ? 0 : (v > rows ? rows : v);
}

__device__ __forceinline__ int align_up_i(int x, int a) { return (x + a - 1) & ~(a - 1); }

// Wave-wide reductions and scans over 64 lanes (ds_swizzle/bpermute based).
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_or_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, kWave);
  return v;
}
// Inclusive prefix sum over lanes, with DPP moves (VALU, a few cycles each,
// where a shuffle is an LDS-crossbar round trip): a Hillis-Steele scan within
// each row of 16 lanes (row_shr 1, 2, 4, 8; lanes whose source falls before
// the row keep 0), then lane 15's total added to rows 1 and 3 (row_bcast:15)
// and lane 31's to rows 2 and 3 (row_bcast:31).  Every lane must be active.
__device__ __forceinline__ int wave_incl_scan_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// UE8M0 byte of the smallest power of two not below the fp32 scale s: the
// biased exponent, plus one unless the mantissa is zero; the largest finite
// exponent is not bumped, and neither is a denormal of at most half the
// smallest normal (SGLang moe_runner/deep_gemm.py source,
// _cast_to_e8m0_with_rounding_up).
__device__ __forceinline__ uint32_t e8m0_round_up(float s) {
  const uint32_t bits = __float_as_uint(s);
  const uint32_t ex = bits >> 23, mant = bits & 0x7fffffu;
  const bool bump = (mant > 0) && (ex != 0xfe) && !(ex == 0 && mant <= 0x400000u);
  return ex + (bump ? 1u : 0u);
}

}  // namespace moe
