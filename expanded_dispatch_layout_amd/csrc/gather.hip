// moe_gather: each token's expert rows summed back into one bf16 row.
//
// Sources: SGLang moe_runner/deep_gemm.py source, post_permute_deep_gemm_to_
// deepep_v2 (expanded branch: rows weighted, then combined) and ep_gather's
// use in post_permute_deep_gemm_to_deepep_normal; SGLang PR 37261
// Modifications/Core (under UE8M0 scales the top-k weight is applied to the
// down output rather than folded into the scale).
//
// One wave per token row; each lane owns 8 bf16 columns per 16-byte chunk.
// All of a row's live slots are loaded before the sums, k ascending, each
// product and sum rounded to fp32 (no contraction), one bf16 rounding at the
// end.  HBM-bound: reads A rows of expert output, writes R_v token rows.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;

__device__ __forceinline__ void acc8(float* a, const u32x4& v, float c, bool weighted) {
  const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = __uint_as_float(w[i] << 16);
    float hi = __uint_as_float(w[i] & 0xffff0000u);
    if (weighted) {
      lo = __fmul_rn(c, lo);
      hi = __fmul_rn(c, hi);
    }
    a[2 * i] = __fadd_rn(a[2 * i], lo);
    a[2 * i + 1] = __fadd_rn(a[2 * i + 1], hi);
  }
}

__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint16_t* __restrict__ eo, const int32_t* __restrict__ src2dst,
    const float* __restrict__ topk_w, const int32_t* __restrict__ psum_rank, int nsrc,
    int64_t rows, int hidden, int topk, int64_t capacity, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int64_t nv = valid_rows(psum_rank, nsrc, rows);
  if (r >= nv) return;
  // Wave-uniform list of live slots (k ascending), compacted into LDS.
  __shared__ int l_dst[kRowsPerBlock][MOE_MAX_TOPK];
  __shared__ float l_w[kRowsPerBlock][MOE_MAX_TOPK];
  const int wid = threadIdx.x >> 6;
  int d = -1;
  float wk = 1.f;
  if (lane < topk) {
    d = src2dst[r * topk + lane];
    if (topk_w) wk = topk_w[r * topk + lane];
  }
  const bool live = lane < topk && d >= 0 && d < capacity;
  const uint64_t mask = __ballot(live);
  if (live) {
    const int idx = __popcll(mask & ((1ull << lane) - 1ull));
    l_dst[wid][idx] = d;
    l_w[wid][idx] = wk;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  const int n = __popcll(mask);
  const int* dst = l_dst[wid];
  const float* wt = l_w[wid];
  const bool weighted = topk_w != nullptr;
  const int nch = hidden / 8;  // 16-byte chunks of 8 bf16
  u32x4* orow = reinterpret_cast<u32x4*>(out + r * hidden);
  for (int c = lane; c < nch; c += 64) {
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = 0.f;
    int k = 0;
    for (; k + 4 <= n; k += 4) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = reinterpret_cast<const u32x4*>(eo + (int64_t)dst[k + u] * hidden)[c];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc8(a, v[u], wt[k + u], weighted);
    }
    for (; k < n; ++k) {
      u32x4 v = reinterpret_cast<const u32x4*>(eo + (int64_t)dst[k] * hidden)[c];
      acc8(a, v, wt[k], weighted);
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)f32_to_bf16_rne(a[2 * i]) | ((uint32_t)f32_to_bf16_rne(a[2 * i + 1]) << 16);
    orow[c] = o;
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_gather(const void* expert_out, const int32_t* src2dst,
                                 const float* topk_weights, const int32_t* psum_recv_per_rank,
                                 int num_src_ranks, int64_t rows, int hidden, int topk,
                                 int64_t capacity, void* out, void* stream) {
  if (rows < 0 || hidden <= 0 || hidden % kGroup != 0 || topk < 1 || topk > MOE_MAX_TOPK ||
      capacity < 0 || rows > (1LL << 30))
    return MOE_ERR_SHAPE;
  if (num_src_ranks < 0 || (psum_recv_per_rank && num_src_ranks == 0)) return MOE_ERR_SHAPE;
  if (rows > 0 && (!src2dst || !out)) return MOE_ERR_NULL;
  if (capacity > 0 && !expert_out) return MOE_ERR_NULL;
  if (((uintptr_t)expert_out % 16) || ((uintptr_t)out % 16)) return MOE_ERR_ALIGNMENT;
  if (rows == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t grid = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s,
                     (const uint16_t*)expert_out, src2dst, topk_weights, psum_recv_per_rank,
                     num_src_ranks, rows, hidden, topk, capacity, (uint16_t*)out);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
  return MOE_OK;
}
