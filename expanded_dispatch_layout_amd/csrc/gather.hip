// moe_gather: each token's expert rows summed back into one bf16 row.
//
// Sources: SGLang moe_runner/deep_gemm.py source, post_permute_deep_gemm_to_
// deepep_v2 (expanded branch: rows weighted, then combined) and ep_gather's
// use in post_permute_deep_gemm_to_deepep_normal; SGLang PR 37261
// Modifications/Core (under UE8M0 scales the top-k weight is applied to the
// down output rather than folded into the scale).
//
// One workgroup per token row; each thread owns up to four 16-byte chunks
// (8 bf16 each) of the row.  The slots are summed in ascending k, each
// product and sum rounded to fp32 (no contraction), with one bf16 rounding at
// the end.  HBM-bound: reads A rows of expert output, writes R_v token rows
// (non-temporal stores: the output is not re-read by this layer).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;  // one token row per workgroup
constexpr int kChunksPerThread = 4;  // 16-byte chunks; H <= 8192 in one pass

__device__ __forceinline__ void acc8(float* a, const u32x4& v, float c, bool weighted) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = __uint_as_float(v[i] << 16);
    float hi = __uint_as_float(v[i] & 0xffff0000u);
    if (weighted) {
      lo = __fmul_rn(c, lo);
      hi = __fmul_rn(c, hi);
    }
    a[2 * i] = __fadd_rn(a[2 * i], lo);
    a[2 * i + 1] = __fadd_rn(a[2 * i + 1], hi);
  }
}

// One workgroup per token row: every thread owns up to four 16-byte chunks
// of the row, so all of a slot's loads are issued together and the row's
// latency is one memory round trip per group of four slots.
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint16_t* __restrict__ eo, const int32_t* __restrict__ src2dst,
    const float* __restrict__ topk_w, const int32_t* __restrict__ psum_rank, int nsrc,
    int64_t rows, int hidden, int topk, int64_t capacity, uint16_t* __restrict__ out) {
  __shared__ int l_dst[MOE_MAX_TOPK];
  __shared__ float l_w[MOE_MAX_TOPK];
  __shared__ int l_n;
  const int t = threadIdx.x, lane = t & 63;
  const int nch = hidden / 8;  // 16-byte chunks of 8 bf16
  const bool weighted = topk_w != nullptr;
  // The first row's slots are read together with the valid-row boundary
  // (the grid never exceeds the row count, so row blockIdx.x is in bounds).
  int d0 = -1;
  float w0 = 1.f;
  if (t < 64 && lane < topk) {
    d0 = src2dst[(int64_t)blockIdx.x * topk + lane];
    if (weighted) w0 = topk_w[(int64_t)blockIdx.x * topk + lane];
  }
  const int64_t nv = valid_rows(psum_rank, nsrc, rows);
  for (int64_t r = blockIdx.x; r < nv; r += gridDim.x) {
    // Live slots in k order, compacted into LDS by wave 0.
    if (t < 64) {
      int d = d0;
      float wk = w0;
      if (r != blockIdx.x && lane < topk) {
        d = src2dst[r * topk + lane];
        if (weighted) wk = topk_w[r * topk + lane];
      }
      const bool live = lane < topk && d >= 0 && d < capacity;
      const uint64_t mask = __ballot(live);
      if (live) {
        const int idx = __popcll(mask & ((1ull << lane) - 1ull));
        l_dst[idx] = d;
        l_w[idx] = wk;
      }
      if (lane == 0) l_n = __popcll(mask);
    }
    __syncthreads();
    const int n = l_n;
    float a[kChunksPerThread][8];
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) a[i][j] = 0.f;
    for (int k0 = 0; k0 < n; k0 += 4) {
      u32x4 v[4][kChunksPerThread];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (k0 + u < n) {
          const u32x4* src = reinterpret_cast<const u32x4*>(eo + (int64_t)l_dst[k0 + u] * hidden);
#pragma unroll
          for (int i = 0; i < kChunksPerThread; ++i) {
            const int c = t + i * kThreads;
            if (c < nch) v[u][i] = src[c];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (k0 + u < n) {
          const float wk = l_w[k0 + u];
#pragma unroll
          for (int i = 0; i < kChunksPerThread; ++i) acc8(a[i], v[u][i], wk, weighted);
        }
      }
    }
    u32x4* orow = reinterpret_cast<u32x4*>(out + r * hidden);
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int c = t + i * kThreads;
      if (c < nch) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = (uint32_t)f32_to_bf16_rne(a[i][2 * j]) |
                 ((uint32_t)f32_to_bf16_rne(a[i][2 * j + 1]) << 16);
        __builtin_nontemporal_store(o, orow + c);
      }
    }
    __syncthreads();  // l_dst / l_n are rewritten for the next row
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
  if (hidden / 8 > kThreads * kChunksPerThread) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t grid = rows < 4096 ? rows : 4096;  // grid-stride over the rows
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s,
                     (const uint16_t*)expert_out, src2dst, topk_weights, psum_recv_per_rank,
                     num_src_ranks, rows, hidden, topk, capacity, (uint16_t*)out);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
  return MOE_OK;
}
