// moe_gather: each token's expert rows summed back into one bf16 row.
//
// Sources: SGLang moe_runner/deep_gemm.py source, post_permute_deep_gemm_to_
// deepep_v2 (expanded branch: rows weighted, then combined) and ep_gather's
// use in post_permute_deep_gemm_to_deepep_normal; SGLang PR 37261
// Modifications/Core (under UE8M0 scales the top-k weight is applied to the
// down output rather than folded into the scale); the standard path's
// post_permute_deep_gemm_to_standard (post_reorder_deepgemm: the top-k
// weighted sum times the routed scaling factor).
//
// Four token rows per workgroup; each thread owns up to four 16-byte chunks
// (8 bf16 each) of a row.  The slots are summed in ascending k, each
// product and sum rounded to fp32 (no contraction), the sum multiplied by the
// routed scaling factor (1 on the expand path: exact), with one bf16 rounding
// at the end.  HBM-bound: reads A rows of expert output, writes R_v token rows
// (non-temporal stores: the output is not re-read by this layer).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;  // four waves: one per row of a quad
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

constexpr int kRowsPerBlock = 4;  // one wave reads each row's slot list

// Row r's fp32 sums (zeros for a row without a live slot) times `scale`,
// rounded once to bf16, non-temporal 16-byte stores.
__device__ __forceinline__ void store_row(uint16_t* __restrict__ out, int64_t r, int hidden,
                                          const float (&a)[kChunksPerThread][8], float scale) {
  const int t = threadIdx.x, nch = hidden / 8;
  u32x4* orow = reinterpret_cast<u32x4*>(out + r * hidden);
#pragma unroll
  for (int i = 0; i < kChunksPerThread; ++i) {
    const int c = t + i * kThreads;
    if (c < nch) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = (uint32_t)f32_to_bf16_rne(__fmul_rn(a[i][2 * j], scale)) |
               ((uint32_t)f32_to_bf16_rne(__fmul_rn(a[i][2 * j + 1], scale)) << 16);
      __builtin_nontemporal_store(o, orow + c);
    }
  }
}

// Four token rows per workgroup (grid-stride over row quads).  Wave j reads
// row j's slot list and compacts the live slots into LDS (one memory round
// trip for the four rows); the rows without a live slot are stored (zeros)
// first, so their stores are under way while the live rows' expert rows are
// loaded: every thread owns up to four 16-byte chunks of the row, a slot's
// loads are issued together, one round trip per group of four slots.  The
// slots are summed in ascending k, each product and sum rounded to fp32 (no
// contraction).
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint16_t* __restrict__ eo, const int32_t* __restrict__ src2dst,
    const float* __restrict__ topk_w, float scale, const int32_t* __restrict__ psum_rank,
    int nsrc, int64_t rows, int hidden, int topk, int64_t capacity, uint16_t* __restrict__ out) {
  __shared__ int l_dst[kRowsPerBlock][MOE_MAX_TOPK];
  __shared__ float l_w[kRowsPerBlock][MOE_MAX_TOPK];
  __shared__ int l_n[kRowsPerBlock];
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int nch = hidden / 8;  // 16-byte chunks of 8 bf16
  const bool weighted = topk_w != nullptr;
  const int64_t nv = valid_rows(psum_rank, nsrc, rows);
  const int64_t nquads = (nv + kRowsPerBlock - 1) / kRowsPerBlock;
  for (int64_t q = blockIdx.x; q < nquads; q += gridDim.x) {
    const int64_t r0 = q * kRowsPerBlock;
    if (wid < kRowsPerBlock) {  // wave j: row r0 + j's live slots, in k order
      const int64_t r = r0 + wid;
      int d = -1;
      float wk = 1.f;
      if (r < nv && lane < topk) {
        d = src2dst[r * topk + lane];
        if (weighted) wk = topk_w[r * topk + lane];
      }
      const bool live = r < nv && lane < topk && d >= 0 && d < capacity;
      const uint64_t mask = __ballot(live);
      if (live) {
        const int idx = __popcll(mask & ((1ull << lane) - 1ull));
        l_dst[wid][idx] = d;
        l_w[wid][idx] = wk;
      }
      if (lane == 0) l_n[wid] = r < nv ? __popcll(mask) : -1;
    }
    __syncthreads();
    // Loads of one group of up to four slots of row j (starting at slot k0).
    u32x4 v[4][kChunksPerThread];
    auto load_slots = [&](int j, int k0, int n) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (k0 + u < n) {
          const u32x4* src =
              reinterpret_cast<const u32x4*>(eo + (int64_t)l_dst[j][k0 + u] * hidden);
#pragma unroll
          for (int i = 0; i < kChunksPerThread; ++i) {
            const int c = t + i * kThreads;
            if (c < nch) v[u][i] = src[c];
          }
        }
      }
    };
    // The first live row's first slots are loaded before the zero rows are
    // stored, so that those loads are not queued behind the stores.
    int jl = -1;
    for (int j = kRowsPerBlock - 1; j >= 0; --j)
      if (l_n[j] > 0) jl = j;
    if (jl >= 0) load_slots(jl, 0, l_n[jl]);
    float a[kChunksPerThread][8];
    // Rows without a live slot: zeros.
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) a[i][j] = 0.f;
    for (int j = 0; j < kRowsPerBlock; ++j)
      if (l_n[j] == 0) store_row(out, r0 + j, hidden, a, 1.f);
    // Rows with live slots.
    for (int j = (jl >= 0 ? jl : kRowsPerBlock); j < kRowsPerBlock; ++j) {
      const int n = l_n[j];
      if (n <= 0) continue;
#pragma unroll
      for (int i = 0; i < kChunksPerThread; ++i)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) a[i][jj] = 0.f;
      for (int k0 = 0; k0 < n; k0 += 4) {
        if (j != jl || k0 > 0) load_slots(j, k0, n);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (k0 + u < n) {
            const float wk = l_w[j][k0 + u];
#pragma unroll
            for (int i = 0; i < kChunksPerThread; ++i) acc8(a[i], v[u][i], wk, weighted);
          }
        }
      }
      store_row(out, r0 + j, hidden, a, scale);
    }
    __syncthreads();  // the slot lists are rewritten for the next quad
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_gather(const void* expert_out, const int32_t* src2dst,
                                 const float* topk_weights, float routed_scaling_factor,
                                 const int32_t* psum_recv_per_rank,
                                 int num_src_ranks, int64_t rows, int hidden, int topk,
                                 int64_t capacity, void* out, void* stream) {
  if (rows < 0 || hidden <= 0 || hidden % kGroup != 0 || topk < 1 || topk > MOE_MAX_TOPK ||
      capacity < 0 || rows > (1LL << 30))
    return MOE_ERR_SHAPE;
  if (num_src_ranks < 0 || (psum_recv_per_rank && num_src_ranks == 0)) return MOE_ERR_SHAPE;
  if (rows > 0 && (!src2dst || !out)) return MOE_ERR_NULL;
  if (!(routed_scaling_factor == routed_scaling_factor) ||
      __builtin_isinf(routed_scaling_factor))
    return MOE_ERR_UNSUPPORTED;  // a NaN or infinite factor
  if (capacity > 0 && !expert_out) return MOE_ERR_NULL;
  if (((uintptr_t)expert_out % 16) || ((uintptr_t)out % 16)) return MOE_ERR_ALIGNMENT;
  if (hidden / 8 > kThreads * kChunksPerThread) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Grid-stride over row quads; 1024 workgroups keep every quad of the
  // DeepSeek-V3-shape share resident at once.
  const int64_t quads = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t grid = quads < 1024 ? quads : 1024;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s,
                     (const uint16_t*)expert_out, src2dst, topk_weights, routed_scaling_factor,
                     psum_recv_per_rank,
                     num_src_ranks, rows, hidden, topk, capacity, (uint16_t*)out);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
  return MOE_OK;
}
