// Bridges between the expanded layout and the decode path's masked slab.
//
// Sources: SGLang PR 37261, "Why decode stays on V1 low_latency" (the masked
// GEMM takes a fixed-height slab [num_local_experts, max_m, H] so the decode
// step keeps static shapes; the expanded layout reaches it through
// expand_to_masked_slab before the GEMMs and masked_slab_to_expand after);
// SGLang moe_runner/deep_gemm.py source, pre_permute_deepep_v2_to_deep_gemm
// (masked branch: slab, scales and masked_m from the expanded rows and the
// psum; masked_m bounds each expert independently of the buffer capacity)
// and post_permute_deep_gemm_to_deepep_v2 (masked branch: back to the
// expanded rows with the top-k weights applied, the combine takes none).
//
// Both are row copies, one wave per row, 16-byte accesses: HBM-bound.
//  - to_slab: slab row e * max_m + i <- expanded row align(psum[e-1]) + i
//    for i < masked_m[e] = min(count_e, max_m) (and below the capacity);
//    scales K-block-major on both sides; other slab rows untouched.  The
//    workgroup holding row e * max_m writes masked_m[e] and flags an expert
//    whose live rows exceed max_m.
//  - from_slab: expanded row m (below the device-side total) of expert e at
//    i = m - align(psum[e-1]) <- bf16(w[m] * slab[e * max_m + i]) for
//    i < masked_m[e] (fp32 product, one rounding; a copy without weights);
//    rows the slab height dropped (masked_m[e] <= i < count_e) are zeroed,
//    since their slots still point at them; alignment pad rows are left
//    alone (no slot points at them, the combine never reads them).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;  // four waves: one row each
constexpr int kRowsPerBlock = kThreads / 64;

__global__ __launch_bounds__(kThreads) void to_slab_kernel(
    const uint8_t* __restrict__ ex, const uint8_t* __restrict__ ex_scale, int sbytes,
    const int32_t* __restrict__ psum, int32_t* __restrict__ status, int64_t capacity,
    int hidden, int E, int align, int max_m, uint8_t* __restrict__ slab,
    uint8_t* __restrict__ slab_scale, int32_t* __restrict__ masked_m) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t srows = (int64_t)E * max_m;
  const int64_t nrows = min((int64_t)status[0], capacity);  // expanded rows defined
  const int nch = hidden / 16, nsc = hidden / kGroup;
  for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wid; row < srows;
       row += (int64_t)gridDim.x * kRowsPerBlock) {
    const int e = (int)(row / max_m);
    const int i = (int)(row - (int64_t)e * max_m);
    const int st = e ? align_up_i(psum[e - 1], align) : 0;
    const int cnt = psum[e] - st;
    const int n = (int)max((int64_t)0, min((int64_t)min(cnt, max_m), nrows - st));
    if (i == 0 && lane == 0) {
      masked_m[e] = n;
      if (cnt > max_m) atomicOr(status + 1, MOE_FLAG_SLAB_OVERFLOW);
    }
    if (i >= n) continue;
    const int64_t src = (int64_t)st + i;
    const u32x4* s = reinterpret_cast<const u32x4*>(ex + src * hidden);
    u32x4* d = reinterpret_cast<u32x4*>(slab + row * hidden);
    u32x4 v[8];
    for (int c0 = 0; c0 < nch; c0 += 64 * 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < nch) v[u] = s[c];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < nch) d[c] = v[u];
      }
    }
    for (int b = lane; b < nsc; b += 64) {
      if (sbytes == 4)
        reinterpret_cast<float*>(slab_scale)[b * srows + row] =
            reinterpret_cast<const float*>(ex_scale)[b * capacity + src];
      else
        slab_scale[b * srows + row] = ex_scale[b * capacity + src];
    }
  }
}

__global__ __launch_bounds__(kThreads) void from_slab_kernel(
    const uint16_t* __restrict__ so, const int32_t* __restrict__ masked_m, int max_m,
    const int32_t* __restrict__ psum, const int32_t* __restrict__ status,
    const int32_t* __restrict__ m_indices, const float* __restrict__ row_weight,
    int64_t capacity, int hidden, int E, int align, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t nrows = min((int64_t)status[0], capacity);
  const int nch = hidden / 8;  // 16-byte chunks of 8 bf16
  for (int64_t m = (int64_t)blockIdx.x * kRowsPerBlock + wid; m < nrows;
       m += (int64_t)gridDim.x * kRowsPerBlock) {
    const int e = m_indices[m];
    u32x4* d = reinterpret_cast<u32x4*>(out + m * hidden);
    int i = -1, n = 0, cnt = 0;
    if (e >= 0 && e < E) {
      const int st = e ? align_up_i(psum[e - 1], align) : 0;
      i = (int)(m - st);
      n = max(0, min(masked_m[e], max_m));
      cnt = psum[e] - st;
    }
    if (i < 0 || i >= cnt) continue;  // alignment pad row: not read by anyone
    if (i >= n) {                     // dropped by the slab height: zeros
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int c = lane; c < nch; c += 64) d[c] = z;
      continue;
    }
    const u32x4* s = reinterpret_cast<const u32x4*>(so + ((int64_t)e * max_m + i) * hidden);
    const float w = row_weight ? row_weight[m] : 1.f;
    u32x4 v[4];
    for (int c0 = 0; c0 < nch; c0 += 64 * 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < nch) v[u] = s[c];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c >= nch) continue;
        u32x4 o = v[u];
        if (row_weight) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float lo = __fmul_rn(w, __uint_as_float(o[j] << 16));
            const float hi = __fmul_rn(w, __uint_as_float(o[j] & 0xffff0000u));
            o[j] = (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
          }
        }
        d[c] = o;
      }
    }
  }
}

int64_t grid_for(int64_t rows) {
  int64_t g = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  return g < 1 ? 1 : (g > 16384 ? 16384 : g);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_expand_to_masked_slab(
    const void* ex, const void* ex_scale, moe_scale_fmt fmt, const int32_t* psum,
    int32_t* status, int64_t capacity, int hidden, int num_experts, int align, int max_m,
    void* slab, void* slab_scale, int32_t* masked_m, void* stream) {
  if (capacity < 0 || capacity > (1LL << 30) || hidden <= 0 || hidden % kGroup != 0 ||
      num_experts < 1 || num_experts > MOE_MAX_EXPERTS || max_m < 16 || max_m % 16 ||
      (int64_t)max_m * num_experts > (1LL << 30))
    return MOE_ERR_SHAPE;
  if (align < MOE_MIN_ALIGN || align > MOE_MAX_ALIGN || (align & (align - 1)))
    return MOE_ERR_UNSUPPORTED;
  if (fmt != MOE_SCALE_F32 && fmt != MOE_SCALE_UE8M0) return MOE_ERR_UNSUPPORTED;
  if (!psum || !status || !masked_m || !slab || !slab_scale) return MOE_ERR_NULL;
  if (capacity > 0 && (!ex || !ex_scale)) return MOE_ERR_NULL;
  if (((uintptr_t)ex % 16) || ((uintptr_t)slab % 16)) return MOE_ERR_ALIGNMENT;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t rows = (int64_t)max_m * num_experts;
  hipLaunchKernelGGL(to_slab_kernel, dim3((unsigned)grid_for(rows)), dim3(kThreads), 0, s,
                     (const uint8_t*)ex, (const uint8_t*)ex_scale,
                     fmt == MOE_SCALE_F32 ? 4 : 1, psum, status, capacity, hidden, num_experts,
                     align, max_m, (uint8_t*)slab, (uint8_t*)slab_scale, masked_m);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

extern "C" moe_status moe_masked_slab_to_expand(
    const void* slab_out, const int32_t* masked_m, int max_m, const int32_t* psum,
    const int32_t* status, const int32_t* m_indices, const float* row_weight,
    int64_t capacity, int hidden, int num_experts, int align, void* out, void* stream) {
  if (capacity < 0 || capacity > (1LL << 30) || hidden <= 0 || hidden % kGroup != 0 ||
      num_experts < 1 || num_experts > MOE_MAX_EXPERTS || max_m < 16 || max_m % 16 ||
      (int64_t)max_m * num_experts > (1LL << 30))
    return MOE_ERR_SHAPE;
  if (align < MOE_MIN_ALIGN || align > MOE_MAX_ALIGN || (align & (align - 1)))
    return MOE_ERR_UNSUPPORTED;
  if (!masked_m || !psum || !status || !m_indices || !slab_out) return MOE_ERR_NULL;
  if (capacity > 0 && !out) return MOE_ERR_NULL;
  if (((uintptr_t)slab_out % 16) || ((uintptr_t)out % 16)) return MOE_ERR_ALIGNMENT;
  if (capacity == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(from_slab_kernel, dim3((unsigned)grid_for(capacity)), dim3(kThreads), 0, s,
                     (const uint16_t*)slab_out, masked_m, max_m, psum, status, m_indices,
                     row_weight, capacity, hidden, num_experts, align, (uint16_t*)out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}
