// moe_act_quant: SiLU(gate)*up with per-1x128 fp8 quantisation of every
// live expanded row, and the top-k weight folded into the fp32 scale.
//
// Sources: SGLang moe_runner/deep_gemm.py source, _run_contiguous_gemm
// (SiLU*up between the two grouped GEMMs, then per-token-group fp8 quant
// with 128-wide groups), _situ_mul_quant_contig_kernel (the quantisation
// rule: amax clamped at 1e-10, codes y * (448 / amax), scale amax / 448),
// _cast_to_e8m0_with_rounding_up (power-of-two scales rounded up); SGLang
// PR 37261 Modifications/Core (fold the row's top-k weight into the down
// projection's fp32 input scale; not under UE8M0).
//
// One workgroup per row (grid-stride over rows up to the device-side total);
// each thread handles 8 columns per 2048-column pass, so a whole I=2048 row is
// one round trip; the 16 lanes of a 128-column group reduce their max with
// xor-shuffles.  HBM-bound: reads the bf16 gate/up row once, writes fp8 codes
// and one scale per group.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;  // one expanded row per workgroup

__device__ __forceinline__ float silu_mul(float g, float u) {
  const float den = __fadd_rn(1.0f, expf(-g));
  return __fmul_rn(__fdiv_rn(g, den), u);
}

// kMasked (the decode path's slab, rows e * max_m + i): `m_indices` is
// masked_m, `psum` and `status` are unused, capacity = E * max_m; rows with
// i >= masked_m[e] are neither read nor written (nothing reads them).
// kBfOut (the bf16-weight path, SGLang moe_runner/deep_gemm.py source,
// _run_bf16_contiguous_gemm: silu_and_mul to bf16 between the bf16 GEMMs):
// y is rounded to bf16 and stored to `out` as [capacity, inter] bf16, with no
// quantisation; pad rows are not written (the GEMM never reads them).
// kMx (MXFP8, with kUe8m0): 1x32 groups (4 lanes), each group's UE8M0 byte
// stored as byte (col / 32) % 4 of the row's word for its 128-wide block.
template <bool kUe8m0, bool kFold, bool kMasked, bool kBfOut = false, bool kMx = false>
__global__ __launch_bounds__(kThreads) void act_quant_kernel(
    const uint16_t* __restrict__ gu, const int32_t* __restrict__ m_indices,
    const int32_t* __restrict__ psum, const int32_t* __restrict__ status, int64_t capacity,
    int inter, int E, int max_m, const float* __restrict__ fold_w, uint8_t* __restrict__ out,
    uint8_t* __restrict__ out_scale) {
  const int t = threadIdx.x, lane = t & 63;
  const int ngroups = inter / kGroup;
  // Round trip 1: the total, this workgroup's first label and every
  // expert's end together (the grid never exceeds the capacity, so row
  // blockIdx.x is in bounds): with at most 64 experts lane e holds psum[e],
  // with more the workgroup copies psum into LDS.
  __shared__ int l_pe[kMasked ? 1 : MOE_MAX_EXPERTS];
  int64_t m = blockIdx.x;
  int e_next = kMasked ? 0 : m_indices[m];
  const bool psum_lanes = !kMasked && E <= 64;
  const int pl = psum_lanes && lane < E ? psum[lane] : 0;
  if (!kMasked && !psum_lanes) {  // uniform
    for (int e = t; e < E; e += kThreads) l_pe[e] = psum[e];
    __syncthreads();
  }
  const int64_t nrows = kMasked ? capacity : min((int64_t)status[0], capacity);
  for (; m < nrows; m += gridDim.x) {
    int e, pe;
    if constexpr (kMasked) {
      e = (int)(m / max_m);
      pe = e * max_m + max(0, min(m_indices[e], max_m));
      if (m >= pe) continue;  // past the slab's live rows
    } else {
      e = e_next;
      if (m + gridDim.x < nrows) e_next = m_indices[m + gridDim.x];
      if (e < 0 || e >= E) continue;  // uniform per workgroup
    }
    // Round trip 2: the fold weight and the row's first pass together (a
    // pad row loads none).
    if constexpr (!kMasked) pe = psum_lanes ? __shfl(pl, e, 64) : l_pe[e];
    const float w = kFold ? fold_w[m] : 1.f;
    const uint16_t* grow = gu + m * (int64_t)(2 * inter);
    u32x4 gv0 = {0u, 0u, 0u, 0u}, uv0 = {0u, 0u, 0u, 0u};
    if (t * 8 < inter && m < pe) {
      gv0 = *reinterpret_cast<const u32x4*>(grow + t * 8);
      uv0 = *reinterpret_cast<const u32x4*>(grow + inter + t * 8);
    }
    uint8_t* qrow = out + m * inter;
    if constexpr (kBfOut) {
      if (m >= pe) continue;  // alignment pad row: never read
      uint16_t* brow = reinterpret_cast<uint16_t*>(out) + m * inter;
      for (int c0 = 0; c0 < inter; c0 += kThreads * 8) {
        const int col = c0 + t * 8;
        if (col >= inter) continue;
        const u32x4 gv = c0 == 0 ? gv0 : *reinterpret_cast<const u32x4*>(grow + col);
        const u32x4 uv = c0 == 0 ? uv0 : *reinterpret_cast<const u32x4*>(grow + inter + col);
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo =
              silu_mul(__uint_as_float(gv[i] << 16), __uint_as_float(uv[i] << 16));
          const float hi = silu_mul(__uint_as_float(gv[i] & 0xffff0000u),
                                    __uint_as_float(uv[i] & 0xffff0000u));
          o[i] = (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
        }
        *reinterpret_cast<u32x4*>(brow + col) = o;
      }
      continue;
    }
    // out_scale is K-block-major: scale (row m, group g) at g * capacity + m.
    if (m >= pe) {  // alignment pad row: zeros
      for (int c = t; c < inter / 16; c += kThreads)
        reinterpret_cast<u32x4*>(qrow)[c] = u32x4{0u, 0u, 0u, 0u};
      for (int g = t; g < ngroups; g += kThreads) {
        if (kMx) reinterpret_cast<uint32_t*>(out_scale)[g * capacity + m] = 0u;
        else if (kUe8m0) out_scale[g * capacity + m] = 0;
        else reinterpret_cast<float*>(out_scale)[g * capacity + m] = 0.f;
      }
      continue;
    }
    // Each thread owns 8 consecutive columns per pass of kThreads*8 columns;
    // the 16 threads of a 128-column group are 16 consecutive lanes.
    for (int c0 = 0; c0 < inter; c0 += kThreads * 8) {
      const int col = c0 + t * 8;
      const bool active = col < inter;
      float y[8];
      float amax = 0.f;
      if (active) {
        const u32x4 gv = c0 == 0 ? gv0 : *reinterpret_cast<const u32x4*>(grow + col);
        const u32x4 uv = c0 == 0 ? uv0 : *reinterpret_cast<const u32x4*>(grow + inter + col);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[2 * i] = silu_mul(__uint_as_float(gv[i] << 16), __uint_as_float(uv[i] << 16));
          y[2 * i + 1] =
              silu_mul(__uint_as_float(gv[i] & 0xffff0000u), __uint_as_float(uv[i] & 0xffff0000u));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
      }
#pragma unroll
      for (int o = kMx ? 2 : 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      amax = fmaxf(amax, 1e-10f);
      if (!active) continue;
      float scale_out = 0.f;
      uint32_t sbyte = 0;
      float p[8];
      if (kUe8m0) {
        sbyte = e8m0_round_up(__fdiv_rn(amax, 448.0f));
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = ldexpf(y[i], 127 - (int)sbyte);
      } else {
        const float inv = __fdiv_rn(448.0f, amax);
        scale_out = __fdiv_rn(amax, 448.0f);
        if (kFold) scale_out = __fmul_rn(scale_out, w);
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = __fmul_rn(y[i], inv);
      }
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[4], p[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[6], p[7], hi, true);
      *reinterpret_cast<uint2*>(qrow + col) = make_uint2((uint32_t)lo, (uint32_t)hi);
      if constexpr (kMx) {
        if ((lane & 3) == 0)
          out_scale[((int64_t)(col / kGroup) * capacity + m) * 4 + (col / 32) % 4] =
              (uint8_t)sbyte;
      } else if ((lane & 15) == 0) {
        const int grp = col / kGroup;
        if (kUe8m0) out_scale[grp * capacity + m] = (uint8_t)sbyte;
        else reinterpret_cast<float*>(out_scale)[grp * capacity + m] = scale_out;
      }
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_act_quant(const void* gate_up, const int32_t* m_indices,
                                    const int32_t* psum, const int32_t* status, int64_t capacity,
                                    int inter, int num_experts, int align, moe_scale_fmt fmt,
                                    const float* fold_weight, void* out, void* out_scale,
                                    void* stream) {
  if (capacity < 0 || capacity > (1LL << 30) || inter <= 0 || inter % kGroup != 0 ||
      num_experts < 1 || num_experts > MOE_MAX_EXPERTS)
    return MOE_ERR_SHAPE;
  if (align < MOE_MIN_ALIGN || align > MOE_MAX_ALIGN || (align & (align - 1)))
    return MOE_ERR_UNSUPPORTED;
  if (capacity % align != 0) return MOE_ERR_SHAPE;
  if (fmt != MOE_SCALE_F32 && fmt != MOE_SCALE_UE8M0 && fmt != MOE_SCALE_MXFP8)
    return MOE_ERR_UNSUPPORTED;
  if (fmt != MOE_SCALE_F32 && fold_weight) return MOE_ERR_UNSUPPORTED;
  if (!m_indices || !psum || !status) return MOE_ERR_NULL;
  if (capacity > 0 && (!gate_up || !out || !out_scale)) return MOE_ERR_NULL;
  if (((uintptr_t)gate_up % 16) || ((uintptr_t)out % 16)) return MOE_ERR_ALIGNMENT;
  if (fmt != MOE_SCALE_UE8M0 && ((uintptr_t)out_scale % 4)) return MOE_ERR_ALIGNMENT;
  if (capacity == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int64_t grid = capacity < 2048 ? capacity : 2048;  // grid-stride over the live rows
  auto kern = fmt == MOE_SCALE_MXFP8 ? act_quant_kernel<true, false, false, false, true>
              : fmt == MOE_SCALE_UE8M0 ? act_quant_kernel<true, false, false>
              : fold_weight           ? act_quant_kernel<false, true, false>
                                      : act_quant_kernel<false, false, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, s, (const uint16_t*)gate_up,
                     m_indices, psum, status, capacity, inter, num_experts, 0, fold_weight,
                     (uint8_t*)out, (uint8_t*)out_scale);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
  return MOE_OK;
}

extern "C" moe_status moe_silu_mul_bf16(const void* gate_up, const int32_t* m_indices,
                                        const int32_t* psum, const int32_t* status,
                                        int64_t capacity, int inter, int num_experts, int align,
                                        void* out, void* stream) {
  if (capacity < 0 || capacity > (1LL << 30) || inter <= 0 || inter % 8 != 0 ||
      num_experts < 1 || num_experts > MOE_MAX_EXPERTS)
    return MOE_ERR_SHAPE;
  if (align < MOE_MIN_ALIGN || align > MOE_MAX_ALIGN || (align & (align - 1)))
    return MOE_ERR_UNSUPPORTED;
  if (capacity % align != 0) return MOE_ERR_SHAPE;
  if (!m_indices || !psum || !status) return MOE_ERR_NULL;
  if (capacity > 0 && (!gate_up || !out)) return MOE_ERR_NULL;
  if (((uintptr_t)gate_up % 16) || ((uintptr_t)out % 16)) return MOE_ERR_ALIGNMENT;
  if (capacity == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int64_t grid = capacity < 2048 ? capacity : 2048;
  hipLaunchKernelGGL((act_quant_kernel<false, false, false, true>), dim3((unsigned)grid),
                     dim3(kThreads), 0, s, (const uint16_t*)gate_up, m_indices, psum, status,
                     capacity, inter, num_experts, 0, nullptr, (uint8_t*)out, nullptr);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
  return MOE_OK;
}

extern "C" moe_status moe_act_quant_masked(const void* gate_up, const int32_t* masked_m,
                                           int max_m, int inter, int num_experts,
                                           moe_scale_fmt fmt, void* out, void* out_scale,
                                           void* stream) {
  if (max_m < 0 || max_m > (1 << 24) || max_m % 16 || inter <= 0 || inter % kGroup != 0 ||
      num_experts < 1 || num_experts > MOE_MAX_EXPERTS ||
      (int64_t)max_m * num_experts > (1LL << 30))
    return MOE_ERR_SHAPE;
  if (fmt != MOE_SCALE_F32 && fmt != MOE_SCALE_UE8M0) return MOE_ERR_UNSUPPORTED;
  if (!masked_m) return MOE_ERR_NULL;
  if (max_m > 0 && (!gate_up || !out || !out_scale)) return MOE_ERR_NULL;
  if (((uintptr_t)gate_up % 16) || ((uintptr_t)out % 16)) return MOE_ERR_ALIGNMENT;
  const int64_t rows = (int64_t)max_m * num_experts;
  if (rows == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t grid = rows < 2048 ? rows : 2048;  // grid-stride over the slab rows
  auto kern = fmt == MOE_SCALE_UE8M0 ? act_quant_kernel<true, false, true>
                                     : act_quant_kernel<false, false, true>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, s, (const uint16_t*)gate_up,
                     masked_m, nullptr, nullptr, rows, inter, num_experts, max_m, nullptr,
                     (uint8_t*)out, (uint8_t*)out_scale);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
  return MOE_OK;
}
