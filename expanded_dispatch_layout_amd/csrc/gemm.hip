// moe_grouped_gemm_fp8: contiguous grouped fp8 GEMM ("NT") over the expanded
// rows, with 1x128 activation scales and 128x128 weight block scales.
//
// Sources: SGLang moe_runner/deep_gemm.py source, _run_contiguous_gemm (the
// gate_up GEMM [rows, 2I] and the down GEMM [rows, H], both bf16 out, rows
// labelled -1 skipped via m_indices; N = w13.size(1)); SGLang PR 37261
// Modifications/Core (the row labels come from the device psum).
//
// gfx950 design:
//  - Workgroup tile BM x 128 (BM = min(align, 128) so a tile never spans two
//    experts), 4 waves; K advances one 128-wide scale block per step, which
//    is exactly one v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 sub-tile.
//  - A and B tiles are staged through LDS (16-byte chunks XOR-swizzled by
//    row so the 16-row fragment reads are bank-conflict free), double
//    buffered with one barrier per K step; global loads for step k+1 are in
//    flight while step k computes.
//  - fp32 scales: each K step's MFMA result is promoted into the fp32
//    accumulator with that row's activation scale times the block's weight
//    scale (the scales do not factor out of the K sum).
//  - UE8M0 scales: the exponent bytes go straight into the MFMA's hardware
//    scale operands (the 1x128 group's byte repeats over its four 32-wide
//    sub-blocks), so the matrix core accumulates the scaled products.
//  - Tiles past the device-side total, or made only of alignment padding,
//    exit before loading anything.  The output tile is staged through LDS
//    and written with 16-byte stores.
#include "common.hpp"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BN = 128;
constexpr int BK = 128;

__device__ __forceinline__ int swz(int row, int chunk) {  // byte offset in a [rows][128] tile
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

template <int BM>
struct Cfg {
  static constexpr int WAVES_M = BM >= 128 ? 2 : 1;
  static constexpr int WAVES_N = 4 / WAVES_M;
  static constexpr int WTM = BM / WAVES_M;
  static constexpr int WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 16;
  static constexpr int FN = WTN / 16;
  static constexpr int A_CHUNKS = BM * 8;  // 16-byte chunks per A tile
  static constexpr int NA = (A_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int NB = BN * 8 / kThreads;
  static constexpr int A_BYTES = BM * BK;
  static constexpr int B_BYTES = BN * BK;
  static constexpr int S_BYTES = BM * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int C_BYTES = BM * BN * 2;
  static constexpr int LDS = (2 * STAGE > C_BYTES) ? 2 * STAGE : C_BYTES;
};

template <int BM, bool kUe8m0>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a, const void* __restrict__ a_scale, const uint8_t* __restrict__ w,
    const void* __restrict__ w_scale, const int32_t* __restrict__ m_indices,
    const int32_t* __restrict__ psum, const int32_t* __restrict__ status, int64_t capacity, int N,
    int K, int E, uint16_t* __restrict__ out) {
  using C = Cfg<BM>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int wm = wid / C::WAVES_N, wn = wid % C::WAVES_N;
  const int KB = K / BK, NBLK = N / BN;
  const int64_t nrows = min((int64_t)status[0], capacity);
  const int n0 = blockIdx.x * BN;
  const int nb = blockIdx.x;

  for (int64_t mt = blockIdx.y; mt * BM < nrows; mt += gridDim.y) {
    const int64_t m0 = mt * BM;
    const int e = m_indices[m0];
    if (e < 0 || e >= E || m0 >= psum[e]) continue;  // uniform per workgroup

    const uint8_t* abase = a + m0 * K;
    const uint8_t* bbase = w + ((int64_t)e * N + n0) * K;
    const float* asf = reinterpret_cast<const float*>(a_scale);
    const uint8_t* asb = reinterpret_cast<const uint8_t*>(a_scale);
    const int64_t wsoff = ((int64_t)e * NBLK + nb) * KB;

    uint4 areg[C::NA], breg[C::NB];
    uint32_t sreg = 0;
    auto gload = [&](int kb) {
#pragma unroll
      for (int i = 0; i < C::NA; ++i) {
        int li = t + i * kThreads;
        if (li < C::A_CHUNKS)
          areg[i] = *reinterpret_cast<const uint4*>(abase + (int64_t)(li >> 3) * K + kb * BK +
                                                    (li & 7) * 16);
      }
#pragma unroll
      for (int i = 0; i < C::NB; ++i) {
        int li = t + i * kThreads;
        breg[i] = *reinterpret_cast<const uint4*>(bbase + (int64_t)(li >> 3) * K + kb * BK +
                                                  (li & 7) * 16);
      }
      if (t < BM) {
        if (kUe8m0) sreg = asb[(m0 + t) * KB + kb];
        else sreg = __float_as_uint(asf[(m0 + t) * KB + kb]);
      }
    };
    auto lstore = [&](int buf) {
      uint8_t* sa = lds + buf * C::STAGE;
      uint8_t* sb = sa + C::A_BYTES;
      uint32_t* ss = reinterpret_cast<uint32_t*>(sb + C::B_BYTES);
#pragma unroll
      for (int i = 0; i < C::NA; ++i) {
        int li = t + i * kThreads;
        if (li < C::A_CHUNKS) *reinterpret_cast<uint4*>(sa + swz(li >> 3, li & 7)) = areg[i];
      }
#pragma unroll
      for (int i = 0; i < C::NB; ++i) {
        int li = t + i * kThreads;
        *reinterpret_cast<uint4*>(sb + swz(li >> 3, li & 7)) = breg[i];
      }
      if (t < BM) ss[t] = sreg;
    };

    v4f acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    gload(0);
    lstore(0);
    __syncthreads();
    const int frow = lane & 15, fk = (lane >> 4) * 2;  // fragment row, first chunk
    for (int kb = 0; kb < KB; ++kb) {
      const int cur = kb & 1;
      if (kb + 1 < KB) gload(kb + 1);
      const uint8_t* sa = lds + cur * C::STAGE;
      const uint8_t* sb = sa + C::A_BYTES;
      const uint32_t* ss = reinterpret_cast<const uint32_t*>(sb + C::B_BYTES);
      v8i bf[C::FN];
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int r = wn * C::WTN + j * 16 + frow;
        uint4 lo = *reinterpret_cast<const uint4*>(sb + swz(r, fk));
        uint4 hi = *reinterpret_cast<const uint4*>(sb + swz(r, fk + 1));
        bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      if constexpr (kUe8m0) {
        const int sbyte = reinterpret_cast<const uint8_t*>(w_scale)[wsoff + kb];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          const int r = wm * C::WTM + i * 16 + frow;
          uint4 lo = *reinterpret_cast<const uint4*>(sa + swz(r, fk));
          uint4 hi = *reinterpret_cast<const uint4*>(sa + swz(r, fk + 1));
          v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          const int abyte = (int)ss[r];
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af, bf[j], acc[i][j], 0, 0, 0, abyte, 0, sbyte);
        }
      } else {
        const float sbv = reinterpret_cast<const float*>(w_scale)[wsoff + kb];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          const int r = wm * C::WTM + i * 16 + frow;
          uint4 lo = *reinterpret_cast<const uint4*>(sa + swz(r, fk));
          uint4 hi = *reinterpret_cast<const uint4*>(sa + swz(r, fk + 1));
          v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          float sc[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int orow = wm * C::WTM + i * 16 + (lane >> 4) * 4 + q;
            sc[q] = __uint_as_float(ss[orow]) * sbv;
          }
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af, bf[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][j][q] += p[q] * sc[q];
          }
        }
      }
      if (kb + 1 < KB) lstore(cur ^ 1);
      __syncthreads();
    }

    // Epilogue: bf16 tile through LDS, then 16-byte row stores.
    uint16_t* ct = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm * C::WTM + i * 16 + (lane >> 4) * 4 + q;
          const int c = wn * C::WTN + j * 16 + (lane & 15);
          ct[r * BN + c] = f32_to_bf16_rne(acc[i][j][q]);
        }
    __syncthreads();
    for (int li = t; li < BM * (BN / 8); li += kThreads) {
      const int r = li / (BN / 8), c8 = li % (BN / 8);
      *reinterpret_cast<uint4*>(out + (m0 + r) * N + n0 + c8 * 8) =
          *reinterpret_cast<const uint4*>(ct + r * BN + c8 * 8);
    }
    __syncthreads();
  }
}

template <int BM>
moe_status launch(const void* a, const void* a_scale, bool ue8m0, const void* w,
                  const void* w_scale, const int32_t* m_indices, const int32_t* psum,
                  const int32_t* status, int64_t capacity, int n, int k, int E, void* out,
                  hipStream_t s) {
  const int64_t mtiles = capacity / BM;
  const unsigned gy = (unsigned)(mtiles > 65535 ? 65535 : mtiles);
  dim3 grid(n / BN, gy);
  if (ue8m0)
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, true>), grid, dim3(kThreads), 0, s,
                       (const uint8_t*)a, a_scale, (const uint8_t*)w, w_scale, m_indices, psum,
                       status, capacity, n, k, E, (uint16_t*)out);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, false>), grid, dim3(kThreads), 0, s,
                       (const uint8_t*)a, a_scale, (const uint8_t*)w, w_scale, m_indices, psum,
                       status, capacity, n, k, E, (uint16_t*)out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_grouped_gemm_fp8(const void* a, const void* a_scale, moe_scale_fmt fmt,
                                           const void* w, const void* w_scale,
                                           const int32_t* m_indices, const int32_t* psum,
                                           const int32_t* status, int64_t capacity, int n, int k,
                                           int num_experts, int align, void* out, void* stream) {
  if (capacity < 0 || capacity > (1LL << 30) || n <= 0 || k <= 0 || n % BN || k % BK ||
      num_experts < 1 || num_experts > MOE_MAX_EXPERTS)
    return MOE_ERR_SHAPE;
  if (align < MOE_MIN_ALIGN || align > MOE_MAX_ALIGN || (align & (align - 1)))
    return MOE_ERR_UNSUPPORTED;
  if (capacity % align != 0) return MOE_ERR_SHAPE;
  if (fmt != MOE_SCALE_F32 && fmt != MOE_SCALE_UE8M0) return MOE_ERR_UNSUPPORTED;
  if (!m_indices || !psum || !status || !w || !w_scale) return MOE_ERR_NULL;
  if (capacity > 0 && (!a || !a_scale || !out)) return MOE_ERR_NULL;
  if (((uintptr_t)a % 16) || ((uintptr_t)w % 16) || ((uintptr_t)out % 16))
    return MOE_ERR_ALIGNMENT;
  if (capacity == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool ue = fmt == MOE_SCALE_UE8M0;
  if (align >= 128)
    return launch<128>(a, a_scale, ue, w, w_scale, m_indices, psum, status, capacity, n, k,
                       num_experts, out, s);
  if (align == 64)
    return launch<64>(a, a_scale, ue, w, w_scale, m_indices, psum, status, capacity, n, k,
                      num_experts, out, s);
  if (align == 32)
    return launch<32>(a, a_scale, ue, w, w_scale, m_indices, psum, status, capacity, n, k,
                      num_experts, out, s);
  return launch<16>(a, a_scale, ue, w, w_scale, m_indices, psum, status, capacity, n, k,
                    num_experts, out, s);
}
