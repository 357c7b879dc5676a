// moe_grouped_gemm_fp8: contiguous grouped fp8 GEMM ("NT") over the expanded
// rows, with 1x128 activation scales and 128x128 weight block scales.
//
// Sources: SGLang moe_runner/deep_gemm.py source, _run_contiguous_gemm (the
// gate_up GEMM [rows, 2I] and the down GEMM [rows, H], both bf16 out, rows
// labelled -1 skipped via m_indices; N = w13.size(1)); SGLang PR 37261
// Modifications/Core (the row labels come from the device psum).
//
// gfx950 design:
//  - Work item = (expert, group of up to 256 of its expanded rows, 128-wide N
//    tile).  A group never spans two experts, so one weight tile serves it;
//    when an expert has at most 256 rows (the DeepSeek-V3-shape share) its
//    weight slab is streamed from HBM exactly once.
//  - Persistent grid, one workgroup per CU, walking the items of the
//    device-side layout (read from psum, no host sync).  Items are numbered
//    group-major, so the 32..56 N tiles of one row group are consecutive and
//    land on one XCD (dispatch is round-robin over the 8 XCDs): that XCD keeps
//    the group's activations in its L2 while it streams the expert's weights.
//  - K advances one 128-wide scale block per step = one
//    v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 sub-tile.  Four waves in a
//    2x2 grid, each owning 128 x 64 outputs (8 x 4 MFMA tiles).
//  - Operands go HBM -> LDS directly (global_load_lds_dwordx4), three LDS
//    stages, two K steps in flight; each wave waits only for its own oldest
//    stage (explicit vmcnt) and a bare s_barrier publishes it.  The 16-byte
//    chunks of every 128-byte row are XOR-swizzled by row, chosen per lane on
//    the global side, so the 16-row fragment reads are bank-conflict free.
//  - fp32 scales: each step's MFMA result is promoted into the fp32
//    accumulator with the row's activation scale times the block's weight
//    scale (the scales do not factor out of the K sum).
//  - UE8M0 scales: the exponent bytes are the MFMA's hardware scale operands
//    (the group's byte repeats over its four 32-wide sub-blocks), so the
//    matrix core accumulates the scaled products directly.
//  - The bf16 output tile is staged through LDS and written with 16-byte
//    stores; rows past the group are never written.
#include "common.hpp"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;  // 8 waves: 2 per SIMD
constexpr int kWaves = kThreads / 64;
constexpr int kXcds = 8;       // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr int GM = 256;        // rows per work item
constexpr int BN = 128;
constexpr int BK = 128;
constexpr int kStages = 3;
constexpr int WAVES_N = 2;
constexpr int WTM = 64, WTN = 64;            // wave tile: 4 x 2 waves cover 256 x 128
constexpr int FM = WTM / 16, FN = WTN / 16;  // 4 x 4 MFMA tiles per wave
constexpr int A_BYTES = GM * BK;             // 32 KB
constexpr int B_BYTES = BN * BK;             // 16 KB
constexpr int SA_BYTES = GM * 4;             // one scale dword per row
constexpr int SB_BYTES = 4 * 64 * 4;         // four copies of the block scale
constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
constexpr int LDS_BYTES = kStages * STAGE;   // 150 KB of the CU's 160 KB
constexpr int A_LOADS = A_BYTES / (kThreads * 16);  // 16-byte loads per lane per stage
constexpr int B_LOADS = B_BYTES / (kThreads * 16);
constexpr int LOADS_PER_STAGE = A_LOADS + B_LOADS + 1;  // + one scale dword
static_assert(GM * BN * 2 <= LDS_BYTES, "output tile must fit in LDS");
static_assert(kWaves * 64 == 2 * GM, "scale loads: waves 0-3 A rows, 4-7 block scale");

__device__ __forceinline__ int swz(int row, int chunk) {  // byte offset in a [rows][128] tile
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(size_t)(__attribute__((address_space(3))) const void*)p);
}

// Direct HBM -> LDS loads.  Issued from inline assembly so the compiler does
// not treat them as LDS writes that every later LDS read must wait for: the
// kernel orders them itself (vmcnt waits + s_barrier).  Lane i's data lands
// at lds + i * size.
__device__ __forceinline__ void dma16(const uint8_t* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory");
}
__device__ __forceinline__ void dma4(const uint8_t* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

struct Item {
  const uint8_t* a;     // first row of the group
  const uint8_t* b;     // first weight row of the N tile
  const uint8_t* as;    // activation scale array (4-byte aligned base)
  const uint8_t* bs;    // weight scale array (4-byte aligned base)
  int64_t as0;          // element index of the group's first row's scales
  int64_t bs0;          // element index of (expert, N tile, k block 0)
  int live;             // rows of the group that hold a slot (1..GM); the
                        // rest of the group is alignment padding
  int KB;               // K / 128
  int K;
  int sbytes;           // 4 (fp32) or 1 (UE8M0)
};

// Issue the direct-to-LDS loads of K step kb into `stage`.  Every wave issues
// exactly LOADS_PER_STAGE instructions (rows past the live rows reload the
// last live row) so the vmcnt bookkeeping is the same for all waves.
__device__ __forceinline__ void issue_stage(const Item& it, uint8_t* stage, int kb, int lane,
                                            int wid) {
#ifdef PROBE_NO_LOADS
  return;
#endif
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    const int base = (wid * A_LOADS + j) * 8;  // 8 rows per wave instruction
    const int r = base + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    const int rr = r < it.live ? r : it.live - 1;
    dma16(it.a + (int64_t)rr * it.K + kb * BK + c * 16, lds_addr(stage + base * 128));
  }
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    const int base = (wid * B_LOADS + j) * 8;
    const int r = base + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    dma16(it.b + (int64_t)r * it.K + kb * BK + c * 16, lds_addr(stage + A_BYTES + base * 128));
  }
  // Scales: the aligned dword holding each element (UE8M0 bytes are picked
  // out of it when used).  Waves 0-3: one activation row each lane; waves
  // 4-7: a copy of the weight block scale.
  if (wid < 4) {
    const int r = wid * 64 + lane;
    const int rr = r < it.live ? r : it.live - 1;
    const int64_t off = (it.as0 + (int64_t)rr * it.KB + kb) * it.sbytes;
    dma4(it.as + (off & ~(int64_t)3), lds_addr(stage + A_BYTES + B_BYTES + wid * 256));
  } else {
    const int64_t boff = (it.bs0 + kb) * it.sbytes;
    dma4(it.bs + (boff & ~(int64_t)3),
         lds_addr(stage + A_BYTES + B_BYTES + SA_BYTES + (wid - 4) * 256));
  }
}

__device__ __forceinline__ v8i frag(const uint8_t* tile, int r, int fk) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4 lo = *reinterpret_cast<const u4*>(tile + swz(r, fk));
  const u4 hi = *reinterpret_cast<const u4*>(tile + swz(r, fk + 1));
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
             (int)hi[3]};
}

__device__ __forceinline__ v4f mfma_plain(const v8i& a, const v8i& b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                          127, 0, 127);
}

template <bool kUe8m0>
__device__ __forceinline__ void compute_stage(const uint8_t* stage, v4f (&acc)[FM][FN],
                                              const Item& it, int kb, int lane, int wm,
                                              int wn) {
#ifdef PROBE_NO_COMPUTE
  return;
#endif
  const uint8_t* sa = stage;
  const uint8_t* sb = stage + A_BYTES;
  const uint32_t* ssa = reinterpret_cast<const uint32_t*>(stage + A_BYTES + B_BYTES);
  const uint32_t* ssb = reinterpret_cast<const uint32_t*>(stage + A_BYTES + B_BYTES + SA_BYTES);
  const int frow = lane & 15, fk = (lane >> 4) * 2;
  const int r0 = wm * WTM;
  v8i bf[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) bf[j] = frag(sb, wn * WTN + j * 16 + frow, fk);
  if constexpr (kUe8m0) {
    const int sbyte = (int)((ssb[0] >> (8 * (int)((it.bs0 + kb) & 3))) & 0xffu);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = r0 + i * 16 + frow;
      const v8i af = frag(sa, r, fk);
      const int apos = (int)((it.as0 + (int64_t)r * it.KB + kb) & 3);
      const int abyte = (int)((ssa[r] >> (8 * apos)) & 0xffu);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 0, 0,
                                                                     0, abyte, 0, sbyte);
    }
  } else {
    // Software pipeline: the MFMAs of row tile i+1 are issued before the
    // promotion of row tile i, so the matrix core always has work queued
    // while the VALU scales and accumulates.
    const float sbv = __uint_as_float(ssb[0]);
    v4f p[2][FN];
    {
      const v8i af = frag(sa, r0 + frow, fk);
#pragma unroll
      for (int j = 0; j < FN; ++j) p[0][j] = mfma_plain(af, bf[j]);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i + 1 < FM) {
        const v8i af = frag(sa, r0 + (i + 1) * 16 + frow, fk);
#pragma unroll
        for (int j = 0; j < FN; ++j) p[(i + 1) & 1][j] = mfma_plain(af, bf[j]);
      }
      float sc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sc[q] = __uint_as_float(ssa[r0 + i * 16 + (lane >> 4) * 4 + q]) * sbv;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] += p[i & 1][j][q] * sc[q];
    }
  }
}

template <bool kUe8m0>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_scale,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_scale,
    const int32_t* __restrict__ psum, const int32_t* __restrict__ status, int64_t capacity, int N,
    int K, int E, int align, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  __shared__ int gp[MOE_MAX_EXPERTS + 1];  // prefix of row groups per expert
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int64_t nrows = min((int64_t)status[0], capacity);
  const int sbytes = kUe8m0 ? 1 : 4;
  const int KB = K / BK, NT = N / BN;

  // Row groups: expert e's block [start_e, end_e) (clamped to the valid rows)
  // is cut into ceil(len / GM) groups.
  if (wid == 0) {
    int run = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      int ng = 0;
      if (e < E) {
        const int64_t st = e ? align_up_i(psum[e - 1], align) : 0;
        const int64_t en = min((int64_t)align_up_i(psum[e], align), nrows);
        ng = en > st ? (int)((en - st + GM - 1) / GM) : 0;
      }
      const int incl = wave_incl_scan_i(ng);
      if (e < E) gp[e] = run + incl - ng;
      run += __shfl(incl, 63, 64);
    }
    if (lane == 0) gp[E] = run;
  }
  __syncthreads();
  const int64_t nitems = (int64_t)gp[E] * NT;
  const int per_xcd = gridDim.x / kXcds;
  const int64_t slot = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;

  for (int64_t item = slot; item < nitems; item += gridDim.x) {
    const int gi = (int)(item / NT), nt = (int)(item % NT);
    int lo = 0, hi = E - 1;  // expert of group gi: last e with gp[e] <= gi
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (gp[mid] <= gi) lo = mid;
      else hi = mid - 1;
    }
    const int e = lo;
    const int64_t st = e ? align_up_i(psum[e - 1], align) : 0;
    const int64_t m0 = st + (int64_t)(gi - gp[e]) * GM;
    const int64_t live = min((int64_t)GM, min((int64_t)psum[e], nrows) - m0);
    if (live <= 0) continue;  // only alignment padding: nothing to compute
    Item it;
    it.live = (int)live;
    it.K = K;
    it.KB = KB;
    it.sbytes = sbytes;
    it.a = a + m0 * K;
    it.b = w + ((int64_t)e * N + (int64_t)nt * BN) * K;
    it.as = a_scale;
    it.bs = w_scale;
    it.as0 = m0 * KB;
    it.bs0 = ((int64_t)e * NT + nt) * KB;
    const bool active = wm * WTM < it.live;  // this wave's rows hold slots

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    wait_vmcnt<0>();  // nothing older (previous item's stores) left in flight
    issue_stage(it, lds, 0, lane, wid);
    if (KB > 1) issue_stage(it, lds + STAGE, 1, lane, wid);
    for (int kb = 0; kb < KB; ++kb) {
      if (kb + 1 < KB) wait_vmcnt<LOADS_PER_STAGE>();
      else wait_vmcnt<0>();
      barrier();  // stage kb landed for every wave; stage kb-1 fully consumed
      if (kb + 2 < KB) issue_stage(it, lds + ((kb + 2) % kStages) * STAGE, kb + 2, lane, wid);
      if (active)
        compute_stage<kUe8m0>(lds + (kb % kStages) * STAGE, acc, it, kb, lane, wm, wn);
    }
    barrier();  // every wave is done reading the stages

    // Epilogue: bf16 tile through LDS, then 16-byte stores of the live rows.
    uint16_t* ct = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm * WTM + i * 16 + (lane >> 4) * 4 + q;
          const int c = wn * WTN + j * 16 + (lane & 15);
          ct[r * BN + c] = f32_to_bf16_rne(acc[i][j][q]);
        }
    __syncthreads();
    uint16_t* obase = out + m0 * N + (int64_t)nt * BN;
    for (int li = t; li < it.live * (BN / 8); li += kThreads) {
      const int r = li / (BN / 8), c8 = li % (BN / 8);
      *reinterpret_cast<u32x4*>(obase + (int64_t)r * N + c8 * 8) =
          *reinterpret_cast<const u32x4*>(ct + r * BN + c8 * 8);
    }
    __syncthreads();
  }
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_grouped_gemm_fp8(const void* a, const void* a_scale, moe_scale_fmt fmt,
                                           const void* w, const void* w_scale, const int32_t* psum,
                                           const int32_t* status, int64_t capacity, int n, int k,
                                           int num_experts, int align, void* out, void* stream) {
  if (capacity < 0 || capacity > (1LL << 30) || n <= 0 || k <= 0 || n % BN || k % BK ||
      num_experts < 1 || num_experts > MOE_MAX_EXPERTS)
    return MOE_ERR_SHAPE;
  if (align < MOE_MIN_ALIGN || align > MOE_MAX_ALIGN || (align & (align - 1)))
    return MOE_ERR_UNSUPPORTED;
  if (capacity % align != 0) return MOE_ERR_SHAPE;
  if (fmt != MOE_SCALE_F32 && fmt != MOE_SCALE_UE8M0) return MOE_ERR_UNSUPPORTED;
  if (!psum || !status || !w || !w_scale) return MOE_ERR_NULL;
  if (capacity > 0 && (!a || !a_scale || !out)) return MOE_ERR_NULL;
  if (((uintptr_t)a % 16) || ((uintptr_t)w % 16) || ((uintptr_t)out % 16) ||
      ((uintptr_t)a_scale % 4) || ((uintptr_t)w_scale % 4))
    return MOE_ERR_ALIGNMENT;
  if (capacity == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // One workgroup per CU (the kernel uses ~154 KB of LDS), a whole number per
  // XCD, never more than the largest possible number of work items.
  const int64_t max_items = ((capacity + GM - 1) / GM + num_experts) * (int64_t)(n / BN);
  int64_t grid = device_cus();
  if (grid > max_items) grid = max_items;
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  if (fmt == MOE_SCALE_UE8M0)
    hipLaunchKernelGGL((grouped_gemm_kernel<true>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                       (const uint8_t*)a, (const uint8_t*)a_scale, (const uint8_t*)w,
                       (const uint8_t*)w_scale, psum, status, capacity, n, k, num_experts, align,
                       (uint16_t*)out);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<false>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                       (const uint8_t*)a, (const uint8_t*)a_scale, (const uint8_t*)w,
                       (const uint8_t*)w_scale, psum, status, capacity, n, k, num_experts, align,
                       (uint16_t*)out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}
