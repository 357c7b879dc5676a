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
//    chunks of every 128-byte row are XOR-swizzled by row (swz), chosen per
//    lane on the global side, so the 16-row fragment reads are bank-conflict
//    free.
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

// Physical 16-byte chunk of logical chunk c in row r of a [rows][128 B] tile:
// c ^ key(r), key(r) = (r & 7) ^ ((r >> 3) & 1).  A fragment read serves 16
// consecutive rows (an aligned 16) at one logical chunk.  The key is a
// permutation of the 8 chunks over any aligned 8 rows (conflict-free when 8
// lanes are served per cycle over 32 banks), and over the 8 even (odd) rows
// of an aligned 16 (conflict-free when 16 lanes are served over 64 banks,
// where rows r and r+8 share banks).  It depends only on r mod 16, so every
// fragment of a wave is one per-lane base plus a compile-time offset.
__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) {  // byte offset in a [rows][128] tile
  return row * 128 + ((chunk ^ swz_key(row)) << 4);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(size_t)(__attribute__((address_space(3))) const void*)p);
}

// Direct HBM -> LDS loads.  Issued from inline assembly so the compiler does
// not treat them as LDS writes that every later LDS read must wait for: the
// kernel orders them itself (vmcnt waits + s_barrier).  Address = 64-bit
// scalar base + 32-bit per-lane offset; lane i's data lands at lds + i * size.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
               "s"(lds)
               : "memory");
}
__device__ __forceinline__ void dma4(const uint8_t* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base),
               "s"(lds)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wait until at most n of this wave's vector-memory operations are
// outstanding (n is wave-uniform; s_waitcnt takes an immediate).
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    default: wait_vmcnt<LOADS_PER_STAGE>(); break;
  }
}

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

// Per-lane byte offsets of one item's loads, fixed over its K steps.
struct LoadOffsets {
  uint32_t a[A_LOADS];  // from it.a (+ kb * BK)
  uint32_t b[B_LOADS];  // from it.b (+ kb * BK)
  int scale_row;        // activation row whose scale this lane loads
};

__device__ __forceinline__ LoadOffsets load_offsets(const Item& it, int lane, int wid) {
  LoadOffsets o;
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    const int r = (wid * A_LOADS + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz_key(r);
    const int rr = r < it.live ? r : it.live - 1;  // reload the last live row
    o.a[j] = (uint32_t)rr * (uint32_t)it.K + (uint32_t)c * 16u;
  }
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    const int r = (wid * B_LOADS + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz_key(r);
    o.b[j] = (uint32_t)r * (uint32_t)it.K + (uint32_t)c * 16u;
  }
  const int r = wid * 64 + lane;
  o.scale_row = r < it.live ? r : it.live - 1;
  return o;
}

// Issue the direct-to-LDS loads of K step kb into `stage`.  A wave skips the
// activation loads whose 8 rows are all alignment padding (rows past the
// live rows inside a loaded 8-row block reload the last live row); the number
// of loads a wave issues per stage is the same for every stage of an item
// (stage_loads), which is what its vmcnt waits count on.
__device__ __forceinline__ void issue_stage(const Item& it, const LoadOffsets& o, uint8_t* stage,
                                            int kb, int wid) {
#ifdef PROBE_NO_LOADS
  return;
#endif
  const uint8_t* abase = it.a + kb * BK;
  const uint8_t* bbase = it.b + kb * BK;
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    const int base = (wid * A_LOADS + j) * 8;  // 8 rows per wave instruction
    if (base >= it.live) break;                // only padding rows: not loaded
    dma16(abase, o.a[j], lds_addr(stage + base * 128));
  }
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    const int base = (wid * B_LOADS + j) * 8;
    dma16(bbase, o.b[j], lds_addr(stage + A_BYTES + base * 128));
  }
  // Scales: the aligned dword holding each element (UE8M0 bytes are picked
  // out of it when used).  Waves 0-3: one activation row each lane; waves
  // 4-7: a copy of the weight block scale.
  if (wid < 4) {
    const int64_t off = (it.as0 + (int64_t)o.scale_row * it.KB + kb) * it.sbytes;
    dma4(it.as, (uint32_t)(off & ~(int64_t)3), lds_addr(stage + A_BYTES + B_BYTES + wid * 256));
  } else {
    const int64_t boff = ((it.bs0 + kb) * it.sbytes) & ~(int64_t)3;
    dma4(it.bs + boff, 0u, lds_addr(stage + A_BYTES + B_BYTES + SA_BYTES + (wid - 4) * 256));
  }
}

// Per-lane LDS byte offsets (within a stage) of the two 16-byte halves of
// this lane's A and B fragments for row/column tile 0; tile i adds i * 2048.
struct FragOffsets {
  int a_lo, a_hi, b_lo, b_hi, s_row;
};

__device__ __forceinline__ FragOffsets frag_offsets(int lane, int wm, int wn) {
  const int frow = lane & 15, fk = (lane >> 4) * 2;
  FragOffsets f;
  const int ra = wm * WTM + frow, rb = wn * WTN + frow;
  f.a_lo = swz(ra, fk);
  f.a_hi = swz(ra, fk + 1);
  f.b_lo = A_BYTES + swz(rb, fk);
  f.b_hi = A_BYTES + swz(rb, fk + 1);
  f.s_row = wm * WTM + (lane >> 4) * 4;  // first output row of this lane
  return f;
}

__device__ __forceinline__ v8i frag2(const uint8_t* stage, int lo_off, int hi_off) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4 lo = *reinterpret_cast<const u4*>(stage + lo_off);
  const u4 hi = *reinterpret_cast<const u4*>(stage + hi_off);
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
             (int)hi[3]};
}

__device__ __forceinline__ v4f mfma_plain(const v8i& a, const v8i& b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                          127, 0, 127);
}

// NFM: how many of the wave's four 16-row tiles hold live rows.
template <bool kUe8m0, int NFM>
__device__ __forceinline__ void compute_stage(const uint8_t* stage, v4f (&acc)[FM][FN],
                                              const Item& it, const FragOffsets& fo, int kb,
                                              int lane, int nfm_rt) {
#ifdef PROBE_NO_COMPUTE
  return;
#endif
  const uint32_t* ssa = reinterpret_cast<const uint32_t*>(stage + A_BYTES + B_BYTES);
  const uint32_t* ssb = reinterpret_cast<const uint32_t*>(stage + A_BYTES + B_BYTES + SA_BYTES);
  v8i bf[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) bf[j] = frag2(stage + j * 2048, fo.b_lo, fo.b_hi);
  if constexpr (kUe8m0) {
    const int sbyte = (int)((ssb[0] >> (8 * (int)((it.bs0 + kb) & 3))) & 0xffu);
    const int arow = fo.s_row - (lane >> 4) * 4 + (lane & 15);  // this lane's A row
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i >= nfm_rt) break;  // uniform per wave
      const int r = arow + i * 16;
      const v8i af = frag2(stage + i * 2048, fo.a_lo, fo.a_hi);
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
    if constexpr (NFM > 0) {
      const v8i af = frag2(stage, fo.a_lo, fo.a_hi);
#pragma unroll
      for (int j = 0; j < FN; ++j) p[0][j] = mfma_plain(af, bf[j]);
    }
#pragma unroll
    for (int i = 0; i < NFM; ++i) {
      if (i + 1 < NFM) {
        const v8i af = frag2(stage + (i + 1) * 2048, fo.a_lo, fo.a_hi);
#pragma unroll
        for (int j = 0; j < FN; ++j) p[(i + 1) & 1][j] = mfma_plain(af, bf[j]);
      }
      float sc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) sc[q] = __uint_as_float(ssa[fo.s_row + i * 16 + q]) * sbv;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] += p[i & 1][j][q] * sc[q];
    }
  }
}

// The K loop of one item: wait for stage kb (this wave's loads; the barrier
// makes every wave's visible and retires the stage read one step ago), refill
// that older stage with step kb+2, compute on stage kb.
template <bool kUe8m0, int NFM>
__device__ __forceinline__ void kloop(uint8_t* lds, v4f (&acc)[FM][FN], const Item& it,
                                      const LoadOffsets& lo_, const FragOffsets& fo, int lane,
                                      int wid, int nfm, int stage_loads) {
  for (int kb = 0; kb < it.KB; ++kb) {
    if (kb + 1 < it.KB) wait_vmcnt_rt(stage_loads);
    else wait_vmcnt<0>();
    barrier();
    if (kb + 2 < it.KB) issue_stage(it, lo_, lds + ((kb + 2) % kStages) * STAGE, kb + 2, wid);
    if (NFM > 0 || (kUe8m0 && nfm > 0))
      compute_stage<kUe8m0, NFM>(lds + (kb % kStages) * STAGE, acc, it, fo, kb, lane, nfm);
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
  const FragOffsets fo = frag_offsets(lane, wm, wn);
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
    // Live 16-row MFMA tiles of this wave, and the loads it issues per stage.
    const int nfm = (int)max(0, min(FM, (it.live - wm * WTM + 15) / 16));
    const int na = (int)max(0, min(A_LOADS, (it.live - wid * A_LOADS * 8 + 7) / 8));
    const int stage_loads = na + B_LOADS + 1;

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const LoadOffsets lo_ = load_offsets(it, lane, wid);
    wait_vmcnt<0>();  // nothing older (previous item's stores) left in flight
    issue_stage(it, lo_, lds, 0, wid);
    if (KB > 1) issue_stage(it, lo_, lds + STAGE, 1, wid);
    if constexpr (kUe8m0) {
      kloop<true, FM>(lds, acc, it, lo_, fo, lane, wid, nfm, stage_loads);
    } else {
      switch (nfm) {  // uniform per wave; one K loop per live-tile count
        case 4: kloop<false, 4>(lds, acc, it, lo_, fo, lane, wid, 4, stage_loads); break;
        case 3: kloop<false, 3>(lds, acc, it, lo_, fo, lane, wid, 3, stage_loads); break;
        case 2: kloop<false, 2>(lds, acc, it, lo_, fo, lane, wid, 2, stage_loads); break;
        case 1: kloop<false, 1>(lds, acc, it, lo_, fo, lane, wid, 1, stage_loads); break;
        default: kloop<false, 0>(lds, acc, it, lo_, fo, lane, wid, 0, stage_loads); break;
      }
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
