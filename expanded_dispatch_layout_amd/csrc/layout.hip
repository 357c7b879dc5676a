// moe_expand_layout: received fp8 tokens -> per-(token, expert) rows grouped
// by expert, each expert block padded to `align` rows, with row labels, the
// slot->row map and the expand-mode prefix sum.  No host synchronisation.
//
// Sources: SGLang PR 37261 "expanded (do_expand=True) prefill dispatch for
// DeepEP-V2" (Modifications/Core: row labels from the device psum; review
// thread: psum[e] = align(psum[e-1]) + count[e], total = align(psum[E-1]));
// vLLM PR 54109 PaddedStandard (Motivation/Design: -1 slots, device-side
// real/padding boundary, zeroed alignment gaps).
//
// Small receive buffers (rows * topk <= 65536 slots, at most 8 local
// experts, rows copied as they are: the DeepSeek-V3-shape share, the padded
// buffer, the decode share): ONE launch.  Every 1024-thread workgroup reads
// the buffer's ids itself (128 KB at the DeepSeek-V3 share; the first pass
// of loads is issued before the valid-row bound arrives) and counts, per
// expert, the valid slots and those before its own 16-row group in 7-bit
// per-thread fields, summed over each wave by a DPP transpose-reduce; it
// requests its first row's data, scans the counts into the aligned starts
// and psum (workgroup 0 writes them and the status) and scatters its group,
// a wave per row.
//
// Larger buffers: up to three kernels on one stream (two when the block
// table is small: every scatter workgroup then scans it itself):
//  1. count   a block covers G = 16 16-row groups; its threads read the
//             block's (row, k) ids coalesced, all loads in flight at once.
//             Order-free per-expert counts of every group (LDS atomics), then, per
//             expert, the exclusive offset of each group within the block
//             and the block's total -> workspace.
//  2. scan    one workgroup: per-expert exclusive scan over the block totals
//             (a few per expert), then the expert starts as the exclusive
//             scan of the aligned counts (every start is aligned, so
//             start[e] = sum of align(count) over e' < e), psum, total,
//             flags.
//  3. scatter 768 workgroups, each wave walking received rows grid-stride,
//             software-pipelined: while one row is stored, the next row's
//             data and the ids of the row after are in flight.
// Either way the scatter works the same on a row: the stable rank of slot
// (r, k) among its expert's slots is its block's (or, fused, the rows
// before the group's) count plus its group's offset in the block plus the
// number of that expert's slots in the earlier rows of the group plus those
// at k' < k in row r: two ballots over the group's ids.  Destination =
// start[e] + rank; the row (16-byte chunks) and its scales are read once and
// written to each destination.  The same grid zero-fills the alignment pad
// rows and writes the row labels (grid-stride), so no extra pass is needed.
// Rows at or past the valid-row boundary are never read as routing: their
// ids are either not loaded or loaded with their neighbours and ignored, and
// their slots get -1.
//
// bf16 input (the standard path, SGLang moe_runner/deep_gemm.py source,
// pre_permute_standard_to_deep_gemm: per-token-group quantisation, then the
// scatter): the same kernels; the scatter reads each bf16 row once,
// quantises it per 1x128 group in registers (16 lanes per group, max by
// xor-shuffles) and writes the codes and the group scales to every
// destination, so the quantised rows never make a round trip through HBM.
// With MOE_SCALE_NONE (bf16 weights) the bf16 rows are copied as they are
// (the fp8 byte-copy scatter over rows of 2 * H bytes, no scales).
//
// MXFP8 (SGLang moe_runner/deep_gemm.py source, DeepGemmMoeQuantInfo: block
// shape [1, 32], UE8M0 scales): the received scales are one byte per 1x32
// group; the scatter copies each 128-wide block's four bytes as one 4-byte
// word, K-block-major like the other formats' scales.
#include <algorithm>
#include <mutex>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kGroupRows = 16;      // rows per counted group
constexpr int kCountThreads = 256;  // one row per thread: 16 groups per block
constexpr int kScanThreads = 1024;
constexpr int kScatterThreads = 256;
constexpr int kFusedThreads = 1024;  // fused layout: a wave per row of a 16-row group

// Groups per count block (the [groups][E] count table stays in LDS).
__host__ __device__ inline int groups_per_block(int) { return kCountThreads / kGroupRows; }
constexpr int kFoldScanInts = 4096;  // block table size up to which the scatter scans it
constexpr int64_t kFusedSlots = 65536;  // receive-buffer slots up to which no count kernel runs

struct Workspace {
  int32_t* grp;       // [ngroups][E]: offset of each group within its block
  int32_t* blk;       // [nblocks][E]: block totals, then exclusive block offsets
  int32_t* blk_flag;  // [nblocks]
  int32_t* starts;    // [E]
  int32_t* padbase;   // [E + 1] exclusive prefix of pad rows per expert
};

__host__ __device__ inline int64_t num_groups(int64_t rows) {
  return (rows + kGroupRows - 1) / kGroupRows;
}
__host__ __device__ inline int64_t num_blocks(int64_t rows, int E) {
  const int64_t br = (int64_t)groups_per_block(E) * kGroupRows;
  return (rows + br - 1) / br;
}

__host__ __device__ inline size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

__host__ __device__ inline size_t workspace_bytes(int64_t rows, int E) {
  const int64_t ng = num_groups(rows), nb = num_blocks(rows, E);
  return round256(size_t(ng) * E * 4) + round256(size_t(nb) * E * 4) + round256(size_t(nb) * 4) +
         round256(size_t(E) * 4) + round256(size_t(E + 1) * 4);
}

__host__ __device__ inline Workspace carve(void* base, int64_t rows, int E) {
  const int64_t ng = num_groups(rows), nb = num_blocks(rows, E);
  char* p = (char*)base;
  Workspace w;
  w.grp = (int32_t*)p;
  p += round256(size_t(ng) * E * 4);
  w.blk = (int32_t*)p;
  p += round256(size_t(nb) * E * 4);
  w.blk_flag = (int32_t*)p;
  p += round256(size_t(nb) * 4);
  w.starts = (int32_t*)p;
  p += round256(size_t(E) * 4);
  w.padbase = (int32_t*)p;
  return w;
}

__global__ __launch_bounds__(kCountThreads) void expand_count_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ psum_rank, int nsrc,
    int64_t rows, int topk, int E, int G, int64_t ngroups, int32_t* __restrict__ grp,
    int32_t* __restrict__ blk, int32_t* __restrict__ blk_flag) {
  extern __shared__ int32_t cnt[];  // [G][E]
  __shared__ int lflag;
  const int t = threadIdx.x;
  // The block's ids, slot i * 256 + t of its (row, k) slots per thread: read
  // coalesced, every load issued before any is used.
  const int64_t r0 = (int64_t)blockIdx.x * G * kGroupRows;
  const int nslots = (int)min((int64_t)G * kGroupRows, rows - r0) * topk;
  const int32_t* bids = ids + r0 * topk;
  int idv[MOE_MAX_TOPK];
#pragma unroll
  for (int i = 0; i < MOE_MAX_TOPK; ++i) {
    const int sl = i * kCountThreads + t;
    idv[i] = (i < topk && sl < nslots) ? bids[sl] : -1;
  }
  const int64_t nv = valid_rows(psum_rank, nsrc, rows);
  for (int i = t; i < G * E; i += kCountThreads) cnt[i] = 0;
  if (t == 0) lflag = 0;
  __syncthreads();
  // Rows of the block below the valid-row boundary.
  const int nvb = (int)max((int64_t)0, min(nv - r0, (int64_t)G * kGroupRows));
  int bad = 0;
#pragma unroll
  for (int i = 0; i < MOE_MAX_TOPK; ++i) {
    if (i < topk) {
      const int lr = (i * kCountThreads + t) / topk;  // row within the block
      const int e = idv[i];
      if (lr < nvb) {
        if (e >= E) bad = 1;
        else if (e >= 0) atomicAdd(&cnt[(lr / kGroupRows) * E + e], 1);
      }
    }
  }
  if (bad) atomicOr(&lflag, MOE_FLAG_EXPERT_ID_RANGE);
  __syncthreads();
  // Each group's exclusive offset within the block per expert (group order
  // preserved), and the block total.  Few experts: one wave per expert, lane
  // = group (G <= 64).  Many: one thread per expert walks the G groups in
  // order (a wave per expert would run E / 4 scans one after another).
  const int lane = t & 63, wid = t >> 6;
  const int64_t g0 = (int64_t)blockIdx.x * G;
  if (E <= 32) {
    for (int e = wid; e < E; e += kCountThreads / 64) {
      const int c = lane < G ? cnt[lane * E + e] : 0;
      const int incl = wave_incl_scan_i(c);
      if (lane < G && g0 + lane < ngroups) grp[(g0 + lane) * E + e] = incl - c;
      if (lane == 63) blk[(int64_t)blockIdx.x * E + e] = incl;
    }
  } else {
    for (int e = t; e < E; e += kCountThreads) {
      int run = 0;
      for (int g = 0; g < G; ++g) {
        const int c = cnt[g * E + e];
        if (g0 + g < ngroups) grp[(g0 + g) * E + e] = run;
        run += c;
      }
      blk[(int64_t)blockIdx.x * E + e] = run;
    }
  }
  if (t == 0) blk_flag[blockIdx.x] = lflag;
}

// Exclusive scan over the whole 1024-thread workgroup; returns the exclusive
// prefix of v and writes the total to *total (all threads).
__device__ int block_excl_scan(int v, int* lds16, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int incl = wave_incl_scan_i(v);
  if (lane == 63) lds16[wid] = incl;
  __syncthreads();
  int wsum = (lane < kScanThreads / 64) ? lds16[lane] : 0;
  int wincl = wave_incl_scan_i(wsum);
  int wbase = __shfl(wincl - wsum, wid, 64);
  *total = __shfl(wincl, kScanThreads / 64 - 1, 64);
  __syncthreads();
  return wbase + incl - v;
}

__global__ __launch_bounds__(kScanThreads) void expand_scan_kernel(
    int32_t* __restrict__ blk, const int32_t* __restrict__ blk_flag, int64_t nblocks, int E,
    int align, int64_t capacity, int32_t* __restrict__ starts, int32_t* __restrict__ padbase,
    int32_t* __restrict__ psum, int32_t* __restrict__ status) {
  __shared__ int lds_count[MOE_MAX_EXPERTS];
  __shared__ int lds16[16];
  __shared__ int lds_flag;
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  if (t == 0) lds_flag = 0;
  __syncthreads();
  // Column scans over the block totals: wave `wid` owns experts wid, wid+16,
  // ...; lane l owns a contiguous run of blocks so block order is preserved.
  const int64_t per = (nblocks + 63) / 64;
  for (int e = wid; e < E; e += kScanThreads / 64) {
    const int64_t lo = lane * per, hi = min(lo + per, nblocks);
    int s = 0;
    for (int64_t b = lo; b < hi; ++b) s += blk[b * E + e];
    const int incl = wave_incl_scan_i(s);
    int run = incl - s;
    for (int64_t b = lo; b < hi; ++b) {
      const int c = blk[b * E + e];
      blk[b * E + e] = run;
      run += c;
    }
    if (lane == 63) lds_count[e] = incl;
  }
  int f = 0;
  for (int64_t b = t; b < nblocks; b += kScanThreads) f |= blk_flag[b];
  if (f) atomicOr(&lds_flag, f);
  __syncthreads();
  const int cnt = t < E ? lds_count[t] : 0;
  const int blk_rows = align_up_i(cnt, align);
  int total;
  const int start = block_excl_scan(blk_rows, lds16, &total);
  int padtot;
  const int pb = block_excl_scan(blk_rows - cnt, lds16, &padtot);
  if (t < E) {
    starts[t] = start;
    psum[t] = start + cnt;
    padbase[t] = pb;
  }
  if (t == 0) {
    padbase[E] = padtot;
    status[0] = total;
    status[1] = lds_flag | (total > capacity ? MOE_FLAG_CAPACITY_OVERFLOW : 0);
  }
}

// Largest index i in [0, n) with a[i] <= v (a non-decreasing, a[0] <= v).
__device__ __forceinline__ int last_le(const int32_t* a, int n, int v) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= v) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Exclusive scan over a workgroup of NTH threads of n <= 1024 values held as
// v[i] (i < n); each thread owns a contiguous run of them.  Writes the
// exclusive prefixes to out[i] and returns the total (all threads).  lds_w:
// NTH / 64 ints of scratch.
template <int NTH>
__device__ int block_excl_scan_n(const int* v, int* out, int n, int* lds_w) {
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int per = (n + NTH - 1) / NTH;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += v[i];
  const int incl = wave_incl_scan_i(sum);
  if (lane == 63) lds_w[wid] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < NTH / 64; ++w) {
    if (w < wid) base += lds_w[w];
    total += lds_w[w];
  }
  int run = base + incl - sum;
  for (int i = lo; i < hi; ++i) {
    out[i] = run;
    run += v[i];
  }
  __syncthreads();
  return total;
}

// Ids of row r's group predecessors (up to 15 * topk <= 480 values, eight
// per lane; -1 past them) and, in lane k < topk, of slot (r, k).  Rows at or
// past the valid boundary route nowhere and are not read (a valid row's
// group predecessors are valid too).
struct RowIds {
  int prev[8];
  int myid;

  __device__ __forceinline__ void load(const int32_t* __restrict__ ids, int64_t r, int64_t nv,
                                       int topk, int lane) {
#pragma unroll
    for (int i = 0; i < 8; ++i) prev[i] = -1;
    myid = -1;
    if (r >= nv) return;
    const int64_t g_first = r / kGroupRows * kGroupRows;
    const int nprev = (int)(r - g_first) * topk;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = i * 64 + lane;
      if (idx < nprev) prev[i] = ids[g_first * topk + idx];
    }
    if (lane < topk) myid = ids[r * topk + lane];
  }
  // Rows loaded against the buffer's size, then cut at the valid-row bound.
  __device__ __forceinline__ void clip(int64_t r, int64_t nv) {
    if (r < nv) return;
#pragma unroll
    for (int i = 0; i < 8; ++i) prev[i] = -1;
    myid = -1;
  }
};

// The loads of a row with a local slot that do not depend on the
// destinations: its first 8 KB, its first 64 scales, each local slot's
// weight, its group's offset within its block and (block table in global
// memory) the block's offset: issued together, before the next row's
// prefetch, so that computing the destinations waits for nothing later.
struct RowData {
  u32x4 v[8];
  uint32_t sc;  // the scale: fp32 bits, a 4-byte MXFP8 word or a UE8M0 byte
  float wt;
  int grp;
  int blk;

  // kQ: the row is bf16 (2 bytes per element) and has no scales.  mine: this
  // lane's slot is local (lane k < topk holds slot k).
  template <bool kQ>
  __device__ __forceinline__ void load(const uint8_t* __restrict__ x, int64_t x_stride,
                                       const uint8_t* __restrict__ x_scale,
                                       int64_t x_scale_stride_bytes, int scale_bytes,
                                       const float* __restrict__ topk_w,
                                       const int32_t* __restrict__ grp_off,
                                       const int32_t* __restrict__ blk_off, int G, bool weights,
                                       int64_t r, int hidden, int topk, int E, int lane,
                                       bool mine, int myid) {
    const int nch = kQ ? hidden / 8 : hidden / 16, nsc = hidden / kGroup;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + r * x_stride);
    const uint8_t* srow = x_scale + r * x_scale_stride_bytes;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = u * 64 + lane;
      if (c < nch) v[u] = src[c];
    }
    // (one register for either width: two registers, each written by a load
    // on one branch only, make the compiler wait for every load in flight)
    sc = 0u;
    if (!kQ && scale_bytes && lane < nsc)
      sc = scale_bytes == 4 ? reinterpret_cast<const uint32_t*>(srow)[lane] : srow[lane];
    wt = 0.f;
    grp = 0;
    blk = 0;
    if (mine) {
      if (weights) wt = topk_w[r * topk + lane];
      if (grp_off) grp = grp_off[(r / kGroupRows) * E + myid];
      if (blk_off) blk = blk_off[(r / kGroupRows / G) * E + myid];
    }
  }
};

// One pass of a bf16 row (chunk c = c0 + u * 64 + lane, 8 elements each)
// quantised per 1x128 group: the 16 lanes of a group share its amax; codes
// (8 bytes per chunk) and the group's scale (fp32, or the UE8M0 byte in the
// low bits) per u.  Inactive chunks (c >= nch) give amax 0 and are not
// stored by the caller.  Every lane runs the shuffles.
template <bool kUe8m0>
__device__ __forceinline__ void quant_pass(const u32x4 (&v)[8], int c0, int nch, int lane,
                                           uint2 (&q)[8], uint32_t (&sc)[8]) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const bool active = c0 + u * 64 + lane < nch;
    float y[8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[2 * i] = __uint_as_float(v[u][i] << 16);
      y[2 * i + 1] = __uint_as_float(v[u][i] & 0xffff0000u);
    }
    if (active) {
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    amax = fmaxf(amax, 1e-10f);
    float p[8];
    if (kUe8m0) {
      const uint32_t b = e8m0_round_up(__fdiv_rn(amax, 448.0f));
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = ldexpf(y[i], 127 - (int)b);
      sc[u] = b;
    } else {
      const float inv = __fdiv_rn(448.0f, amax);
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = __fmul_rn(y[i], inv);
      sc[u] = __float_as_uint(__fdiv_rn(amax, 448.0f));
    }
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[4], p[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[6], p[7], hi, true);
    q[u] = make_uint2((uint32_t)lo, (uint32_t)hi);
  }
}

// Count of the valid slots with local ids, per expert, over the whole
// receive buffer (into tot) and over the slots before `npre` (into pre), for
// E <= 8: every workgroup of the fused launch runs this itself (at most
// kFusedSlots slots, so 32-bit slot indices); tot and pre are cleared here.
// The first pass of loads covers the buffer's slots (up to 8 x NTH vectors)
// whatever the valid-row bound, so that it need not wait for it; slots at or
// past `nslot` are not counted.  ids are
// read as 16-byte vectors when aligned (four slots each), eight in flight
// per thread.
// Each thread keeps its counts in 7-bit fields of a 64-bit word, expert e
// in field e and every id outside [0, 8) in a ninth field that is never read,
// so a slot costs a min, a multiply, a shift and an add with no compare; ids
// >= E are caught by a running max.  npre is a multiple of 4 or equal to
// nslot, so a vector of four valid slots lies wholly before or after it.
// The words are widened to 16-bit fields and summed over the wave by a
// transpose-reduce (DPP moves within rows of 16 lanes, two shuffles across
// rows), and eight lanes per wave add the sums to LDS.
__device__ __forceinline__ uint64_t slot_inc7(int id) {
  return 1ull << (min((unsigned)id, 8u) * 7u);
}

// a + the value of lane (lane ^ m) within rows of 16 lanes, m = 1, 2, 7, 8
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_add(uint32_t keep, uint32_t send) {
  return keep + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, kCtrl, 0xf, 0xf, false);
}

template <int NTH>
__device__ __forceinline__ void count_all(const int32_t* __restrict__ ids, int nall, int nslot,
                                          int npre, int E, bool vec, int32_t* tot,
                                          int32_t* pre, int& bad) {
  static_assert(kFusedSlots / NTH + 1 <= 127, "7-bit per-thread counters");
  const int t = threadIdx.x, lane = t & 63;
  uint64_t ct = 0ull, cp = 0ull;
  int mx = -1;
  auto one = [&](int id, int s) __attribute__((always_inline)) {  // any slot
    if (s < nslot) {
      const uint64_t inc = slot_inc7(id);
      ct += inc;
      if (s < npre) cp += inc;
      mx = max(mx, id);
    }
  };
  int done = 0;
  if (vec) {
    const int n4 = nall >> 2;
    const int n4v = min(n4, (nslot + 3) >> 2);  // vectors holding valid slots
    const int4* ids4 = reinterpret_cast<const int4*>(ids);
    constexpr int U = 8;
    // (only the first pass reads past the valid slots: by the second the
    // bound has arrived)
    for (int i0 = 0; i0 < (i0 == 0 ? n4 : n4v); i0 += U * NTH) {
      int4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * NTH + t;
        v[u] = i < n4 ? ids4[i] : make_int4(-1, -1, -1, -1);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = (i0 + u * NTH + t) * 4;
        if (s + 4 <= nslot) {  // four valid slots
          const uint64_t q = slot_inc7(v[u].x) + slot_inc7(v[u].y) + slot_inc7(v[u].z) +
                             slot_inc7(v[u].w);
          ct += q;
          cp += s < npre ? q : 0ull;
          mx = max(mx, max(max(v[u].x, v[u].y), max(v[u].z, v[u].w)));
        } else if (s < nslot) {
          one(v[u].x, s);
          one(v[u].y, s + 1);
          one(v[u].z, s + 2);
          one(v[u].w, s + 3);
        }
      }
    }
    done = n4 * 4;
  }
  for (int s = done + t; s < nslot; s += NTH) one(ids[s], s);
  bad |= (int)(mx >= E);
  // 16-bit fields: word k holds experts 2 (k & 3) and 2 (k & 3) + 1 of tot
  // (k < 4) or pre (k >= 4).
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint64_t x = k < 4 ? ct : cp;
    const int e = 2 * (k & 3);
    w[k] = (uint32_t)((x >> (7 * e)) & 127u) | ((uint32_t)((x >> (7 * e + 7)) & 127u) << 16);
  }
  // Transpose-reduce: each step pairs lanes that differ in one bit of
  // (lane & 7), each lane keeping half of its words (chosen by that bit)
  // plus its partner's copy of them; lane l ends with word l & 7 summed over
  // its 8 lanes, then over the wave.  (row_half_mirror pairs l with l ^ 7,
  // which differ in bit 2, while every lane still holds all eight words.)
  const bool b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
  uint32_t h[4], g[2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    h[j] = dpp_add<0x141>(b2 ? w[4 + j] : w[j], b2 ? w[j] : w[4 + j]);  // row_half_mirror
#pragma unroll
  for (int j = 0; j < 2; ++j)
    g[j] = dpp_add<0x4e>(b1 ? h[2 + j] : h[j], b1 ? h[j] : h[2 + j]);  // quad_perm 2,3,0,1
  uint32_t sum = dpp_add<0xb1>(b0 ? g[1] : g[0], b0 ? g[0] : g[1]);  // quad_perm 1,0,3,2
  sum = dpp_add<0x128>(sum, sum);                                     // row_ror:8 (lane ^ 8)
  sum += (uint32_t)__shfl_xor((int)sum, 16, 64);
  sum += (uint32_t)__shfl_xor((int)sum, 32, 64);
  for (int e = t; e < E; e += NTH) {
    tot[e] = 0;
    pre[e] = 0;
  }
  __syncthreads();  // (no barrier before the loads above)
  if (lane < 8) {
    int32_t* dst = lane < 4 ? tot : pre;
    const int e = 2 * (lane & 3);
    if (e < E && (sum & 0xffffu)) atomicAdd(&dst[e], (int)(sum & 0xffffu));
    if (e + 1 < E && (sum >> 16)) atomicAdd(&dst[e + 1], (int)(sum >> 16));
  }
}

// kQ: bf16 input rows quantised here (x_scale unused), with UE8M0 scales
// when kQU8 (else fp32); otherwise fp8 rows and their scales are copied.
// kFused: no count kernel ran; every workgroup counts the whole buffer's
// valid slots itself (count_all) and owns one 16-row group (rows
// 16 * blockIdx.x ..), wave w its rows w, w + 4, w + 8, w + 12.  Otherwise
// the count kernel's tables are used (with `fold`, the block table is
// scanned here by every workgroup) and the waves walk the rows grid-stride.
template <bool kQ, bool kQU8, bool kFused>
__global__ __launch_bounds__(kFused ? kFusedThreads : kScatterThreads) void expand_scatter_kernel(
    const uint8_t* __restrict__ x, int64_t x_stride, const uint8_t* __restrict__ x_scale,
    int64_t x_scale_stride_bytes, int scale_bytes, const int32_t* __restrict__ ids,
    const float* __restrict__ topk_w, const int32_t* __restrict__ psum_rank, int nsrc,
    int64_t rows, int hidden, int topk, int E, int64_t capacity, int align,
    const int32_t* __restrict__ grp_off, const int32_t* __restrict__ blk_g, int G, int nblk,
    const int32_t* __restrict__ blk_flag, int fold, const int32_t* __restrict__ starts_g,
    const int32_t* __restrict__ padbase_g, int32_t* __restrict__ psum_g,
    int32_t* __restrict__ status, uint8_t* __restrict__ ex, uint8_t* __restrict__ ex_scale,
    int32_t* __restrict__ m_indices, int32_t* __restrict__ src2dst, float* __restrict__ row_weight,
    int ids_vec) {
  constexpr int NT = kFused ? kFusedThreads : kScatterThreads;
  extern __shared__ int32_t lds[];
  int32_t* l_starts = lds;                // [E]
  int32_t* l_padbase = l_starts + E;      // [E + 1]
  int32_t* l_psum = l_padbase + E + 1;    // [E]
  int32_t* l_tmp = l_psum + E;            // [E]
  int32_t* l_blk = l_tmp + E;             // fold: [nblk][E]; fused: [E] (rows before the group)
  __shared__ int lds_w[NT / 64];
  __shared__ int l_total, l_flag;
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int64_t gwaves = (int64_t)gridDim.x * (NT / 64);
  const int64_t wave0 = (int64_t)blockIdx.x * (NT / 64) + wid;
  const int64_t nv = valid_rows(psum_rank, nsrc, rows);
  // This wave's rows: [r_first, r_end) in steps of r_step.
  const int64_t g0 = kFused ? (int64_t)blockIdx.x * kGroupRows : 0;
  const int64_t r_first = kFused ? g0 + wid : wave0;
  const int64_t r_end = kFused ? min(g0 + kGroupRows, rows) : rows;
  const int64_t r_step = kFused ? NT / 64 : gwaves;
  const bool weights = row_weight != nullptr;
  const int32_t* grp_tab = kFused ? nullptr : grp_off;
  const int32_t* blk_tab = kFused || fold ? nullptr : blk_g;  // else the LDS copy

  // The first row's ids (and, fold, the first 256 entries of the count
  // kernel's block table, which is all of it at the DeepSeek-V3 share) are
  // requested before anything waits.
  // (Never in the fused kernel: a register left waiting for such a load
  // makes the compiler drain every load in flight before it is reused.)
  const bool fold_c = !kFused && fold;
  const int nbe = fold_c ? nblk * E : 0;
  const int blk0 = t < nbe ? blk_g[t] : 0;
  const int flg0 = (fold_c && t < nblk) ? blk_flag[t] : 0;
  // (fused: loaded against the buffer's size, so that no load waits for the
  // valid-row bound, and cut at the bound once it is known)
  RowIds ia;
  if (r_first < r_end) ia.load(ids, r_first, kFused ? rows : nv, topk, lane);
  if (t < nbe) l_blk[t] = blk0;
  // The first row's data: fused, requested as soon as the count is in (its
  // ids arrived before the count's), so that it is in flight during the
  // scan; otherwise once the tables are read.
  RowData da;
  bool mine_a = false;
  uint64_t live_a = 0ull;
  auto start_a = [&]() __attribute__((always_inline)) {
    if (kFused) ia.clip(r_first, nv);
    mine_a = r_first < r_end && ia.myid >= 0 && ia.myid < E;
    live_a = __ballot(mine_a);
    if (r_first < r_end && live_a)
      da.load<kQ>(x, x_stride, x_scale, x_scale_stride_bytes, scale_bytes, topk_w, grp_tab,
                  blk_tab, G, weights, r_first, hidden, topk, E, lane, mine_a, ia.myid);
  };
  if (kFused || fold) {
    if (t == 0) l_flag = 0;
    int fl = 0;
    if constexpr (kFused) {
      // l_psum: totals; l_blk: counts before this group
      const int nall = (int)rows * topk, nsl = (int)nv * topk, npre = (int)min(g0, nv) * topk;
      count_all<NT>(ids, nall, nsl, npre, E, ids_vec != 0, l_psum, l_blk, fl);
      fl = fl ? MOE_FLAG_EXPERT_ID_RANGE : 0;
      start_a();
    } else {
      // The scan over the (few) block totals, done by every workgroup: block
      // offsets per expert, expert totals, aligned starts, pad prefix.  The
      // rest of the table and of the flags: every load issued before any is
      // used (one round trip, not one per pass).
      constexpr int kPer = kFoldScanInts / NT;
      int rest[kPer - 1], frest[kPer - 1];
#pragma unroll
      for (int j = 1; j < kPer; ++j) {
        const int i = t + j * NT;
        rest[j - 1] = i < nbe ? blk_g[i] : 0;
        frest[j - 1] = i < nblk ? blk_flag[i] : 0;
      }
      fl = flg0;
#pragma unroll
      for (int j = 1; j < kPer; ++j) {
        const int i = t + j * NT;
        if (i < nbe) l_blk[i] = rest[j - 1];
        fl |= frest[j - 1];
      }
    }
    __syncthreads();
    if (fl) atomicOr(&l_flag, fl);
    if constexpr (!kFused) {
      if (nblk <= 8 || E >= 64) {  // a thread per expert walks the blocks in order
        for (int e = t; e < E; e += NT) {
          int run = 0;
          for (int b = 0; b < nblk; ++b) {
            const int c = l_blk[b * E + e];
            l_blk[b * E + e] = run;
            run += c;
          }
          l_psum[e] = run;  // the count, for now
        }
      } else {  // a wave per expert scans 64 blocks at a time
        for (int e = wid; e < E; e += NT / 64) {
          int carry = 0;
          for (int b0 = 0; b0 < nblk; b0 += 64) {
            const int b = b0 + lane;
            const int c = b < nblk ? l_blk[b * E + e] : 0;
            const int incl = wave_incl_scan_i(c);
            if (b < nblk) l_blk[b * E + e] = carry + incl - c;
            carry += __shfl(incl, 63, 64);
          }
          if (lane == 0) l_psum[e] = carry;
        }
      }
      __syncthreads();
    }
    if (E <= 64) {  // one wave: aligned starts, pad prefix, psum, total
      if (wid == 0) {
        const int c = lane < E ? l_psum[lane] : 0;
        const int al = align_up_i(c, align);
        const int ia_ = wave_incl_scan_i(al);
        const int ip = wave_incl_scan_i(al - c);
        if (lane < E) {
          l_starts[lane] = ia_ - al;
          l_padbase[lane] = ip - (al - c);
          l_psum[lane] = ia_ - al + c;
        }
        if (lane == 63) {
          l_padbase[E] = ip;
          l_total = ia_;
        }
      }
    } else {
      for (int e = t; e < E; e += NT) l_tmp[e] = align_up_i(l_psum[e], align);
      __syncthreads();
      const int total = block_excl_scan_n<NT>(l_tmp, l_starts, E, lds_w);
      for (int e = t; e < E; e += NT) l_tmp[e] -= l_psum[e];  // pad rows
      __syncthreads();
      const int padtot = block_excl_scan_n<NT>(l_tmp, l_padbase, E, lds_w);
      for (int e = t; e < E; e += NT) l_psum[e] += l_starts[e];
      if (t == 0) {
        l_padbase[E] = padtot;
        l_total = total;
      }
    }
    __syncthreads();
    const int total = l_total;
    if (blockIdx.x == 0) {  // the layout's outputs
      for (int e = t; e < E; e += NT) psum_g[e] = l_psum[e];
      if (t == 0) {
        status[0] = total;
        status[1] = l_flag | (total > capacity ? MOE_FLAG_CAPACITY_OVERFLOW : 0);
      }
    }
  } else {
    for (int i = t; i < E; i += NT) {
      l_starts[i] = starts_g[i];
      l_psum[i] = psum_g[i];
    }
    for (int i = t; i <= E; i += NT) l_padbase[i] = padbase_g[i];
    if (t == 0) l_total = status[0];
    __syncthreads();
  }
  const int total = l_total;
  const int64_t nrows_ex = min((int64_t)total, capacity);
  const int nsc = scale_bytes ? hidden / kGroup : 0;  // no scales: bf16 rows kept
  const int nch = hidden / 16;                     // 16-byte chunks of an expanded row
  const int nch_in = kQ ? hidden / 8 : nch;        // ... of a received row

  // ---- the wave's rows, software-pipelined: while row r is stored, the
  // data of the next row and the ids of the row after are in flight ----
  if constexpr (!kFused) start_a();
  RowIds ib;  // (fused: each wave has one row, nothing to prefetch)
  if (!kFused && r_first + r_step < r_end) ib.load(ids, r_first + r_step, nv, topk, lane);
  for (int64_t r = r_first; r < r_end; r += r_step) {
    // next row's data (its ids have been in flight since the last row), and
    // the ids of the row after it
    // (ids first: the next iteration waits for them while this data may
    // still be in flight, loads completing in order)
    const int64_t rn = r + r_step;
    bool mine_b = false;
    uint64_t live_b = 0ull;
    RowIds ic;
    RowData db;
    if constexpr (!kFused) {
      mine_b = ib.myid >= 0 && ib.myid < E;
      live_b = rn < r_end ? __ballot(mine_b) : 0ull;
      if (rn + r_step < r_end) ic.load(ids, rn + r_step, nv, topk, lane);
      if (live_b)
        db.load<kQ>(x, x_stride, x_scale, x_scale_stride_bytes, scale_bytes, topk_w, grp_tab,
                    blk_tab, G, weights, rn, hidden, topk, E, lane, mine_b, ib.myid);
    }

    if (live_a == 0) {
      if (lane < topk) src2dst[r * topk + lane] = -1;
    } else {
      const int64_t g = r / kGroupRows;
      // Stable rank of each live slot among its expert's slots of the group:
      // earlier rows' slots, then this row's slots at smaller k.
      int rank = 0;
      for (uint64_t mm = live_a; mm; mm &= mm - 1) {
        const int k = __builtin_ctzll(mm);
        const int e = __shfl(ia.myid, k, 64);
        int rk = __popcll(__ballot(ia.myid == e) & ((1ull << k) - 1ull));
#pragma unroll
        for (int i = 0; i < 8; ++i) rk += __popcll(__ballot(ia.prev[i] == e));
        if (lane == k) rank = rk;
      }
      int d = -1;
      if (mine_a) {
        // (l_blk is LDS: the fused counts before this group, or the folded
        // block table; otherwise the block offset came with the row's data)
        const int64_t off = kFused ? (int64_t)l_blk[ia.myid]
                            : (int64_t)(fold ? l_blk[(g / G) * E + ia.myid] : da.blk) + da.grp;
        const int64_t dd = (int64_t)l_starts[ia.myid] + off + rank;
        if (dd < capacity) {
          d = (int)dd;
          if (weights) row_weight[d] = da.wt;
        }
      }
      if (lane < topk) src2dst[r * topk + lane] = d;
      const uint64_t mask = __ballot(d >= 0);
      if (mask != 0) {
        const u32x4* src = reinterpret_cast<const u32x4*>(x + r * x_stride);
        const uint8_t* srow = x_scale + r * x_scale_stride_bytes;
        for (int c0 = 0; c0 < nch_in; c0 += 64 * 8) {
          if (c0 > 0) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int c = c0 + u * 64 + lane;
              if (c < nch_in) da.v[u] = src[c];
            }
          }
          if constexpr (kQ) {
            // Quantise the pass once, then store it to every destination: the
            // codes of chunk c at byte 8c of the expanded row, the scale of
            // group c / 16 (K-block-major) from the group's first lane.
            uint2 q[8];
            uint32_t sc[8];
            quant_pass<kQU8>(da.v, c0, nch_in, lane, q, sc);
            for (uint64_t mm = mask; mm; mm &= mm - 1) {
              const int dk = __shfl(d, __builtin_ctzll(mm), 64);
              uint2* dst = reinterpret_cast<uint2*>(ex + (int64_t)dk * hidden);
#pragma unroll
              for (int u = 0; u < 8; ++u) {
                const int c = c0 + u * 64 + lane;
                if (c < nch_in) {
                  dst[c] = q[u];
                  if ((lane & 15) == 0) {
                    const int64_t at = (int64_t)(c >> 4) * capacity + dk;
                    if (kQU8) ex_scale[at] = (uint8_t)sc[u];
                    else reinterpret_cast<uint32_t*>(ex_scale)[at] = sc[u];
                  }
                }
              }
            }
          } else {
            for (uint64_t mm = mask; mm; mm &= mm - 1) {
              const int dk = __shfl(d, __builtin_ctzll(mm), 64);
              u32x4* dst = reinterpret_cast<u32x4*>(ex + (int64_t)dk * hidden);
#pragma unroll
              for (int u = 0; u < 8; ++u) {
                const int c = c0 + u * 64 + lane;
                if (c < nch) dst[c] = da.v[u];
              }
            }
          }
        }
        if constexpr (!kQ) {
          // Scales: the shuffles run with every lane active (a lane-divergent
          // shuffle could read an inactive lane), the stores only where c < nsc.
          for (int c0 = 0; c0 < nsc; c0 += 64) {
            const int c = c0 + lane;
            if (c0 > 0 && c < nsc) {
              da.sc = scale_bytes == 4 ? reinterpret_cast<const uint32_t*>(srow)[c] : srow[c];
            }
            // ex_scale is K-block-major: scale (row dk, block c) at c * capacity + dk.
            for (uint64_t mm = mask; mm; mm &= mm - 1) {
              const int dk = __shfl(d, __builtin_ctzll(mm), 64);
              if (c < nsc) {
                const int64_t at = (int64_t)c * capacity + dk;
                if (scale_bytes == 4) reinterpret_cast<uint32_t*>(ex_scale)[at] = da.sc;
                else ex_scale[at] = (uint8_t)da.sc;
              }
            }
          }
        }
      }
    }
    if constexpr (!kFused) {  // rotate the pipeline
      ia = ib;
      ib = ic;
      da = db;
      mine_a = mine_b;
      live_a = live_b;
    }
  }

  // ---- grid-stride: row labels and alignment pad rows ----
  const int64_t gthreads = (int64_t)gridDim.x * NT;
  const int64_t gtid = (int64_t)blockIdx.x * NT + t;
  for (int64_t i = gtid; i < capacity; i += gthreads) {
    int lab = -1;
    if (i < nrows_ex) lab = last_le(l_starts, E, (int)i);
    m_indices[i] = lab;
  }
  const int npad = l_padbase[E];
  for (int64_t p = wave0; p < npad; p += gwaves) {
    const int e = last_le(l_padbase, E, (int)p);
    const int64_t row = (int64_t)l_psum[e] + (p - l_padbase[e]);
    if (row >= capacity) continue;
    u32x4* dst = reinterpret_cast<u32x4*>(ex + row * hidden);
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int c = lane; c < nch; c += 64) dst[c] = z;
    for (int c = lane; c < nsc; c += 64) {
      const int64_t at = (int64_t)c * capacity + row;
      if (scale_bytes == 4) reinterpret_cast<float*>(ex_scale)[at] = 0.f;
      else ex_scale[at] = 0;
    }
    if (lane == 0 && row_weight) row_weight[row] = 0.f;
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_expand_workspace_bytes(int64_t rows, int topk, int num_experts) {
  if (rows < 0 || topk < 1 || topk > MOE_MAX_TOPK || num_experts < 1 ||
      num_experts > MOE_MAX_EXPERTS)
    return 0;
  return workspace_bytes(rows, num_experts);
}

namespace {

// Both entry points.  bf16: x holds bf16 rows, x_stride is in bytes here,
// x_scale is unused; with fmt MOE_SCALE_NONE the rows are kept in bf16 and
// scattered as 2 * hidden bytes with no scales.
moe_status expand_layout(bool bf16, const void* x, int64_t x_stride, const void* x_scale,
                         int64_t x_scale_stride, moe_scale_fmt fmt, const int32_t* topk_ids,
                         const float* topk_weights, const int32_t* psum_recv_per_rank,
                         int num_src_ranks, int64_t rows, int hidden, int topk, int num_experts,
                         int align, int64_t capacity, void* ex, void* ex_scale, int32_t* psum,
                         int32_t* m_indices, int32_t* src2dst, float* row_weight,
                         int32_t* status, void* workspace, size_t workspace_bytes_,
                         void* stream, void* (*scratch_fn)() = nullptr) {
  if (rows < 0 || hidden <= 0 || hidden % kGroup != 0 || topk < 1 || topk > MOE_MAX_TOPK ||
      num_experts < 1 || num_experts > MOE_MAX_EXPERTS || capacity < 0 || rows > (1LL << 30) ||
      capacity > (1LL << 30) || (int64_t)rows * topk > (1LL << 30))
    return MOE_ERR_SHAPE;
  if (align < MOE_MIN_ALIGN || align > MOE_MAX_ALIGN || (align & (align - 1)))
    return MOE_ERR_UNSUPPORTED;
  if (capacity % align != 0) return MOE_ERR_SHAPE;
  if (fmt != MOE_SCALE_F32 && fmt != MOE_SCALE_UE8M0 && !(bf16 && fmt == MOE_SCALE_NONE) &&
      !(!bf16 && fmt == MOE_SCALE_MXFP8))
    return MOE_ERR_UNSUPPORTED;
  // MXFP8: a row's four 1x32 scale bytes of a 128-wide block travel as one
  // 4-byte word (the fp32 path's copy); x_scale_stride is then in bytes.
  const bool mx = fmt == MOE_SCALE_MXFP8;
  const bool keep = fmt == MOE_SCALE_NONE;  // bf16 rows copied as they are
  if (x_stride < (bf16 ? 2 * (int64_t)hidden : hidden) ||
      (!bf16 && x_scale_stride < (mx ? hidden / 32 : hidden / kGroup)) ||
      (mx && x_scale_stride % 4))
    return MOE_ERR_SHAPE;
  if (mx && ((uintptr_t)x_scale % 4)) return MOE_ERR_ALIGNMENT;
  if (num_src_ranks < 0 || (psum_recv_per_rank && num_src_ranks == 0)) return MOE_ERR_SHAPE;
  if (!psum || !m_indices || !src2dst || !status) return MOE_ERR_NULL;
  if (rows > 0 && (!x || (!bf16 && !x_scale) || !topk_ids)) return MOE_ERR_NULL;
  if (capacity > 0 && (!ex || (!keep && !ex_scale))) return MOE_ERR_NULL;
  if (row_weight && !topk_weights && rows > 0) return MOE_ERR_NULL;
  if ((x_stride % 16) || ((uintptr_t)x % 16) || ((uintptr_t)ex % 16)) return MOE_ERR_ALIGNMENT;
  if (scratch_fn) {  // moe_expand_layout_noalloc: the static per-GPU scratch
    if (workspace_bytes(rows, num_experts) > workspace_bytes_) return MOE_ERR_SCRATCH;
    workspace = scratch_fn();
    if (!workspace) return MOE_ERR_LAUNCH;
  }
  if (!workspace || workspace_bytes_ < workspace_bytes(rows, num_experts))
    return MOE_ERR_WORKSPACE;
  if ((uintptr_t)workspace % 256) return MOE_ERR_ALIGNMENT;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int E = num_experts;
  const int64_t ng = num_groups(rows);
  Workspace w = carve(workspace, rows, E);
  const int scale_bytes = keep ? 0 : (fmt == MOE_SCALE_F32 || mx ? 4 : 1);

  const int G = groups_per_block(E);
  const int64_t nb = num_blocks(rows, E);
  // Small receive buffers: no count kernel; every scatter workgroup (1024
  // threads) counts the whole buffer's valid slots itself (at most
  // kFusedSlots ids, one round trip from L2) and owns one 16-row group, a
  // wave per row: one launch for the whole layout.
  // (not when quantising, for registers; E <= 8: per-thread counters)
  const bool fused = rows * topk <= kFusedSlots && !(bf16 && !keep) && E <= 8;
  // Otherwise: count kernel; a small block table is scanned by every scatter
  // workgroup itself (no scan kernel), a large one by the scan kernel once.
  const bool fold = !fused && nb * E <= kFoldScanInts;
  if (!fused) {
    if (ng > 0) {
      const size_t lds = size_t(G) * E * 4;
      hipLaunchKernelGGL(expand_count_kernel, dim3((unsigned)nb), dim3(kCountThreads), lds, s,
                         topk_ids, psum_recv_per_rank, num_src_ranks, rows, topk, E, G, ng,
                         w.grp, w.blk, w.blk_flag);
      if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
    }
    if (!fold) {
      hipLaunchKernelGGL(expand_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, w.blk,
                         w.blk_flag, nb, E, align, capacity, w.starts, w.padbase, psum, status);
      if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
    }
  }
  // Fused: a workgroup per 16-row group (at least one, which writes the
  // psum and the status).  Otherwise 768 workgroups (three per CU, what the
  // kernel's registers allow to be resident at once), each wave walking rows
  // grid-stride with the next row in flight; either way enough workgroups
  // that the label fill and the pad zeroing spread over the chip.
  const int64_t grid = fused ? std::max<int64_t>(1, (rows + kGroupRows - 1) / kGroupRows)
                             : 768;
  const size_t lds = (size_t(4) * E + 1 + (fused ? size_t(E) : fold ? size_t(nb) * E : 0)) * 4;
  const int hdim = keep ? 2 * hidden : hidden;
  const int64_t sstride = mx ? x_scale_stride : x_scale_stride * scale_bytes;
  const int ids_vec = ((uintptr_t)topk_ids % 16) == 0;
  const bool q = bf16 && !keep, qu8 = q && fmt == MOE_SCALE_UE8M0;
#define MOE_SCATTER_ARGS                                                                      \
  (const uint8_t*)x, x_stride, (const uint8_t*)x_scale, sstride, scale_bytes, topk_ids,        \
      topk_weights, psum_recv_per_rank, num_src_ranks, rows, hdim, topk, E, capacity, align,   \
      w.grp, w.blk, G, (int)nb, w.blk_flag, fold ? 1 : 0, w.starts, w.padbase, psum, status,   \
      (uint8_t*)ex, (uint8_t*)ex_scale, m_indices, src2dst, row_weight, ids_vec
  if (fused) {  // (never quantising)
    hipLaunchKernelGGL((expand_scatter_kernel<false, false, true>), dim3((unsigned)grid),
                       dim3(kFusedThreads), lds, s, MOE_SCATTER_ARGS);
  } else {
    auto k = !q ? expand_scatter_kernel<false, false, false>
             : qu8 ? expand_scatter_kernel<true, true, false>
                   : expand_scatter_kernel<true, false, false>;
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kScatterThreads), lds, s, MOE_SCATTER_ARGS);
  }
#undef MOE_SCATTER_ARGS
  if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_expand_layout(
    const void* x, int64_t x_stride, const void* x_scale, int64_t x_scale_stride,
    moe_scale_fmt fmt, const int32_t* topk_ids, const float* topk_weights,
    const int32_t* psum_recv_per_rank, int num_src_ranks, int64_t rows, int hidden, int topk,
    int num_experts, int align, int64_t capacity, void* ex, void* ex_scale, int32_t* psum,
    int32_t* m_indices, int32_t* src2dst, float* row_weight, int32_t* status, void* workspace,
    size_t workspace_bytes_, void* stream) {
  return expand_layout(false, x, x_stride, x_scale, x_scale_stride, fmt, topk_ids, topk_weights,
                       psum_recv_per_rank, num_src_ranks, rows, hidden, topk, num_experts, align,
                       capacity, ex, ex_scale, psum, m_indices, src2dst, row_weight, status,
                       workspace, workspace_bytes_, stream);
}

extern "C" moe_status moe_expand_layout_bf16(
    const void* x, int64_t x_stride, moe_scale_fmt fmt, const int32_t* topk_ids,
    const float* topk_weights, const int32_t* psum_recv_per_rank, int num_src_ranks,
    int64_t rows, int hidden, int topk, int num_experts, int align, int64_t capacity, void* ex,
    void* ex_scale, int32_t* psum, int32_t* m_indices, int32_t* src2dst, float* row_weight,
    int32_t* status, void* workspace, size_t workspace_bytes_, void* stream) {
  if (x_stride < 0 || x_stride > (1LL << 40)) return MOE_ERR_SHAPE;
  return expand_layout(true, x, x_stride * 2, nullptr, 0, fmt, topk_ids, topk_weights,
                       psum_recv_per_rank, num_src_ranks, rows, hidden, topk, num_experts, align,
                       capacity, ex, ex_scale, psum, m_indices, src2dst, row_weight, status,
                       workspace, workspace_bytes_, stream);
}

// ---- the layout with no workspace argument and no allocation ----
//
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation): the workspace lives in a
// file-scope device array of fixed size, one copy per GPU, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): its device address is looked
// up once per device with hipGetSymbolAddress, with that device current, and
// that address is what the kernels get.  Every call on a GPU shares that
// GPU's array, so calls that overlap on one GPU (different streams, no
// ordering between them) race; calls ordered on one stream do not.  The
// kernels overwrite every workspace entry they read before reading it, so
// nothing needs clearing between calls.
namespace {

constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up on the first
// call on each device); nullptr if the runtime cannot give it.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" moe_status moe_expand_layout_noalloc(
    const void* x, int64_t x_stride, const void* x_scale, int64_t x_scale_stride,
    moe_scale_fmt fmt, const int32_t* topk_ids, const float* topk_weights,
    const int32_t* psum_recv_per_rank, int num_src_ranks, int64_t rows, int hidden, int topk,
    int num_experts, int align, int64_t capacity, void* ex, void* ex_scale, int32_t* psum,
    int32_t* m_indices, int32_t* src2dst, float* row_weight, int32_t* status, void* stream) {
  // Every argument is checked as in moe_expand_layout, before the scratch
  // address is looked up; a valid request that needs more workspace than the
  // array holds gets MOE_ERR_SCRATCH.
  return expand_layout(false, x, x_stride, x_scale, x_scale_stride, fmt, topk_ids, topk_weights,
                       psum_recv_per_rank, num_src_ranks, rows, hidden, topk, num_experts, align,
                       capacity, ex, ex_scale, psum, m_indices, src2dst, row_weight, status,
                       nullptr, kNoAllocScratchBytes, stream, scratch_address);
}
