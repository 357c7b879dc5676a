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
//    expert by expert, N tile by N tile, with the expert's row groups
//    innermost; consecutive items land on one XCD (dispatch is round-robin
//    over the 8 XCDs, and the block -> item map undoes that), so the groups of
//    an (expert, N tile) stream the same weights side by side and that XCD's
//    L2 serves them, while neighbouring N tiles share the groups'
//    activations.
//  - In the workgroups' first round of items each N tile walks K from its own
//    start block, k0 = nt * KB / NT, wrapping round: every CU starts at the
//    same moment, and the items of one row group (one XCD at the
//    DeepSeek-V3 share) would otherwise all ask for the same activation
//    block at once and all wait out its HBM miss; staggered, one of them
//    misses and the rest find it in L2.  Later rounds are out of phase
//    already and walk K in order (a staggered walk there only lengthens
//    each activation block's reuse distance in L2).  An output's summation
//    order thus depends only on its N tile and its item's round, the same in
//    the contiguous and masked modes when the item falls in the same round.
//  - K advances one 128-wide scale block per step = one
//    v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 sub-tile.  Eight waves (two
//    per SIMD) in a 4 x 2 grid, each owning 64 x 64 outputs (4 x 4 MFMA tiles).
//  - Operands go HBM -> LDS directly (global_load_lds_dwordx4) in two rings:
//    weights in three slots streamed two K steps ahead by waves 0-3;
//    activations and their scales (re-read by every N tile of the group,
//    L2 hits but for the first reader of a block) in 3-4 slots sized to the
//    group, two or three steps ahead, loaded by waves 4-7.  (Measured: a
//    full 256-row group's activations one step ahead, with the weights four
//    ahead, left every wave waiting at the step's barrier for the late
//    activation block; this split is 2-6% faster at every shape, and giving
//    small groups more weight slots in the space their activations leave
//    free gains nothing.)  vmcnt is per wave, so each stream keeps its own
//    depth.  Each wave's K loop is instantiated for its role (weights, or
//    activations with na blocks per stage) and its live-tile count, so the
//    per-stage load count and every vmcnt wait are compile-time: the loop
//    issues about 175 instructions per step per wave, of which 12..16 are
//    MFMAs and 48..64 the fp32 promotion.  LDS -> registers runs one step ahead: while the matrix core
//    works on step k from registers, the wave reads step k+1's fragments.
//    One bare s_barrier per step publishes the next stage and frees the
//    slots of the step just moved into registers.
//    The 16-byte chunks of every 128-byte row are XOR-swizzled by row (swz),
//    chosen per lane on the global side, so the 16-row fragment reads are
//    bank-conflict free.
//  - fp32 scales: each step's MFMA result is promoted into the fp32
//    accumulator with the row's activation scale times the block's weight
//    scale (the scales do not factor out of the K sum).
//  - UE8M0 scales: the exponent bytes are the MFMA's hardware scale operands
//    (the group's byte repeats over its four 32-wide sub-blocks), so the
//    matrix core accumulates the scaled products directly.
//  - The bf16 outputs pass through LDS (each wave's 64 x 64 tile in its own
//    8 KB of the idle ring) so that every store instruction writes whole
//    128-byte row segments; rows past the group's live rows are never
//    written.
//  - Masked mode (the decode path's fixed-height slab, SGLang
//    moe_runner/deep_gemm.py source, _run_masked_gemm; SGLang PR 37261, "Why
//    decode stays on V1 low_latency"): expert e owns slab rows
//    [e * max_m, e * max_m + masked_m[e]); only the item decode differs.
#include "common.hpp"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Operand formats: fp8 with fp32 scales (promoted in VALU), fp8 with UE8M0
// scales (the MFMA's own scale operands), bf16 (no scales), MXFP8 (a UE8M0
// byte per 1x32 group of every activation row and every weight row: each
// lane passes the bytes of its own rows' 32-wide K chunk).
constexpr int kF32 = 0, kU8 = 1, kBF = 2, kMX = 3;
constexpr int kMxMaxExperts = 256;  // MXFP8: smaller expert tables make room for
constexpr int WSC_SLOT = 1024;      // the weight-scale ring (4 waves x 256 B per slot)

constexpr int kThreads = 512;  // 8 waves: 2 per SIMD
constexpr int kWaves = kThreads / 64;
constexpr int kXcds = 8;       // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr int GM = 256;        // rows per work item
constexpr int BN = 128;
constexpr int BK = 128;
constexpr int WAVES_N = 2;
constexpr int WAVES_M = kWaves / WAVES_N;   // 4
constexpr int WTM = 64, WTN = 64;            // wave tile: 4 x 2 waves cover 256 x 128
constexpr int FM = WTM / 16, FN = WTN / 16;  // 4 x 4 MFMA tiles per wave
// A wave's row tiles are interleaved: M-wave wm owns the 16-row tiles
// wm, wm + 4, wm + 8, wm + 12, so a group's live rows spread evenly over the
// M-waves (and over both waves of every SIMD) whatever the group's size.
constexpr int ROW_TILE_STRIDE = WAVES_M * 16;             // rows between a wave's tiles
constexpr int A_TILE_STRIDE = ROW_TILE_STRIDE * 128;     // LDS bytes between them
constexpr int A_BYTES = GM * BK;             // 32 KB: one K block of a full row group
constexpr int B_BYTES = BN * BK;             // 16 KB: one K block of the N tile's weights
// Two operand rings.  Weights: kBSlots slots, streamed kBSlots - 1 K steps
// ahead by waves 0-3.  Activations (re-read by every N tile of the group;
// the first reader of a K block misses L2): 3..4 slots sized to the group,
// loaded 2..3 steps ahead (with the activation scales) by waves 4-7.  vmcnt
// is per wave, so each stream keeps its own depth.
constexpr int kBSlots = 3;
constexpr int B_RING = kBSlots * B_BYTES;
constexpr int A_BASE = B_RING;
constexpr int A_RING = 3 * A_BYTES;          // three slots of a full group, four if smaller
constexpr int kMaxASlots = 4;
constexpr int DATA_BYTES = B_RING + A_RING;  // 144 KB
constexpr int kScSlots = kMaxASlots + 1;     // the step computed keeps its own
constexpr int SC_SLOT = GM * 4;              // a step's activation scales (<= 4 B per row)
constexpr int SC_BASE = DATA_BYTES;
constexpr int BSC_BYTES = 2048;              // an item's weight block scales, all K blocks
constexpr int BSC_BASE = SC_BASE + kScSlots * SC_SLOT;
constexpr int MAX_KB = BSC_BYTES / 4 - 1;    // K / 128 limit (fits BSC_BYTES incl. alignment)
constexpr int DUMMY_BASE = BSC_BASE + BSC_BYTES;  // landing area of the padding loads
constexpr int DUMMY_BYTES = 3 * 256;
constexpr int LDS_BYTES = DUMMY_BASE + DUMMY_BYTES;  // 152 KB of the CU's 160 KB
constexpr int kLoadWaves = 4;                // waves per stream: 0-3 weights, 4-7 activations
constexpr int B_LOADS = B_BYTES / (kLoadWaves * 64 * 16);  // 16-byte loads per lane per stage
constexpr int A_LOADS = A_BYTES / (kLoadWaves * 64 * 16);  // at most, for a full group
constexpr int W_LOADS = B_LOADS;             // a weight wave's loads per stage
static_assert(kWaves == 2 * kLoadWaves && B_LOADS == 4 && A_LOADS == 8, "load split");

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

// LDS reads by 32-bit LDS address (keeps addresses in single registers and
// lets constant parts fold into the instruction's offset field).
template <typename T>
__device__ __forceinline__ T lds_load(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(addr);
}
template <typename T>
__device__ __forceinline__ void lds_store(uint32_t addr, T v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(addr) = v;
}

// Direct HBM -> LDS loads.  Issued from inline assembly so the compiler does
// not treat them as LDS writes that every later LDS read must wait for: the
// kernel orders them itself (vmcnt waits + s_barrier).  Address = 64-bit
// scalar base + 32-bit per-lane offset; lane i's data lands at lds + i * size,
// the LDS base taken from M0, which the asm names as an input operand so the
// compiler itself writes it and knows it is in use.
// A wave-uniform pointer, held in scalar registers (the loads' base operand).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint32_t lds) {
  base = uniform_ptr(base);                   // wave-uniform by construction
  lds = __builtin_amdgcn_readfirstlane(lds);  // M0: wave-uniform by construction
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const uint8_t* base, uint32_t off, uint32_t lds) {
  base = uniform_ptr(base);
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("global_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }
// Keep the compiler's scheduler from moving instructions across this point
// (bounds how far it hoists the next step's fragment reads, and with them
// the registers they occupy).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// All of this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Wait until at most a * NL of this wave's vector-memory operations are
// outstanding, a in [0, MAXA] at run time (s_waitcnt takes an immediate: a
// short compare chain picks it).
template <int NL, int MAXA>
__device__ __forceinline__ void wait_ahead(int a) {
  if constexpr (MAXA <= 0) {
    wait_vmcnt<0>();
  } else {
    if (a >= MAXA) wait_vmcnt<MAXA * NL>();
    else wait_ahead<NL, MAXA - 1>(a);
  }
}

// Activation ring geometry for na 8-row blocks per loading wave per stage
// (a slot holds 32 * na rows): slots that fit the ring.
__host__ __device__ constexpr int act_slots(int na) { return na <= 6 ? 4 : 3; }
static_assert(4 * 6 * 4096 <= A_RING && 3 * 8 * 4096 <= A_RING,
              "activation ring");

struct Item {
  const uint8_t* a;     // first row of the group
  const uint8_t* b;     // first weight row of the N tile
  const uint8_t* as;    // scale of the group's first row in K block 0
  int64_t as_kstride;   // bytes from one K block's activation scales to the next
  const uint8_t* bs;    // aligned word holding the weight scale of (expert, N tile, block 0)
  int bs_skew;          // byte offset of that scale within the word (UE8M0: 0..3)
  int live;             // rows of the group that hold a slot (1..GM); the
                        // rest of the group is alignment padding
  int KB;               // K / 128
  int k0;               // first K block of this item's walk (then k0+1, .., wrapping)
  int K;
  int sbytes;           // 4 (fp32, MXFP8 words) or 1 (UE8M0)
  const uint8_t* ws;    // MXFP8: scales of the N tile's first weight row (K/32 bytes per row)
  uint32_t wsc_lds;     // MXFP8: LDS address of the weight-scale ring
  int blocks;           // 8-row blocks holding live rows
  int na;               // blocks per activation-loading wave per stage (1..8)
  int a_slot_bytes;     // activation slot: 32 * na rows x 128 B
  int na_slots;         // activation slots: act_slots(na)
};

// Byte offset of this lane's 16-byte chunk of row r in a [rows][K] operand:
// 8 lanes per 128-byte row segment, chunk order swizzled by row (swz).
__device__ __forceinline__ uint32_t row_chunk_offset(int r, int lane, int K) {
  return (uint32_t)r * (uint32_t)K + (uint32_t)((lane & 7) ^ swz_key(r)) * 16u;
}

// An item's weight block scales for every K block (KB consecutive elements
// from it.bs + bs_skew), copied into LDS once per item by the last wave as
// aligned 4-byte words; words past the last one needed re-read it.
__device__ __forceinline__ void load_item_wscales(const Item& it, uint32_t lds0, int lane) {
  const int words = (it.bs_skew + it.KB * it.sbytes + 3) >> 2;
  for (int c = 0; c * 64 < words; ++c) {
    const int w = c * 64 + lane;
    dma4(it.bs, (uint32_t)(w < words ? w : words - 1) * 4u, lds0 + BSC_BASE + c * 256);
  }
}

// One wave's share of the direct-to-LDS loads of a K step, with the per-lane
// source offsets and the LDS offsets computed once per item.  Load j covers
// one 8-row block (8 lanes per 128-byte row), landing at the block's offset
// in the slot.
//
// Weights (waves 0-3): wave w loads blocks j * 4 + w of the N tile's 128
// rows, B_LOADS per stage.
// Activations (waves 4-7): wave w loads blocks j * 4 + w that hold live
// rows (rows past the live rows inside a block reload the last live row);
// every loading wave issues exactly na loads per stage, the ones past its
// share reloading the group's last block into its own place (same bytes, so
// the duplicate write is harmless), so that the per-stage count is a
// compile-time constant.  Then one 4-byte-per-lane scale load (the scales
// are K-block-major, so a step's scales of the group are one contiguous
// run): with fp32 scales wave w brings rows w * 64 + lane; with UE8M0 the
// first of these waves brings all of them (lane l: rows 4l..4l+3) and the
// others issue the same load into a dummy area, again to keep the count
// fixed.  Lanes past the live rows re-read the last live row's word.  No
// branch: a branch would let the compiler sink the step's first MFMAs below
// the loads.
struct WaveLoads {
  uint32_t off[A_LOADS];  // weights use the first B_LOADS
  int lds_off[A_LOADS];
  uint32_t scale_off;     // source offset of this lane's scale word
  uint32_t wsc_off;       // MXFP8 weight waves: offset of weight row w * 32 + lane % 32's scales
  uint32_t scale_rel;     // its LDS offset within the scale slot
  uint32_t dummy;         // LDS address of this wave's dummy area (0: none)

  __device__ __forceinline__ void init(const Item& it, int wid, int lane, uint32_t lds0) {
    const bool wload = wid < kLoadWaves;
    const int w = wload ? wid : wid - kLoadWaves;
    wsc_off = (uint32_t)(w * 32 + (lane & 31)) * (uint32_t)(it.K / 32);
    const int nreal = wload ? B_LOADS : max(0, min(it.na, (it.blocks - w + kLoadWaves - 1) / kLoadWaves));
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
      const int b = j < nreal ? j * kLoadWaves + w : it.blocks - 1;
      const int r = b * 8 + (lane >> 3);
      const int rr = wload ? r : min(r, it.live - 1);
      off[j] = row_chunk_offset(r, lane, it.K) - (uint32_t)(r - rr) * (uint32_t)it.K;
      lds_off[j] = b * 1024;
    }
    if (it.sbytes == 4) {  // fp32: wave w, rows w * 64 + lane
      scale_off = (uint32_t)min(w * 64 + lane, it.live - 1) * 4u;
      scale_rel = (uint32_t)w * 256u;
      dummy = 0;
    } else {               // UE8M0: one wave, lane l -> rows 4l .. 4l+3
      const int l = (it.live - 1) >> 2;
      scale_off = (uint32_t)min(lane, l) * 4u;
      scale_rel = 0;
      dummy = w > 0 ? lds0 + DUMMY_BASE + (uint32_t)(w - 1) * 256u : 0u;
    }
  }
  // Weights of one stage from src (row 0 at K block q) into the slot at lds.
  __device__ __forceinline__ void weights(const uint8_t* src, uint32_t lds) const {
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) dma16(src, off[j], lds + lds_off[j]);
  }
  // Activations (NA loads) and the scale load of one stage.
  template <int NA, bool kScales>
  __device__ __forceinline__ void acts(const uint8_t* src, uint32_t lds, const uint8_t* ssrc,
                                       uint32_t slds) const {
#pragma unroll
    for (int j = 0; j < NA; ++j) dma16(src, off[j], lds + lds_off[j]);
    if constexpr (kScales) dma4(ssrc, scale_off, dummy ? dummy : slds + scale_rel);
  }
};

// Per-lane LDS byte offsets (within a stage) of the two 16-byte halves of
// this lane's A and B fragments for row/column tile 0; row tile i adds
// i * A_TILE_STRIDE, column tile j adds j * 2048.
struct FragOffsets {
  int a_lo, a_hi, b_lo, b_hi, m_row;
  int wsc_lane;  // MXFP8: this lane's weight row's word in a weight-scale slot (column tile 0)
  int a_mx_lo, a_mx_hi, b_mx_lo, b_mx_hi;  // MXFP8: this lane's two 16-byte chunks
};

__device__ __forceinline__ FragOffsets frag_offsets(int lane, int wm, int wn) {
  const int frow = lane & 15, fk = (lane >> 4) * 2;
  FragOffsets f;
  const int ra = wm * 16 + frow, rb = wn * WTN + frow;
  f.a_lo = swz(ra, fk);
  f.a_hi = swz(ra, fk + 1);
  f.b_lo = swz(rb, fk);  // within a weight slot
  f.b_hi = swz(rb, fk + 1);
  f.m_row = wm * 16 + frow;  // this lane's output row in row tile 0
  // Weight row r = wn * 64 + frow + 16 j sits at (r / 32) * 256 + (r % 32) * 4
  // of a slot: this lane's base plus (j / 2) * 256 + (j % 2) * 64.
  f.wsc_lane = wn * 512 + frow * 4;
  // MXFP8: with a scale per 32-wide K block the order of K inside a lane
  // matters (with one scale per row, as in the other formats, only the
  // pairing of A and B does).  The scaled MFMA takes a lane's 32 bytes as two
  // 16-byte halves, K [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16) for
  // lane group g = lane / 16, with lane l's scale register scaling block g of
  // its row (measured on gfx950 with per-block scales on either operand,
  // against the two other plausible orders).  So lane l brings logical
  // 16-byte chunks g and 4 + g: two 16-byte reads per fragment, like the
  // other formats, one logical chunk per 16 rows (bank-conflict free).
  const int g = lane >> 4;
  f.a_mx_lo = swz(ra, g);
  f.a_mx_hi = swz(ra, 4 + g);
  f.b_mx_lo = swz(rb, g);
  f.b_mx_hi = swz(rb, 4 + g);
  return f;
}

__device__ __forceinline__ v8i frag2(uint32_t base, int lo_off, int hi_off) {
  const u32x4 lo = lds_load<u32x4>(base + lo_off);
  const u32x4 hi = lds_load<u32x4>(base + hi_off);
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
             (int)hi[3]};
}

// Two floats -> packed bf16 pair (low = x), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x, y}, bf16x2_t));
}

__device__ __forceinline__ v4f mfma_plain(const v8i& a, const v8i& b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                          127, 0, 127);
}

// Scales of a K step, read from LDS during the step before (raw words), then
// turned into their register form once those reads have long returned: for
// fp32 scales early in the step itself (the first promotion comes two MFMAs
// in), for UE8M0 at the end of the step before (the MFMAs take them as
// operands).
template <int kFmt, int NFM>
struct StepScales;
template <int NFM>
struct StepScales<kBF, NFM> {  // bf16: no scales
  __device__ __forceinline__ void read(uint32_t, uint32_t, const Item&, const FragOffsets&, int,
                                       int) {}
  __device__ __forceinline__ void finish(const Item&, const FragOffsets&, int, int) {}
};
template <int NFM>
struct StepScales<kF32, NFM> {
  float raw[NFM];  // activation scale of this lane's row, per row tile
  float wraw;      // the weight block scale
  float scl[NFM];  // their products
  __device__ __forceinline__ void read(uint32_t sc, uint32_t bsc, const Item& it,
                                       const FragOffsets& fo, int kb, int) {
    const int blk = kb + it.k0 < it.KB ? kb + it.k0 : kb + it.k0 - it.KB;
    wraw = lds_load<float>(bsc + blk * 4);
#pragma unroll
    for (int i = 0; i < NFM; ++i) raw[i] = lds_load<float>(sc + (fo.m_row + i * ROW_TILE_STRIDE) * 4);
  }
  __device__ __forceinline__ void finish(const Item&, const FragOffsets&, int, int) {
#pragma unroll
    for (int i = 0; i < NFM; ++i) scl[i] = raw[i] * wraw;
  }
};
template <int NFM>
struct StepScales<kMX, NFM> {  // MXFP8: per-lane bytes of its rows' 32-wide K chunk
  int abyte[NFM];  // this lane's activation row, per row tile (the step computed)
  int sbyte[FN];   // this lane's weight row, per column tile
  int nabyte[NFM], nsbyte[FN];  // the same for the next step
  // Step kb's bytes: lane l holds K chunk l / 16 of the step, which is byte
  // l / 16 of its rows' words.  Read into the next-step registers early in
  // the step before (its stage has landed by then), moved into the ones the
  // MFMAs take after that step's last MFMA.
  __device__ __forceinline__ void load(uint32_t sc, const Item& it, const FragOffsets& fo,
                                       int kb, int lane) {
    const uint32_t ws = it.wsc_lds + (uint32_t)(kb % kBSlots) * WSC_SLOT + (lane >> 4);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      nsbyte[j] = lds_load<uint8_t>(ws + fo.wsc_lane + (j >> 1) * 256 + (j & 1) * 64);
#pragma unroll
    for (int i = 0; i < NFM; ++i)
      nabyte[i] = lds_load<uint8_t>(sc + (fo.m_row + i * ROW_TILE_STRIDE) * 4 + (lane >> 4));
  }
  __device__ __forceinline__ void advance() {
#pragma unroll
    for (int j = 0; j < FN; ++j) sbyte[j] = nsbyte[j];
#pragma unroll
    for (int i = 0; i < NFM; ++i) abyte[i] = nabyte[i];
  }
  __device__ __forceinline__ void read(uint32_t, uint32_t, const Item&, const FragOffsets&, int,
                                       int) {}
  __device__ __forceinline__ void finish(const Item&, const FragOffsets&, int, int) {}
};
template <int NFM>
struct StepScales<kU8, NFM> {
  uint32_t raw[NFM];  // row r's exponent byte is byte r of the slot
  uint32_t wraw;
  int abyte[NFM];
  int sbyte;
  __device__ __forceinline__ void read(uint32_t sc, uint32_t bsc, const Item& it,
                                       const FragOffsets& fo, int kb, int lane) {
    const int arow = fo.m_row;  // this lane's activation row
    const int blk = kb + it.k0 < it.KB ? kb + it.k0 : kb + it.k0 - it.KB;
    wraw = lds_load<uint32_t>(bsc + ((it.bs_skew + blk) & ~3));
#pragma unroll
    for (int i = 0; i < NFM; ++i)
      raw[i] = lds_load<uint32_t>(sc + ((arow + i * ROW_TILE_STRIDE) & ~3));
  }
  __device__ __forceinline__ void finish(const Item& it, const FragOffsets& fo, int kb,
                                         int lane) {
    const int arow = fo.m_row;
    const int bpos = it.bs_skew + (kb + it.k0 < it.KB ? kb + it.k0 : kb + it.k0 - it.KB);
    sbyte = (int)((wraw >> (8 * (bpos & 3))) & 0xffu);
#pragma unroll
    for (int i = 0; i < NFM; ++i)
      abyte[i] = (int)((raw[i] >> (8 * ((arow + i * ROW_TILE_STRIDE) & 3))) & 0xffu);
  }
};

// One K step from registers: a[0..NFM) x b[0..FN) with the scales `cur`.
// With kNext, the fragments of step kb+1 replace the old ones as soon as the
// MFMAs that read them are issued (A row tile i after MFMA (i, FN-1), B
// column tile j after MFMA (NFM-1, j), from slots next_a / next_b), step
// kb+1's scales are read into `nxt` (slot next_sc), and `issue` (the wave's
// loads for a later stage) runs in the shadow of the first MFMAs instead of
// delaying them.  NFM: how many of the wave's four 16-row tiles hold live
// rows.
template <int kFmt, int NFM, bool kNext, typename Issue>
__device__ __forceinline__ void step(v8i (&a)[FM], v8i (&b)[FN], v4f (&acc)[FM][FN],
                                     StepScales<kFmt, NFM>& ss, uint32_t next_a,
                                     uint32_t next_b, uint32_t next_sc, uint32_t bsc,
                                     const Item& it, const FragOffsets& fo, int kb, int lane,
                                     Issue&& issue) {
  constexpr int M = NFM * FN;  // MFMAs of this step
  auto refresh = [&](int t) __attribute__((always_inline)) {  // after MFMA t
    if constexpr (kNext) {
      const int i = t / FN, j = t % FN;
      if constexpr (kFmt == kMX) {
        if (i == NFM - 1) b[j] = frag2(next_b + j * 2048, fo.b_mx_lo, fo.b_mx_hi);
        if (j == FN - 1) a[i] = frag2(next_a + i * A_TILE_STRIDE, fo.a_mx_lo, fo.a_mx_hi);
      } else {
        if (i == NFM - 1) b[j] = frag2(next_b + j * 2048, fo.b_lo, fo.b_hi);
        if (j == FN - 1) a[i] = frag2(next_a + i * A_TILE_STRIDE, fo.a_lo, fo.a_hi);
      }
    }
  };
  auto side = [&](int t) __attribute__((always_inline)) {  // after MFMA t: work not feeding this step
    if (t == 0) {
      if constexpr (kFmt == kF32) ss.finish(it, fo, kb, lane);  // this step's products
      if constexpr (kNext) ss.read(next_sc, bsc, it, fo, kb + 1, lane);
    }
    if constexpr (kFmt == kU8 && kNext)
      if (t == M - 1) ss.finish(it, fo, kb + 1, lane);       // the next step's operands
    if constexpr (kFmt == kMX && kNext) {
      if (t == 0) ss.load(next_sc, it, fo, kb + 1, lane);  // the next step's bytes
      if (t == M - 1) ss.advance();                         // after the last MFMA
    }
    if (t == (M > 1 ? 1 : 0)) issue();
  };
  if constexpr (kFmt == kBF) {
    // bf16: a 128-byte K step is 64 values, two 16x16x32 MFMAs per tile on
    // the fragments' two 16-byte halves (A and B split K the same way, so
    // the two products cover the step's K exactly once).  All first halves,
    // then all second halves: the two MFMAs of one accumulator are M slots
    // apart.  The fragments are replaced after their second use.
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    auto half = [](const v8i& f, int h) __attribute__((always_inline)) {
      typedef int v4i __attribute__((ext_vector_type(4)));
      const v4i q = h ? v4i{f[4], f[5], f[6], f[7]} : v4i{f[0], f[1], f[2], f[3]};
      return __builtin_bit_cast(bf16x8, q);
    };
#pragma unroll
    for (int t = 0; t < M; ++t) {
      const int i = t / FN, j = t % FN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(half(b[j], 0), half(a[i], 0),
                                                          acc[i][j], 0, 0, 0);
      sched_fence();
      side(t);
      sched_fence();
    }
#pragma unroll
    for (int t = 0; t < M; ++t) {
      const int i = t / FN, j = t % FN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(half(b[j], 1), half(a[i], 1),
                                                          acc[i][j], 0, 0, 0);
      sched_fence();
      refresh(t);
      sched_fence();
    }
  } else if constexpr (kFmt == kU8 || kFmt == kMX) {
    // The exponent bytes are the MFMA's own scale operands.
#pragma unroll
    for (int t = 0; t < M; ++t) {
      const int i = t / FN, j = t % FN;
      int sb;
      if constexpr (kFmt == kMX) sb = ss.sbyte[j];
      else sb = ss.sbyte;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[j], a[i], acc[i][j], 0, 0, 0,
                                                                   sb, 0, ss.abyte[i]);
      sched_fence();
      side(t);
      refresh(t);
      sched_fence();
    }
  } else {
    // fp32 scales: each 16x16 product is promoted into the accumulator
    // (acc += P * sa * sb) two MFMAs after it was issued, from three product
    // registers in rotation.  The scheduling fences pin the order "MFMA t,
    // then promote t-2": the result read was produced two matrix-core slots
    // earlier, so the promotion needs no wait states and the matrix core
    // always has the next product queued.
    constexpr int kLag = 2;
    v4f p[kLag + 1];
#pragma unroll
    for (int t = 0; t < M + kLag; ++t) {
      if (t < M) p[t % (kLag + 1)] = mfma_plain(b[t % FN], a[t / FN]);
      sched_fence();
      if (t >= kLag) {
        const int u = t - kLag, i = u / FN, j = u % FN;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] += p[u % (kLag + 1)][q] * ss.scl[i];
      }
      if (t < M) {
        side(t);
        refresh(t);
      }
      sched_fence();
    }
  }
}

// The K loop of one item for one wave.  ROLE 0: the wave streams weights
// (kBSlots slots, kBSlots - 1 stages ahead); ROLE na > 0: it streams na
// activation blocks + one scale load per stage (act_slots(na) slots).  Both
// the per-stage load count and the depth are compile-time, so every vmcnt
// wait is an immediate.  Step kb: wait for this wave's loads of stage kb+1
// and for its reads of step kb's fragments; barrier (stage kb+1 is now
// visible to every wave, and every wave holds step kb's fragments in
// registers, so the slots of stage kb are free); refill them with the next
// stage of the stream; compute step kb from registers while reading step
// kb+1's fragments.
template <int kFmt, int NFM, int ROLE>
__device__ __forceinline__ void kloop(uint32_t lds0, v4f (&acc)[FM][FN], const Item& it,
                                      const WaveLoads& wl, const FragOffsets& fo, int lane,
                                      int wid) {
  constexpr bool kW = ROLE == 0;
  constexpr bool kSc = kFmt != kBF;                   // activation scales streamed
  constexpr bool kMxW = kW && kFmt == kMX;            // + the weight rows' scale words
  constexpr int NL = kW ? W_LOADS + (kMxW ? 1 : 0) : ROLE + (kSc ? 1 : 0);  // loads per stage
  constexpr int D = kW ? kBSlots : act_slots(ROLE);   // stream depth (slots)
  const int KB = it.KB;
  const uint32_t a_end = lds0 + A_BASE + (uint32_t)(it.na_slots * it.a_slot_bytes);
  // Stream state: source pointers and destination slots of the next stage to
  // load, advanced one stage per issue.
  int blk = it.k0;  // K block of the next stage to load
  const uint8_t* src = uniform_ptr((kW ? it.b : it.a) + (int64_t)it.k0 * BK);
  const uint8_t* ssrc = uniform_ptr(it.as + it.k0 * it.as_kstride);
  uint32_t dst = kW ? lds0 : lds0 + A_BASE, sdst = lds0 + SC_BASE;
  // MXFP8 weight waves: wave wid brings weight rows wid * 32 .. + 31's scale
  // words of each stage (lanes 32-63 repeat lanes 0-31 into the upper half of
  // its 256 bytes) into the slot that matches the weight slot.
  const uint8_t* wsrc = kMxW ? uniform_ptr(it.ws + it.k0 * 4) : nullptr;
  const uint32_t wbase = kMxW ? it.wsc_lds + (uint32_t)wid * 256u : 0u;
  uint32_t wdst = wbase;
  auto issue = [&]() __attribute__((always_inline)) {
    if constexpr (kW) {
      wl.weights(src, dst);
      dst = dst + B_BYTES == lds0 + B_RING ? lds0 : dst + B_BYTES;
      if constexpr (kMxW) {
        dma4(wsrc, wl.wsc_off, wdst);
        wsrc += blk + 1 == KB ? 4 - 4 * KB : 4;
        wdst = wdst + WSC_SLOT == wbase + kBSlots * WSC_SLOT ? wbase : wdst + WSC_SLOT;
      }
    } else {
      wl.template acts<ROLE, kSc>(src, dst, ssrc, sdst);
      dst = dst + it.a_slot_bytes == a_end ? lds0 + A_BASE : dst + it.a_slot_bytes;
      sdst = sdst + SC_SLOT == lds0 + SC_BASE + kScSlots * SC_SLOT ? lds0 + SC_BASE
                                                                    : sdst + SC_SLOT;
      ssrc += blk + 1 == KB ? it.as_kstride * (1 - KB) : it.as_kstride;
    }
    src += blk + 1 == KB ? (int64_t)BK * (1 - KB) : (int64_t)BK;
    blk = blk + 1 == KB ? 0 : blk + 1;
  };
  // Read-side slots of stage kb+1.
  uint32_t rb = lds0 + B_BYTES, ra = lds0 + A_BASE + it.a_slot_bytes;
  const uint32_t bsc = lds0 + BSC_BASE;

  // The item's weight block scales: issued before this wave's stage 0, so
  // the prologue's wait for stage 0 covers them too (loads complete in order).
  if constexpr (kSc && kFmt != kMX)
    if (wid == kWaves - 1) load_item_wscales(it, lds0, lane);
  // Prologue: stages 0..D-2 of the stream, wait for stage 0 with the rest
  // in flight; after the barrier, read stage 0's fragments and issue the
  // stream's next stage into the last free slot.
  const int pre = min(D - 1, KB);
  for (int q = 0; q < pre; ++q) issue();
  wait_ahead<NL, D - 2>(pre - 1);
  barrier();
  v8i a[FM], b[FN];
  StepScales<kFmt, NFM> ss;
  if constexpr (NFM > 0) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (kFmt == kMX) b[j] = frag2(lds0 + j * 2048, fo.b_mx_lo, fo.b_mx_hi);
      else b[j] = frag2(lds0 + j * 2048, fo.b_lo, fo.b_hi);
    }
#pragma unroll
    for (int i = 0; i < NFM; ++i) {
      if constexpr (kFmt == kMX) a[i] = frag2(lds0 + A_BASE + i * A_TILE_STRIDE, fo.a_mx_lo,
                                              fo.a_mx_hi);
      else a[i] = frag2(lds0 + A_BASE + i * A_TILE_STRIDE, fo.a_lo, fo.a_hi);
    }
    if constexpr (kFmt == kMX) {
      ss.load(lds0 + SC_BASE, it, fo, 0, lane);
      ss.advance();
    } else {
      ss.read(lds0 + SC_BASE, bsc, it, fo, 0, lane);
      if constexpr (kFmt == kU8) ss.finish(it, fo, 0, lane);
    }
  }
  if (pre < KB) issue();  // stages 0 .. min(D, KB) - 1 are now in flight
  // Read-side slot of stage kb+1's scales.
  uint32_t rsn = lds0 + SC_BASE + SC_SLOT;
  // Step kb (not the last): stage kb+1 must have landed, with `ahead` later
  // stages of this wave's stream still in flight; then the step, with the
  // stream's next stage (if any) issued in its shadow.
  auto body = [&](int kb, auto&& wait, auto&& issue_fn) __attribute__((always_inline)) {
    wait();
    wait_lgkm0();
    barrier();
    if constexpr (NFM > 0) {
      step<kFmt, NFM, true>(a, b, acc, ss, ra, rb, rsn, bsc, it, fo, kb, lane, issue_fn);
    } else {
      issue_fn();
    }
    rb = rb + B_BYTES == lds0 + B_RING ? lds0 : rb + B_BYTES;
    ra = ra + it.a_slot_bytes == a_end ? lds0 + A_BASE : ra + it.a_slot_bytes;
    rsn = rsn + SC_SLOT == lds0 + SC_BASE + kScSlots * SC_SLOT ? lds0 + SC_BASE : rsn + SC_SLOT;
  };
  // Steady state (kb < KB - D): D - 2 stages stay in flight and every step
  // issues one more (into the slots stage kb had), without a branch, so the
  // loads really sit in the shadow of the first MFMAs.
  int kb = 0;
  for (; kb < KB - D; ++kb)
    body(kb, [] { wait_vmcnt<(D - 2) * NL>(); }, issue);
  // Tail: every stage is issued; fewer remain in flight each step.
  for (; kb + 1 < KB; ++kb)
    body(kb, [&] { wait_ahead<NL, D - 2>(KB - kb - 2); }, [] {});
  // Last step: nothing left to read ahead or load.
  if constexpr (NFM > 0)
    step<kFmt, NFM, false>(a, b, acc, ss, 0u, 0u, 0u, bsc, it, fo, KB - 1, lane, [] {});
}

// The K loop instantiation for this wave's live-tile count and role.
template <int kFmt, int NFM>
__device__ __forceinline__ void kloop_role(int role, uint32_t lds0, v4f (&acc)[FM][FN],
                                           const Item& it, const WaveLoads& wl,
                                           const FragOffsets& fo, int lane, int wid) {
  switch (role) {  // uniform per wave
    case 0: kloop<kFmt, NFM, 0>(lds0, acc, it, wl, fo, lane, wid); break;
    case 1: kloop<kFmt, NFM, 1>(lds0, acc, it, wl, fo, lane, wid); break;
    case 2: kloop<kFmt, NFM, 2>(lds0, acc, it, wl, fo, lane, wid); break;
    case 3: kloop<kFmt, NFM, 3>(lds0, acc, it, wl, fo, lane, wid); break;
    case 4: kloop<kFmt, NFM, 4>(lds0, acc, it, wl, fo, lane, wid); break;
    case 5: kloop<kFmt, NFM, 5>(lds0, acc, it, wl, fo, lane, wid); break;
    case 6: kloop<kFmt, NFM, 6>(lds0, acc, it, wl, fo, lane, wid); break;
    case 7: kloop<kFmt, NFM, 7>(lds0, acc, it, wl, fo, lane, wid); break;
    default: kloop<kFmt, NFM, 8>(lds0, acc, it, wl, fo, lane, wid); break;
  }
}

// Row groups: expert e's block [start_e, end_e) (clamped to the valid rows)
// is cut into ceil(len / GM) groups.  Wave 0 writes gp (prefix of groups per
// expert, gp[E] = all) and pe (end of each expert's live rows) into LDS.
// kMasked: `psum` is masked_m, `align` is max_m.
template <bool kMasked>
__device__ __forceinline__ void build_groups(const int32_t* __restrict__ psum, int64_t nrows,
                                             int E, int align, int* gp, int* pe, int lane) {
  int run = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    int ng = 0;
    if (e < E) {
      if (kMasked) {  // slab: rows [e * max_m, + masked_m[e]), no padding
        const int64_t st = (int64_t)e * align;
        const int64_t en = st + max(0, min(psum[e], align));
        ng = (int)((en - st + GM - 1) / GM);
        pe[e] = (int)en;
      } else {
        const int p_e = psum[e];
        const int64_t st = e ? align_up_i(psum[e - 1], align) : 0;
        const int64_t en = min((int64_t)align_up_i(p_e, align), nrows);
        ng = en > st ? (int)((en - st + GM - 1) / GM) : 0;
        pe[e] = p_e;
      }
    }
    const int incl = wave_incl_scan_i(ng);
    if (e < E) gp[e] = run + incl - ng;
    run += __shfl(incl, 63, 64);
  }
  if (lane == 0) gp[E] = run;
}

// Work item `item` -> its Item (false: only alignment padding, nothing to
// compute); nt and m0 are its N tile and first row.  Expert e's items are
// [NT * gp[e], NT * gp[e + 1]), N-tile-major with its row groups innermost:
// the groups of one (expert, N tile) share a weight stream and run side by
// side on one XCD, so its L2 serves the weights to all but one of them.
template <int kFmt, bool kMasked>
__device__ __forceinline__ bool decode_item(
    int64_t item, const int* gp, const int* pe, int E, int NT, int KB, int K, int N,
    int64_t nrows, int align, int64_t capacity, const uint8_t* a, const uint8_t* a_scale,
    const uint8_t* w, const uint8_t* w_scale, int sbytes, uint32_t wsc_lds, Item& it, int& nt,
    int64_t& m0) {
  const int q = (int)(item / NT);
  int lo = 0, hi = E - 1;  // last e with gp[e] <= q
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (gp[mid] <= q) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int ge = gp[e + 1] - gp[e];  // row groups of expert e (>= 1 here)
  const int64_t local = item - (int64_t)NT * gp[e];
  nt = (int)(local / ge);
  const int gi = gp[e] + (int)(local % ge);
  const int64_t st = kMasked ? (int64_t)e * align : (e ? align_up_i(pe[e - 1], align) : 0);
  m0 = st + (int64_t)(gi - gp[e]) * GM;
  const int64_t live = min((int64_t)GM, min((int64_t)pe[e], nrows) - m0);
  if (live <= 0) return false;
  it.live = (int)live;
  it.K = K;
  it.KB = KB;
  // Staggered K start for the first round (see the header).
  it.k0 = item < (int64_t)gridDim.x ? (int)(((int64_t)nt * KB) / NT) : 0;
  it.sbytes = sbytes;
  it.blocks = ((int)live + 7) >> 3;
  it.na = (it.blocks + kLoadWaves - 1) / kLoadWaves;  // 1..8
  it.a_slot_bytes = it.na * 4096;
  it.na_slots = act_slots(it.na);
  it.a = a + m0 * K;
  it.b = w + ((int64_t)e * N + (int64_t)nt * BN) * K;
  it.ws = kFmt == kMX ? w_scale + ((int64_t)e * N + (int64_t)nt * BN) * (K / 32) : nullptr;
  it.wsc_lds = wsc_lds;
  it.as = a_scale + m0 * sbytes;
  it.as_kstride = capacity * sbytes;
  const int64_t b0 = ((int64_t)e * NT + nt) * KB * sbytes;  // byte of block 0's scale
  it.bs = w_scale + (b0 & ~(int64_t)3);
  it.bs_skew = (int)(b0 & 3);
  return true;
}

// kMasked: `psum` is masked_m, `align` is max_m, `status` is unused and the
// activation rows are the E * max_m slab rows (capacity).
template <int kFmt, bool kMasked>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_scale,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_scale,
    const int32_t* __restrict__ psum, const int32_t* __restrict__ status, int64_t capacity, int N,
    int K, int E, int align, uint16_t* __restrict__ out) {
  constexpr int kMaxE = kFmt == kMX ? kMxMaxExperts : MOE_MAX_EXPERTS;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  __shared__ int gp[kMaxE + 1];  // prefix of row groups per expert
  __shared__ int pe[kMaxE];      // end of each expert's live rows
  __shared__ __attribute__((aligned(16))) uint8_t wsc[kFmt == kMX ? kBSlots * WSC_SLOT : 16];
  const int t = threadIdx.x, lane = t & 63;
  const int wid = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform per wave
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const FragOffsets fo = frag_offsets(lane, wm, wn);
  const uint32_t lds0 = lds_addr(lds);
  const int64_t nrows = kMasked ? capacity : min((int64_t)status[0], capacity);
  const int sbytes = kFmt == kU8 ? 1 : (kFmt == kF32 || kFmt == kMX ? 4 : 0);
  const int KB = K / BK, NT = N / BN;

  if (wid == 0) build_groups<kMasked>(psum, nrows, E, align, gp, pe, lane);
  __syncthreads();
  const int64_t nitems = (int64_t)gp[E] * NT;
  const int per_xcd = gridDim.x / kXcds;
  const int64_t slot = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;

  for (int64_t item = slot; item < nitems; item += gridDim.x) {
    Item it;
    int nt;
    int64_t m0;
    if (!decode_item<kFmt, kMasked>(item, gp, pe, E, NT, KB, K, N, nrows, align, capacity, a,
                                     a_scale, w, w_scale, sbytes, lds_addr(wsc), it, nt, m0))
      continue;  // only alignment padding: nothing to compute
    // Live 16-row MFMA tiles of this wave, and the loads it issues per stage.
    const int nfm = (int)max(0, min(FM, (it.live - wm * 16 + ROW_TILE_STRIDE - 1) /
                                            ROW_TILE_STRIDE));

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    WaveLoads wl;
    wl.init(it, wid, lane, lds0);
    const int role = wid < kLoadWaves ? 0 : it.na;
    switch (nfm) {  // uniform per wave; one K loop per live-tile count and role
      case 4: kloop_role<kFmt, 4>(role, lds0, acc, it, wl, fo, lane, wid); break;
      case 3: kloop_role<kFmt, 3>(role, lds0, acc, it, wl, fo, lane, wid); break;
      case 2: kloop_role<kFmt, 2>(role, lds0, acc, it, wl, fo, lane, wid); break;
      case 1: kloop_role<kFmt, 1>(role, lds0, acc, it, wl, fo, lane, wid); break;
      default: kloop_role<kFmt, 0>(role, lds0, acc, it, wl, fo, lane, wid); break;
    }
    wait_lgkm0();
    barrier();  // every wave is done reading the slots

    // Epilogue.  The products are computed transposed (weights as the first
    // MFMA operand), so each lane holds 4 consecutive columns (8 bytes) of
    // one row per tile, and a direct store writes 32-byte pieces of 16 rows.
    // Instead each wave passes its 64 x 64 tile through LDS (its own 8 KB of
    // the idle ring; 16-byte chunks XOR-swizzled by row) and writes whole
    // 128-byte row segments: 8 rows per store instruction, live rows only.
    // (Measured: the layer step 3 us faster at the DeepSeek-V3 share, 40 us
    // at the prefill shape.)
    {
      const uint32_t stage = lds0 + (uint32_t)wid * 8192u;
      const int g = lane >> 4, f = lane & 15;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int rho = f + 16 * i;  // the wave's local row: global wm * 16 + f + 64 * i
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int c = (2 * j + (g >> 1)) ^ (rho & 7);
          typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
          lds_store<u32x2>(stage + (uint32_t)(rho * 128 + c * 16 + (g & 1) * 8),
                           u32x2{pk_bf16(acc[i][j][0], acc[i][j][1]),
                                 pk_bf16(acc[i][j][2], acc[i][j][3])});
        }
      }
      // A wave's LDS accesses are performed in order: the reads below see
      // the writes above.
      uint16_t* obase = out + m0 * N + (int64_t)nt * BN + wn * WTN + (lane & 7) * 8;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int rho = q * 8 + (lane >> 3);
        const u32x4 o =
            lds_load<u32x4>(stage + (uint32_t)(rho * 128 + (((lane & 7) ^ (rho & 7)) << 4)));
        const int r = wm * 16 + (rho & 15) + 64 * (rho >> 4);
        if (r < it.live) *reinterpret_cast<u32x4*>(obase + (int64_t)r * N) = o;
      }
      wait_lgkm0();
      barrier();  // every wave is done with its staging area before the next item's loads
    }
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

// One workgroup per CU (the kernel uses ~154 KB of LDS), a whole number per
// XCD, never more than the largest possible number of work items.
// kind: kF32, kU8 or kBF; k is the operand row length in bytes (bf16: 2 per
// value), so every address in the kernel is a byte offset.
moe_status launch_gemm(bool masked, const void* a, const void* a_scale, int kind,
                       const void* w, const void* w_scale, const int32_t* psum,
                       const int32_t* status, int64_t capacity, int n, int k, int num_experts,
                       int align, void* out, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t max_items = ((capacity + GM - 1) / GM + num_experts) * (int64_t)(n / BN);
  int64_t grid = device_cus();
  if (grid > max_items) grid = max_items;
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  auto kern = kind == kMX   ? grouped_gemm_kernel<kMX, false>
              : kind == kU8 ? (masked ? grouped_gemm_kernel<kU8, true>
                                      : grouped_gemm_kernel<kU8, false>)
              : kind == kBF ? (masked ? grouped_gemm_kernel<kBF, true>
                                      : grouped_gemm_kernel<kBF, false>)
                            : (masked ? grouped_gemm_kernel<kF32, true>
                                      : grouped_gemm_kernel<kF32, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, s, (const uint8_t*)a,
                     (const uint8_t*)a_scale, (const uint8_t*)w, (const uint8_t*)w_scale, psum,
                     status, capacity, n, k, num_experts, align, (uint16_t*)out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
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
  if (fmt != MOE_SCALE_F32 && fmt != MOE_SCALE_UE8M0 && fmt != MOE_SCALE_MXFP8)
    return MOE_ERR_UNSUPPORTED;
  if (fmt == MOE_SCALE_MXFP8 && num_experts > kMxMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (!psum || !status || !w || !w_scale) return MOE_ERR_NULL;
  if (capacity > 0 && (!a || !a_scale || !out)) return MOE_ERR_NULL;
  if (k / BK > MAX_KB) return MOE_ERR_UNSUPPORTED;
  if (((uintptr_t)a % 16) || ((uintptr_t)w % 16) || ((uintptr_t)out % 16) ||
      ((uintptr_t)a_scale % (fmt == MOE_SCALE_UE8M0 ? 4 : 16)) || ((uintptr_t)w_scale % 4))
    return MOE_ERR_ALIGNMENT;
  if (capacity == 0) return MOE_OK;
  const int kind = fmt == MOE_SCALE_MXFP8 ? kMX : (fmt == MOE_SCALE_UE8M0 ? kU8 : kF32);
  return launch_gemm(false, a, a_scale, kind, w, w_scale, psum, status, capacity, n, k,
                     num_experts, align, out, stream);
}

extern "C" moe_status moe_grouped_gemm_bf16(const void* a, const void* w, const int32_t* psum,
                                           const int32_t* status, int64_t capacity, int n,
                                           int k, int num_experts, int align, void* out,
                                           void* stream) {
  if (capacity < 0 || capacity > (1LL << 30) || n <= 0 || k <= 0 || n % BN || k % 64 ||
      num_experts < 1 || num_experts > MOE_MAX_EXPERTS)
    return MOE_ERR_SHAPE;
  if (align < MOE_MIN_ALIGN || align > MOE_MAX_ALIGN || (align & (align - 1)))
    return MOE_ERR_UNSUPPORTED;
  if (capacity % align != 0) return MOE_ERR_SHAPE;
  if (!psum || !status || !w) return MOE_ERR_NULL;
  if (capacity > 0 && (!a || !out)) return MOE_ERR_NULL;
  if (2 * k / BK > MAX_KB) return MOE_ERR_UNSUPPORTED;
  if (((uintptr_t)a % 16) || ((uintptr_t)w % 16) || ((uintptr_t)out % 16))
    return MOE_ERR_ALIGNMENT;
  if (capacity == 0) return MOE_OK;
  return launch_gemm(false, a, nullptr, kBF, w, nullptr, psum, status, capacity, n, 2 * k,
                     num_experts, align, out, stream);
}

extern "C" moe_status moe_grouped_gemm_fp8_masked(const void* a, const void* a_scale,
                                                  moe_scale_fmt fmt, const void* w,
                                                  const void* w_scale, const int32_t* masked_m,
                                                  int max_m, int n, int k, int num_experts,
                                                  void* out, void* stream) {
  if (max_m < 0 || max_m > (1 << 24) || n <= 0 || k <= 0 || n % BN || k % BK ||
      num_experts < 1 || num_experts > MOE_MAX_EXPERTS ||
      (int64_t)max_m * num_experts > (1LL << 30))
    return MOE_ERR_SHAPE;
  if (fmt != MOE_SCALE_F32 && fmt != MOE_SCALE_UE8M0) return MOE_ERR_UNSUPPORTED;
  if (!masked_m || !w || !w_scale) return MOE_ERR_NULL;
  if (max_m > 0 && (!a || !a_scale || !out)) return MOE_ERR_NULL;
  if (k / BK > MAX_KB) return MOE_ERR_UNSUPPORTED;
  if (((uintptr_t)a % 16) || ((uintptr_t)w % 16) || ((uintptr_t)out % 16) ||
      ((uintptr_t)a_scale % (fmt == MOE_SCALE_F32 ? 16 : 4)) || ((uintptr_t)w_scale % 4))
    return MOE_ERR_ALIGNMENT;
  // Every expert's slab starts on a 16-row boundary (the UE8M0 scale loads
  // read aligned 4-byte words of a row group's scales).
  if (max_m % 16) return MOE_ERR_SHAPE;
  const int64_t rows = (int64_t)max_m * num_experts;
  if (rows == 0) return MOE_OK;
  return launch_gemm(true, a, a_scale, fmt == MOE_SCALE_UE8M0 ? kU8 : kF32, w, w_scale,
                     masked_m, nullptr, rows, n, k, num_experts, max_m, out, stream);
}
