/*
 * moe_expand.h -- C ABI of libmoe_expand.so: one expert-parallel rank's MoE
 * expert computation on the expanded dispatch layout, for AMD Instinct
 * MI355X (gfx950).
 *
 * The path, in call order (all on one HIP stream, no host synchronisation,
 * no host read of device data):
 *
 *   moe_expand_layout     received fp8 tokens + top-k ids/weights
 *                          -> per-(token, expert) rows grouped by expert,
 *                             each expert block padded to `align` rows,
 *                             row->expert labels, slot->row map, psum
 *   moe_grouped_gemm_fp8  gate_up projection (w13), bf16 out
 *   moe_act_quant         SiLU(gate)*up, per-1x128 fp8 quantisation, and
 *                          (fp32 scales) the top-k weight folded into the
 *                          down projection's input scale
 *   moe_grouped_gemm_fp8  down projection (w2), bf16 out
 *   moe_gather            each token's expert rows summed back into one
 *                          bf16 row (weighted here under UE8M0 scales)
 *
 * The standard (non-EP) path [P3 pre_permute_standard_to_deep_gemm,
 * post_permute_deep_gemm_to_standard] uses the same calls, entering with
 * moe_expand_layout_bf16 (bf16 token rows, quantised per 1x128 group while
 * they are scattered) and leaving through moe_gather with the top-k weights
 * and the routed scaling factor.
 *
 * The decode path's masked slab [P1 "Why decode stays on V1 low_latency";
 * P3 pre_permute_deepep_v2_to_deep_gemm / post_permute_deep_gemm_to_
 * deepep_v2, masked branches; _run_masked_gemm] runs after moe_expand_layout:
 *   moe_expand_to_masked_slab    expanded rows -> fixed-height slab
 *                                [num_experts, max_m, hidden], masked_m
 *   moe_grouped_gemm_fp8_masked  gate_up on each expert's masked_m rows
 *   moe_act_quant_masked         SiLU(gate)*up + per-1x128 quantisation
 *   moe_grouped_gemm_fp8_masked  down
 *   moe_masked_slab_to_expand    back to the expanded rows, times the top-k
 *                                weights
 *   moe_gather                   combine with weight 1
 *
 * Sources, by page and section:
 *  [P1] SGLang pull request 37261, "feat(deepep_v2): expanded (do_expand=True)
 *       prefill dispatch for DeepEP-V2": Modifications/Core (row labels from
 *       the device psum with no cumsum, host copy or sentinel; the weight
 *       fold into down_proj's fp32 input scale and the UE8M0 fallback), the
 *       SGLANG_DEEPEP_V2_PREFILL_DO_EXPAND section (expanded rows grouped by
 *       expert), and the review thread's note on the expand-mode psum
 *       (psum[e] = align(psum[e-1]) + count[e]; total rows = align(psum[E-1])).
 *  [P2] vLLM pull request 54109, PaddedStandard activation format:
 *       Motivation (inactive rows carry -1 in every top-k slot; the real /
 *       padding boundary psum_recv_per_rank lives on the device; prefill
 *       alignment gaps are zeroed) and Design (the kernel must skip inactive
 *       rows or make them safe to discard, and honour -1 markers rather than
 *       trust row contents).
 *  [P3] SGLang moe_runner/deep_gemm.py source page: _run_contiguous_gemm
 *       (gate_up GEMM, SiLU*up, per-token-group fp8 quant, down GEMM),
 *       _get_compact_all_tokens (capacity bound), _cast_to_e8m0_with_
 *       rounding_up (UE8M0 rule), pre_permute_deepep_v2_to_deep_gemm and
 *       post_permute_deep_gemm_to_deepep_v2 (expanded branch),
 *       pre_permute_standard_to_deep_gemm (bf16 rows quantised per token
 *       group, then scattered into 128-aligned expert blocks) and
 *       post_permute_deep_gemm_to_standard (top-k weights and the routed
 *       scaling factor in the reduction).
 *
 * Conventions for every call:
 *  - Pointers named as device buffers are device memory the caller owns
 *    (allocated, e.g., by PyTorch).  The library never allocates, frees,
 *    copies between host and device, synchronises, or reads device data on
 *    the host.  `stream` is a hipStream_t (NULL = the default stream); work
 *    is enqueued asynchronously on it.
 *  - Host-detectable errors (null pointers, bad sizes, misaligned buffers,
 *    unsupported combinations) are returned as a moe_status before anything
 *    is launched, and nothing is written.  MOE_ERR_LAUNCH reports a failed
 *    kernel launch.
 *  - Device-detected conditions are OR-ed into status[1] by
 *    moe_expand_layout (MOE_FLAG_*); later calls clamp to what is valid.
 *  - fp8 is OCP E4M3 ("fn": bias 7, max 448, no infinities).  bf16 buffers
 *    hold raw 16-bit patterns.  fp32 scales are IEEE float; UE8M0 scales are
 *    one unsigned exponent byte per group, value 2^(b-127).
 *  - Scales: one per 1x128 activation group, one per 128x128 weight block.
 *    The received rows' x_scale is row-major [rows, K/128].  The expanded
 *    activation scales that moe_expand_layout and moe_act_quant write and
 *    moe_grouped_gemm_fp8 reads are K-block-major ("MN-major")
 *    [K/128, capacity]: the scale of expanded row m, K block b sits at
 *    b * capacity + m, so one K block's scales for consecutive rows are one
 *    contiguous run (the GEMM of [P3 _run_contiguous_gemm] likewise takes its
 *    activation scales transposed: TMA-aligned, or mn-major under UE8M0).
 *    Weight scales are [E, N/128, K/128].
 *  - Calls are stateless and reentrant; calls that share output buffers
 *    must be ordered by the caller's streams.
 */
#ifndef MOE_EXPAND_H
#define MOE_EXPAND_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,         /* a required pointer is NULL                 */
  MOE_ERR_SHAPE = 2,        /* a size is out of range or inconsistent     */
  MOE_ERR_ALIGNMENT = 3,    /* a pointer or stride is not 16-byte aligned */
  MOE_ERR_UNSUPPORTED = 4,  /* valid in principle, not supported          */
  MOE_ERR_WORKSPACE = 5,    /* workspace missing or too small             */
  MOE_ERR_LAUNCH = 6,       /* a kernel launch (or, for
                               moe_expand_layout_noalloc, the lookup of its
                               scratch address) failed                    */
  MOE_ERR_SCRATCH = 7       /* moe_expand_layout_noalloc: the sizes need
                               more workspace than its static scratch
                               (MOE_NOALLOC_SCRATCH_BYTES) holds          */
} moe_status;

typedef enum {
  MOE_SCALE_F32 = 0,        /* fp32 scale per group                       */
  MOE_SCALE_UE8M0 = 1,      /* one power-of-two exponent byte per group   */
  MOE_SCALE_NONE = 2,       /* moe_expand_layout_bf16 only: keep the rows in
                               bf16, no quantisation, no scales (the bf16-
                               weight path)                               */
  MOE_SCALE_MXFP8 = 3       /* MXFP8: one UE8M0 byte per 1x32 group along K,
                               for activations and for every weight row
                               [P3 DeepGemmMoeQuantInfo: block [1, 32]];
                               activation scales [rows, K/32] bytes
                               (x_scale_stride in bytes, a multiple of 4),
                               expanded ones as one 4-byte word per
                               (128-wide K block, row): the block's four
                               bytes in K order, K-block-major; weight
                               scales [E, N, K/32] bytes.  Supported by
                               moe_expand_layout, moe_grouped_gemm_fp8 (at
                               most 256 experts), moe_act_quant (no fold)  */
} moe_scale_fmt;

/* Bits of status[1] written by moe_expand_layout. */
#define MOE_FLAG_CAPACITY_OVERFLOW 1 /* total rows > capacity: rows at or past
                                        the capacity were dropped (their slots
                                        get -1)                               */
#define MOE_FLAG_EXPERT_ID_RANGE 2   /* a valid row held an id >= num_experts;
                                        that slot was skipped                 */
#define MOE_FLAG_SLAB_OVERFLOW 4     /* (moe_expand_to_masked_slab) an expert
                                        had more than max_m live rows; rows
                                        past max_m were dropped               */

/* Limits of this build. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32
#define MOE_MIN_ALIGN 16
#define MOE_MAX_ALIGN 1024
/* Size of moe_expand_layout_noalloc's static per-GPU scratch: calls with
 * moe_expand_workspace_bytes(rows, topk, num_experts) above it are refused
 * (roughly rows * num_experts <= 15 million). */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)

/* Text for a moe_status value (static storage; never NULL). */
const char* moe_status_string(int status);

/* Host, pure.  Largest padded row total over every routing of rows*topk
 * assignments onto num_experts experts with blocks rounded up to `align`
 * rows: align * (n + (rows*topk - n) / align), n = min(rows*topk, E)
 * [P3 _get_compact_all_tokens].  Use it to size the expanded buffers
 * without reading the device-side row count.  Returns -1 on bad input. */
int64_t moe_expand_capacity(int64_t rows, int topk, int num_experts, int align);

/* Host, pure.  Bytes of device workspace moe_expand_layout needs for
 * `rows` receive-buffer rows.  Returns 0 on bad input. */
size_t moe_expand_workspace_bytes(int64_t rows, int topk, int num_experts);

/*
 * Expanded layout [P1 Core + psum note; P2 Motivation/Design; P3
 * pre_permute_deepep_v2_to_deep_gemm].
 *
 * Inputs (device):
 *   x              [rows, x_stride] bytes, fp8 token rows (hidden bytes used)
 *   x_scale        [rows, x_scale_stride] fp32 or UE8M0 bytes (by fmt)
 *   topk_ids       [rows, topk] int32; id < 0 = not for this rank / inactive;
 *                  id >= num_experts is skipped and flagged
 *   topk_weights   [rows, topk] fp32; may be NULL only if row_weight is NULL
 *   psum_recv_per_rank [num_src_ranks] int32 inclusive prefix sum of rows
 *                  received per source rank; its last entry is the number of
 *                  valid rows R_v (clamped to [0, rows]).  NULL: R_v = rows.
 *                  Rows >= R_v are never read as routing.
 * Sizes: hidden % 128 == 0; 1 <= topk <= MOE_MAX_TOPK; 1 <= num_experts <=
 *   MOE_MAX_EXPERTS; align a power of two in [16, 1024]; capacity a multiple
 *   of align (moe_expand_capacity gives one that cannot overflow);
 *   x_stride % 16 == 0 and x 16-byte aligned.
 * Outputs (device, caller-allocated):
 *   ex             [capacity, hidden] fp8 expanded rows
 *   ex_scale       [hidden/128, capacity] K-block-major scales (same
 *                  format as x_scale): row m, block b at b * capacity + m
 *   psum           [num_experts] int32, psum[e] = align(psum[e-1]) + count[e]
 *   m_indices      [capacity] int32: expert of each expanded row, alignment
 *                  pads included; -1 from the total to the capacity
 *   src2dst        [rows, topk] int32: expanded row of each live slot, -1
 *                  otherwise (all slots of rows >= R_v are -1)
 *   row_weight     [capacity] fp32 top-k weight of each expanded row (0 on
 *                  pads); may be NULL
 *   status         [2] int32: status[0] = total expanded rows
 *                  align(psum[E-1]) (may exceed capacity: see the flag),
 *                  status[1] = MOE_FLAG_* bits
 * Rows of one expert are in ascending (row, k) order.  Alignment pad rows
 * get fp8 zero, scale 0 and weight 0.  Rows from the total up to the
 * capacity are left untouched.
 * workspace: device, >= moe_expand_workspace_bytes(rows, topk, num_experts)
 *   bytes, 256-byte aligned, no initialisation needed.
 */
moe_status moe_expand_layout(
    const void* x, int64_t x_stride, const void* x_scale,
    int64_t x_scale_stride, moe_scale_fmt fmt,
    const int32_t* topk_ids, const float* topk_weights,
    const int32_t* psum_recv_per_rank, int num_src_ranks,
    int64_t rows, int hidden, int topk, int num_experts, int align,
    int64_t capacity,
    void* ex, void* ex_scale, int32_t* psum, int32_t* m_indices,
    int32_t* src2dst, float* row_weight, int32_t* status,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_expand_layout with no workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Every other argument, output and error
 * is as moe_expand_layout's; the call allocates and frees nothing.
 *
 * The workspace is a static device array of MOE_NOALLOC_SCRATCH_BYTES inside
 * the library: each GPU the library runs on holds its own copy until the
 * process ends.  Its address is looked up on the first call on each device
 * (that call must have the device current, as every call must).  Sizes whose
 * workspace (moe_expand_workspace_bytes) exceeds the array return
 * MOE_ERR_SCRATCH before anything is launched; a failed address lookup
 * returns MOE_ERR_LAUNCH.  All calls on one GPU share the array: calls that
 * may run concurrently on one GPU (unordered streams) race and must not be
 * issued; calls ordered on one stream are safe, and nothing needs clearing
 * between them.
 */
moe_status moe_expand_layout_noalloc(
    const void* x, int64_t x_stride, const void* x_scale,
    int64_t x_scale_stride, moe_scale_fmt fmt,
    const int32_t* topk_ids, const float* topk_weights,
    const int32_t* psum_recv_per_rank, int num_src_ranks,
    int64_t rows, int hidden, int topk, int num_experts, int align,
    int64_t capacity,
    void* ex, void* ex_scale, int32_t* psum, int32_t* m_indices,
    int32_t* src2dst, float* row_weight, int32_t* status, void* stream);

/*
 * Expanded layout of bf16 token rows, quantised on the way [P3
 * pre_permute_standard_to_deep_gemm: per-token-group fp8 quantisation of the
 * hidden states, then the scatter into the aligned expert blocks].
 *
 * As moe_expand_layout, except:
 *   x          [rows, x_stride] bf16 token rows (x_stride in elements,
 *              >= hidden; x_stride * 2 % 16 == 0, x 16-byte aligned); there
 *              is no x_scale.  Each valid row with a live slot is read once,
 *              quantised per 1x128 group and written to every destination:
 *                amax = max(max |x| over the group, 1e-10)
 *                fp32:  scale = amax / 448, q = fp8_rne(x * (448 / amax))
 *                UE8M0: b = smallest exponent byte with 2^(b-127) >= amax/448,
 *                       q = fp8_rne(x * 2^(127-b))
 *              (each operation rounded in fp32; the same rule as
 *              moe_act_quant's).  Rows without a live slot are not read.
 *              fmt MOE_SCALE_NONE (the bf16-weight path): the rows are kept
 *              in bf16 and copied as they are; ex is then [capacity, hidden]
 *              bf16, ex_scale is not used (may be NULL), pad rows are 0.
 * Errors, ownership and every other argument: as moe_expand_layout.
 */
moe_status moe_expand_layout_bf16(
    const void* x, int64_t x_stride, moe_scale_fmt fmt,
    const int32_t* topk_ids, const float* topk_weights,
    const int32_t* psum_recv_per_rank, int num_src_ranks,
    int64_t rows, int hidden, int topk, int num_experts, int align,
    int64_t capacity,
    void* ex, void* ex_scale, int32_t* psum, int32_t* m_indices,
    int32_t* src2dst, float* row_weight, int32_t* status,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Contiguous grouped fp8 GEMM, "NT": out[m, :] = A[m, :] . W[e]^T for every
 * expanded row m of expert e [P3 _run_contiguous_gemm; P1 Core].
 *
 *   a        [capacity, k] fp8 (row stride k), a_scale [k/128, capacity]
 *            K-block-major (row m, block b at b * capacity + m)
 *   w        [num_experts, n, k] fp8 (k contiguous), w_scale
 *            [num_experts, n/128, k/128]; a_scale and w_scale in `fmt`
 *   psum, status  as written by moe_expand_layout
 *   out      [capacity, n] bf16
 * Expert e owns rows [align(psum[e-1]), align(psum[e])) -- exactly the rows
 * moe_expand_layout labels e in m_indices -- so the kernel reads the layout
 * from the device psum (no per-row labels needed).  For every such row
 * m < min(status[0], capacity):
 *   out[m,j] = bf16( sum_kb sa[m,kb] * sw[e,j/128,kb] *
 *                    sum_{t in kb} a[m,t] * w[e,j,t] )
 * accumulated in fp32 (UE8M0: the exponents are applied by the matrix
 * cores).  Row groups made only of alignment padding (rows >= psum[e]) may
 * be skipped and left unwritten; rows past the total are never written.
 * Sizes: n % 128 == 0, k % 128 == 0, k / 128 <= 511 (else
 * MOE_ERR_UNSUPPORTED), align as for the layout, capacity a multiple of
 * align.  Alignment: a, w, out 16 bytes; a_scale 16 bytes (fp32) or 4
 * (UE8M0); w_scale 4 bytes.  UE8M0 scale arrays are read in aligned 4-byte
 * words, so their allocations must extend to a multiple of 4 bytes.
 */
moe_status moe_grouped_gemm_fp8(
    const void* a, const void* a_scale, moe_scale_fmt fmt,
    const void* w, const void* w_scale,
    const int32_t* psum, const int32_t* status,
    int64_t capacity, int n, int k, int num_experts, int align,
    void* out, void* stream);

/*
 * SiLU(gate)*up with per-1x128 fp8 quantisation [P3 _run_contiguous_gemm,
 * _situ_mul_quant_contig_kernel (quantisation rule), _cast_to_e8m0_with_
 * rounding_up; P1 Core (fold)].
 *
 *   gate_up   [capacity, 2*inter] bf16: gate = first half, up = second
 *   m_indices, psum, status  as written by moe_expand_layout
 *   fold_weight  [capacity] fp32 (the layout's row_weight) or NULL.  Only
 *                with MOE_SCALE_F32 (UE8M0 + fold -> MOE_ERR_UNSUPPORTED).
 *   out       [capacity, inter] fp8; out_scale [inter/128, capacity] in fmt,
 *             K-block-major (row m, group g at g * capacity + m)
 * For each live row m (m < min(status[0], capacity), m < psum[e]):
 *   y = g / (1 + exp(-g)) * u in fp32; per group amax = max(|y|, 1e-10);
 *   F32:   s = amax / 448, q = fp8_rne(y * (448 / amax)), s *= fold_weight[m]
 *   UE8M0: b = smallest power-of-two exponent byte with 2^(b-127) >= amax/448,
 *          q = fp8_rne(y * 2^(127-b))
 * Alignment pad rows (psum[e] <= m < align(psum[e])) get q = 0, scale 0.
 * Sizes: inter % 128 == 0; gate_up and out 16-byte aligned.
 */
moe_status moe_act_quant(
    const void* gate_up, const int32_t* m_indices, const int32_t* psum,
    const int32_t* status, int64_t capacity, int inter, int num_experts,
    int align, moe_scale_fmt fmt, const float* fold_weight,
    void* out, void* out_scale, void* stream);

/*
 * Weighted gather back to token rows [P3 post_permute_deep_gemm_to_deepep_v2
 * and ep_gather's use in post_permute_deep_gemm_to_deepep_normal; P1 Core
 * (UE8M0 weighting of the down output); P3 post_permute_deep_gemm_to_standard
 * (the routed scaling factor)].
 *
 *   expert_out   [capacity, hidden] bf16 (down projection output)
 *   src2dst      [rows, topk] int32 as written by moe_expand_layout;
 *                entries outside [0, capacity) are treated as -1
 *   topk_weights [rows, topk] fp32, or NULL when the weights were folded
 *   routed_scaling_factor  multiplies each row's sum (1 on the expand path;
 *                the model's factor on the standard path); a NaN or infinite
 *                factor is MOE_ERR_UNSUPPORTED
 *   psum_recv_per_rank / num_src_ranks  as for the layout (R_v)
 *   out          [rows, hidden] bf16
 * For r < R_v: out[r] = bf16( f * sum over k ascending with src2dst[r,k] >= 0
 *   of c_k * float(expert_out[src2dst[r,k]]) ), c_k = topk_weights[r,k] or 1,
 * f = routed_scaling_factor, each product and sum rounded to fp32 in that
 * order.  Valid rows with no live slot become 0.  Rows >= R_v are not
 * written.
 * Sizes: hidden % 128 == 0 and hidden <= 8192 (else MOE_ERR_UNSUPPORTED);
 * buffers 16-byte aligned.
 */
moe_status moe_gather(
    const void* expert_out, const int32_t* src2dst, const float* topk_weights,
    float routed_scaling_factor, const int32_t* psum_recv_per_rank, int num_src_ranks,
    int64_t rows, int hidden, int topk, int64_t capacity,
    void* out, void* stream);

/*
 * Expanded rows -> the decode path's masked slab [P1 "Why decode stays on V1
 * low_latency": the fixed-height slab and the bridge into it; P3
 * pre_permute_deepep_v2_to_deep_gemm, masked branch].
 *
 *   ex, ex_scale   as written by moe_expand_layout (scales [hidden/128,
 *                  capacity] K-block-major), psum and status likewise
 *   slab           [num_experts * max_m, hidden] fp8: row e * max_m + i =
 *                  expanded row align(psum[e-1]) + i for i < masked_m[e]
 *   slab_scale     [hidden/128, num_experts * max_m] K-block-major
 *   masked_m       [num_experts] int32 = min(live rows of e, max_m)
 * Slab rows past masked_m[e] are not written.  An expert with more than
 * max_m live rows sets MOE_FLAG_SLAB_OVERFLOW in status[1] (written here:
 * status is read-write) and its rows past max_m are dropped.
 * Sizes: max_m >= 16 and a multiple of 16; num_experts * max_m <= 2^30.
 */
moe_status moe_expand_to_masked_slab(
    const void* ex, const void* ex_scale, moe_scale_fmt fmt, const int32_t* psum,
    int32_t* status, int64_t capacity, int hidden, int num_experts, int align, int max_m,
    void* slab, void* slab_scale, int32_t* masked_m, void* stream);

/*
 * Contiguous grouped bf16 GEMM, "NT" [P3 _run_bf16_contiguous_gemm,
 * grouped_gemm_nt_bf16_contig]: as moe_grouped_gemm_fp8 with bf16 operands
 * and no scales.
 *   a    [capacity, k] bf16, w [num_experts, n, k] bf16 (k contiguous)
 *   out  [capacity, n] bf16: the fp32 sum of the bf16 products rounded once
 * Sizes: n % 128 == 0, k % 64 == 0; buffers 16-byte aligned.
 */
moe_status moe_grouped_gemm_bf16(
    const void* a, const void* w, const int32_t* psum, const int32_t* status,
    int64_t capacity, int n, int k, int num_experts, int align, void* out,
    void* stream);

/*
 * SiLU(gate)*up to bf16 for every live expanded row [P3
 * _run_bf16_contiguous_gemm: silu_and_mul between the bf16 GEMMs]:
 *   gate_up  [capacity, 2*inter] bf16 -> out [capacity, inter] bf16,
 *   y = bf16_rne(silu(g) * u) with silu(g) = g / (1 + exp(-g)), in fp32.
 * Alignment pad rows are not written (the GEMM never reads them).
 */
moe_status moe_silu_mul_bf16(
    const void* gate_up, const int32_t* m_indices, const int32_t* psum,
    const int32_t* status, int64_t capacity, int inter, int num_experts,
    int align, void* out, void* stream);

/*
 * Masked grouped fp8 GEMM [P3 _run_masked_gemm]: as moe_grouped_gemm_fp8 on
 * the slab, expert e's rows being [e * max_m, e * max_m + masked_m[e]).
 *   a        [num_experts * max_m, k] fp8, a_scale [k/128, num_experts * max_m]
 *   w, w_scale as moe_grouped_gemm_fp8
 *   out      [num_experts * max_m, n] bf16; rows past masked_m[e] unwritten
 * Sizes: max_m a multiple of 16; n, k multiples of 128.
 */
moe_status moe_grouped_gemm_fp8_masked(
    const void* a, const void* a_scale, moe_scale_fmt fmt, const void* w,
    const void* w_scale, const int32_t* masked_m, int max_m, int n, int k,
    int num_experts, void* out, void* stream);

/*
 * SiLU(gate)*up and per-1x128 fp8 quantisation of the slab's live rows
 * [P3 _run_masked_gemm's activation; the rule of moe_act_quant, no fold]:
 *   gate_up  [num_experts * max_m, 2*inter] bf16
 *   out      [num_experts * max_m, inter] fp8, out_scale [inter/128,
 *            num_experts * max_m] K-block-major
 * Rows past masked_m[e] are neither read nor written.
 */
moe_status moe_act_quant_masked(
    const void* gate_up, const int32_t* masked_m, int max_m, int inter,
    int num_experts, moe_scale_fmt fmt, void* out, void* out_scale, void* stream);

/*
 * The slab's down rows back to the expanded layout [P1 "Why decode stays on
 * V1 low_latency"; P3 post_permute_deep_gemm_to_deepep_v2, masked branch:
 * the top-k weights are applied here, the expanded combine takes none].
 *   slab_out    [num_experts * max_m, hidden] bf16
 *   masked_m, max_m  as written / used by moe_expand_to_masked_slab
 *   psum, status, m_indices  from moe_expand_layout
 *   row_weight  [capacity] fp32 top-k weight of each expanded row, or NULL
 *   out         [capacity, hidden] bf16: for every expanded row m below the
 *               total, of expert e at i = m - align(psum[e-1]):
 *               bf16(row_weight[m] * slab_out[e * max_m + i]) if i <
 *               masked_m[e] (fp32 product, one rounding; a copy when
 *               row_weight is NULL); 0 for rows the slab height dropped
 *               (masked_m[e] <= i < psum[e] - align(psum[e-1])).  Alignment
 *               pad rows and rows past the total are not written.
 */
moe_status moe_masked_slab_to_expand(
    const void* slab_out, const int32_t* masked_m, int max_m, const int32_t* psum,
    const int32_t* status, const int32_t* m_indices, const float* row_weight,
    int64_t capacity, int hidden, int num_experts, int align, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EXPAND_H */
