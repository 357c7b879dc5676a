"""Python binding of libmoe_expand.so (gfx950): one expert-parallel rank's
MoE expert computation on the expanded dispatch layout.

Argument marshalling only.  Every step of the path runs in the library's HIP
kernels; torch is used for device memory and the current HIP stream.  The
binding raises if the library is missing: there is no fallback.

Functions mirror the C ABI in ``include/moe_expand.h``:

    moe_expand_layout, moe_expand_layout_noalloc, moe_expand_layout_bf16,
    moe_grouped_gemm_fp8,
    moe_act_quant, moe_gather, moe_expand_to_masked_slab,
    moe_grouped_gemm_fp8_masked, moe_act_quant_masked, moe_masked_slab_to_expand,
    moe_grouped_gemm_bf16, moe_silu_mul_bf16,
    moe_expand_capacity, moe_expand_workspace_bytes, moe_status_string

plus :class:`ExpandedMoE`, which allocates the buffers once for a given
receive-buffer size and runs the five calls of a layer in order, and
:class:`StandardMoE`, the same for the standard (non-EP) path: bf16 token
rows in, top-k weights and the routed scaling factor applied in the gather,
:class:`MaskedMoE`, the decode path on a fixed-height masked slab, and
:class:`StandardBf16MoE`, the standard path with bf16 weights.
"""

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_expand.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moe_expand.h")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGNMENT = 0, 1, 2, 3
MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH, MOE_ERR_SCRATCH = 4, 5, 6, 7
MOE_NOALLOC_SCRATCH_BYTES = 4 << 20
MOE_SCALE_F32, MOE_SCALE_UE8M0, MOE_SCALE_NONE, MOE_SCALE_MXFP8 = 0, 1, 2, 3
MOE_FLAG_CAPACITY_OVERFLOW, MOE_FLAG_EXPERT_ID_RANGE, MOE_FLAG_SLAB_OVERFLOW = 1, 2, 4
FMT = {"f32": MOE_SCALE_F32, "ue8m0": MOE_SCALE_UE8M0, "none": MOE_SCALE_NONE,
       "mxfp8": MOE_SCALE_MXFP8}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_expand_capacity": (_I64, [_I64, _I, _I, _I]),
    "moe_expand_workspace_bytes": (_SZ, [_I64, _I, _I]),
    "moe_expand_layout": (_I, [_P, _I64, _P, _I64, _I, _P, _P, _P, _I, _I64, _I, _I,
                               _I, _I, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_expand_layout_noalloc": (_I, [_P, _I64, _P, _I64, _I, _P, _P, _P, _I, _I64, _I, _I,
                                       _I, _I, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expand_layout_bf16": (_I, [_P, _I64, _I, _P, _P, _P, _I, _I64, _I, _I, _I, _I,
                                    _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_gemm_fp8": (_I, [_P, _P, _I, _P, _P, _P, _P, _I64, _I, _I, _I, _I,
                                  _P, _P]),
    "moe_act_quant": (_I, [_P, _P, _P, _P, _I64, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_gather": (_I, [_P, _P, _P, ctypes.c_float, _P, _I, _I64, _I, _I, _I64, _P, _P]),
    "moe_expand_to_masked_slab": (_I, [_P, _P, _I, _P, _P, _I64, _I, _I, _I, _I, _P, _P, _P,
                                       _P]),
    "moe_grouped_gemm_fp8_masked": (_I, [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "moe_act_quant_masked": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "moe_masked_slab_to_expand": (_I, [_P, _P, _I, _P, _P, _P, _P, _I64, _I, _I, _I, _P, _P]),
    "moe_grouped_gemm_bf16": (_I, [_P, _P, _P, _P, _I64, _I, _I, _I, _I, _P, _P]),
    "moe_silu_mul_bf16": (_I, [_P, _P, _P, _P, _I64, _I, _I, _I, _P, _P]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {status_string(code)} (status {code})")
        self.code = code


def lib():
    """Load libmoe_expand.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python expanded_dispatch_layout_amd/build.py` (hipcc, gfx950)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def header_functions():
    """Names of the functions include/moe_expand.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def status_string(code: int) -> str:
    return lib().moe_status_string(int(code)).decode()


def moe_expand_capacity(rows, topk, num_experts, align) -> int:
    return int(lib().moe_expand_capacity(rows, topk, num_experts, align))


def moe_expand_workspace_bytes(rows, topk, num_experts) -> int:
    return int(lib().moe_expand_workspace_bytes(rows, topk, num_experts))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, code):
    if code != MOE_OK:
        raise MoeError(fn, code)


def _fmt(fmt):
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


def moe_expand_layout(x, x_scale, fmt, topk_ids, topk_weights, psum_recv_per_rank,
                      num_experts, align, capacity, ex, ex_scale, psum, m_indices,
                      src2dst, row_weight, status, workspace, stream=None):
    """x [rows, >=hidden] fp8 (uint8 view ok), x_scale [rows, >=hidden/128];
    ex_scale [hidden/128, capacity] (K-block-major); see moe_expand.h for
    every argument."""
    rows, hidden = topk_ids.shape[0], ex.shape[1]
    code = lib().moe_expand_layout(
        _ptr(x), x.stride(0) * x.element_size(), _ptr(x_scale), x_scale.stride(0), _fmt(fmt),
        _ptr(topk_ids), _ptr(topk_weights), _ptr(psum_recv_per_rank),
        0 if psum_recv_per_rank is None else psum_recv_per_rank.numel(),
        rows, hidden, topk_ids.shape[1], num_experts, align, capacity,
        _ptr(ex), _ptr(ex_scale), _ptr(psum), _ptr(m_indices), _ptr(src2dst),
        _ptr(row_weight), _ptr(status), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("moe_expand_layout", code)


def moe_expand_layout_noalloc(x, x_scale, fmt, topk_ids, topk_weights, psum_recv_per_rank,
                              num_experts, align, capacity, ex, ex_scale, psum, m_indices,
                              src2dst, row_weight, status, stream=None):
    """moe_expand_layout with the library's static per-GPU scratch as the
    workspace: no workspace argument, nothing allocated (see moe_expand.h)."""
    rows, hidden = topk_ids.shape[0], ex.shape[1]
    code = lib().moe_expand_layout_noalloc(
        _ptr(x), x.stride(0) * x.element_size(), _ptr(x_scale), x_scale.stride(0), _fmt(fmt),
        _ptr(topk_ids), _ptr(topk_weights), _ptr(psum_recv_per_rank),
        0 if psum_recv_per_rank is None else psum_recv_per_rank.numel(),
        rows, hidden, topk_ids.shape[1], num_experts, align, capacity,
        _ptr(ex), _ptr(ex_scale), _ptr(psum), _ptr(m_indices), _ptr(src2dst),
        _ptr(row_weight), _ptr(status), _stream(stream))
    _check("moe_expand_layout_noalloc", code)


def moe_expand_layout_bf16(x, fmt, topk_ids, topk_weights, psum_recv_per_rank,
                           num_experts, align, capacity, ex, ex_scale, psum, m_indices,
                           src2dst, row_weight, status, workspace, stream=None):
    """x [rows, >=hidden] bf16 token rows, quantised per 1x128 group while
    they are scattered; otherwise as moe_expand_layout."""
    rows, hidden = topk_ids.shape[0], ex.shape[1]
    code = lib().moe_expand_layout_bf16(
        _ptr(x), x.stride(0), _fmt(fmt), _ptr(topk_ids), _ptr(topk_weights),
        _ptr(psum_recv_per_rank),
        0 if psum_recv_per_rank is None else psum_recv_per_rank.numel(),
        rows, hidden, topk_ids.shape[1], num_experts, align, capacity,
        _ptr(ex), _ptr(ex_scale), _ptr(psum), _ptr(m_indices), _ptr(src2dst),
        _ptr(row_weight), _ptr(status), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("moe_expand_layout_bf16", code)


def moe_grouped_gemm_fp8(a, a_scale, fmt, w, w_scale, psum, status, align, out,
                         stream=None):
    """a [capacity, k] fp8, a_scale [k/128, capacity], w [E, n, k] fp8,
    out [capacity, n] bf16."""
    capacity, k = a.shape
    E, n, _ = w.shape
    code = lib().moe_grouped_gemm_fp8(
        _ptr(a), _ptr(a_scale), _fmt(fmt), _ptr(w), _ptr(w_scale), _ptr(psum), _ptr(status),
        capacity, n, k, E, align, _ptr(out), _stream(stream))
    _check("moe_grouped_gemm_fp8", code)


def moe_act_quant(gate_up, m_indices, psum, status, num_experts, align, fmt, fold_weight,
                  out, out_scale, stream=None):
    """gate_up [capacity, 2I] bf16 -> out [capacity, I] fp8, out_scale [I/128, capacity]."""
    capacity, two_i = gate_up.shape
    code = lib().moe_act_quant(
        _ptr(gate_up), _ptr(m_indices), _ptr(psum), _ptr(status), capacity, two_i // 2,
        num_experts, align, _fmt(fmt), _ptr(fold_weight), _ptr(out), _ptr(out_scale),
        _stream(stream))
    _check("moe_act_quant", code)


def moe_gather(expert_out, src2dst, topk_weights, psum_recv_per_rank, out, stream=None,
               routed_scaling_factor=1.0):
    """expert_out [capacity, H] bf16, src2dst [rows, topk] -> out [rows, H] bf16."""
    rows, topk = src2dst.shape
    capacity, hidden = expert_out.shape
    code = lib().moe_gather(
        _ptr(expert_out), _ptr(src2dst), _ptr(topk_weights), float(routed_scaling_factor),
        _ptr(psum_recv_per_rank),
        0 if psum_recv_per_rank is None else psum_recv_per_rank.numel(),
        rows, hidden, topk, capacity, _ptr(out), _stream(stream))
    _check("moe_gather", code)


def moe_expand_to_masked_slab(ex, ex_scale, fmt, psum, status, num_experts, align, max_m,
                              slab, slab_scale, masked_m, stream=None):
    """ex [capacity, H] fp8, ex_scale [H/128, capacity] -> slab [E*max_m, H],
    slab_scale [H/128, E*max_m], masked_m [E]."""
    capacity, hidden = ex.shape
    code = lib().moe_expand_to_masked_slab(
        _ptr(ex), _ptr(ex_scale), _fmt(fmt), _ptr(psum), _ptr(status), capacity, hidden,
        num_experts, align, max_m, _ptr(slab), _ptr(slab_scale), _ptr(masked_m),
        _stream(stream))
    _check("moe_expand_to_masked_slab", code)


def moe_grouped_gemm_fp8_masked(a, a_scale, fmt, w, w_scale, masked_m, max_m, out,
                                stream=None):
    """a [E*max_m, k] fp8, a_scale [k/128, E*max_m], w [E, n, k] -> out [E*max_m, n]."""
    E, n, k = w.shape
    code = lib().moe_grouped_gemm_fp8_masked(
        _ptr(a), _ptr(a_scale), _fmt(fmt), _ptr(w), _ptr(w_scale), _ptr(masked_m), max_m,
        n, k, E, _ptr(out), _stream(stream))
    _check("moe_grouped_gemm_fp8_masked", code)


def moe_act_quant_masked(gate_up, masked_m, max_m, num_experts, fmt, out, out_scale,
                         stream=None):
    """gate_up [E*max_m, 2I] bf16 -> out [E*max_m, I] fp8, out_scale [I/128, E*max_m]."""
    code = lib().moe_act_quant_masked(
        _ptr(gate_up), _ptr(masked_m), max_m, gate_up.shape[1] // 2, num_experts, _fmt(fmt),
        _ptr(out), _ptr(out_scale), _stream(stream))
    _check("moe_act_quant_masked", code)


def moe_masked_slab_to_expand(slab_out, masked_m, max_m, psum, status, m_indices, row_weight,
                              num_experts, align, out, stream=None):
    """slab_out [E*max_m, H] bf16 -> out [capacity, H] bf16 (weighted rows)."""
    capacity, hidden = out.shape
    code = lib().moe_masked_slab_to_expand(
        _ptr(slab_out), _ptr(masked_m), max_m, _ptr(psum), _ptr(status), _ptr(m_indices),
        _ptr(row_weight), capacity, hidden, num_experts, align, _ptr(out), _stream(stream))
    _check("moe_masked_slab_to_expand", code)


def moe_grouped_gemm_bf16(a, w, psum, status, align, out, stream=None):
    """a [capacity, k] bf16, w [E, n, k] bf16 -> out [capacity, n] bf16."""
    capacity, k = a.shape
    E, n, _ = w.shape
    code = lib().moe_grouped_gemm_bf16(_ptr(a), _ptr(w), _ptr(psum), _ptr(status), capacity,
                                       n, k, E, align, _ptr(out), _stream(stream))
    _check("moe_grouped_gemm_bf16", code)


def moe_silu_mul_bf16(gate_up, m_indices, psum, status, num_experts, align, out, stream=None):
    """gate_up [capacity, 2I] bf16 -> out [capacity, I] bf16 (live rows)."""
    capacity, two_i = gate_up.shape
    code = lib().moe_silu_mul_bf16(_ptr(gate_up), _ptr(m_indices), _ptr(psum), _ptr(status),
                                   capacity, two_i // 2, num_experts, align, _ptr(out),
                                   _stream(stream))
    _check("moe_silu_mul_bf16", code)


class ExpandedMoE:
    """Buffers for one receive-buffer size, and the layer's five calls.

    Weights: w13 [E, 2I, H] fp8 + w13_scale [E, 2I/128, H/128];
    w2 [E, H, I] fp8 + w2_scale [E, H/128, I/128] (fp32 or UE8M0 bytes).
    Scale format 'f32' folds the top-k weight into the down GEMM's input
    scale; 'ue8m0' and 'mxfp8' (1x32 UE8M0 groups, weight scales [E, N,
    K/32]) weight the down output in the gather."""

    def __init__(self, rows, topk, w13, w13_scale, w2, w2_scale, align, fmt="f32",
                 device="cuda"):
        import torch
        self.fmt = fmt
        self.align = align
        self.w13, self.w13_scale, self.w2, self.w2_scale = w13, w13_scale, w2, w2_scale
        E, two_i, H = w13.shape
        self.E, self.I, self.H = E, two_i // 2, H
        self.rows, self.topk = rows, topk
        cap = moe_expand_capacity(rows, topk, E, align)
        self.capacity = cap
        # expanded scales: fp32 or UE8M0 bytes per (128-wide block, row); MXFP8
        # one 4-byte word (the block's four 1x32 bytes) per (block, row)
        sdt = {"f32": torch.float32, "ue8m0": torch.uint8, "mxfp8": torch.int32}[fmt]
        dev = device
        u8 = torch.uint8
        self.ex = torch.empty((cap, H), dtype=u8, device=dev)
        # expanded activation scales are K-block-major: [K/128, capacity]
        self.ex_scale = torch.empty((H // 128, cap), dtype=sdt, device=dev)
        self.psum = torch.empty(E, dtype=torch.int32, device=dev)
        self.m_indices = torch.empty(cap, dtype=torch.int32, device=dev)
        self.src2dst = torch.empty((rows, topk), dtype=torch.int32, device=dev)
        self.row_weight = torch.empty(cap, dtype=torch.float32, device=dev)
        self.status = torch.empty(2, dtype=torch.int32, device=dev)
        wsb = moe_expand_workspace_bytes(rows, topk, E)
        self.workspace = torch.empty(max(wsb, 256), dtype=u8, device=dev)
        self.gate_up = torch.empty((cap, 2 * self.I), dtype=torch.bfloat16, device=dev)
        self.dq = torch.empty((cap, self.I), dtype=u8, device=dev)
        self.ds = torch.empty((self.I // 128, cap), dtype=sdt, device=dev)
        self.down = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)

    def layout(self, x, x_scale, topk_ids, topk_weights, psum_recv_per_rank=None,
               stream=None):
        moe_expand_layout(x, x_scale, self.fmt, topk_ids, topk_weights, psum_recv_per_rank,
                          self.E, self.align, self.capacity, self.ex, self.ex_scale,
                          self.psum, self.m_indices, self.src2dst, self.row_weight,
                          self.status, self.workspace, stream)

    def experts(self, stream=None):
        moe_grouped_gemm_fp8(self.ex, self.ex_scale, self.fmt, self.w13, self.w13_scale,
                             self.psum, self.status, self.align, self.gate_up, stream)
        fold = self.row_weight if self.fmt == "f32" else None
        moe_act_quant(self.gate_up, self.m_indices, self.psum, self.status, self.E,
                      self.align, self.fmt, fold, self.dq, self.ds, stream)
        moe_grouped_gemm_fp8(self.dq, self.ds, self.fmt, self.w2, self.w2_scale,
                             self.psum, self.status, self.align, self.down, stream)

    def gather(self, topk_weights, psum_recv_per_rank, out, stream=None):
        wts = None if self.fmt == "f32" else topk_weights
        moe_gather(self.down, self.src2dst, wts, psum_recv_per_rank, out, stream)

    def __call__(self, x, x_scale, topk_ids, topk_weights, psum_recv_per_rank=None,
                 out=None, stream=None):
        import torch
        if out is None:
            out = torch.empty((self.rows, self.H), dtype=torch.bfloat16, device=x.device)
        self.layout(x, x_scale, topk_ids, topk_weights, psum_recv_per_rank, stream)
        self.experts(stream)
        self.gather(topk_weights, psum_recv_per_rank, out, stream)
        return out


class StandardMoE(ExpandedMoE):
    """The standard (non-EP) path: bf16 token rows (every expert local) are
    quantised per 1x128 group while they are scattered into the 128-aligned
    expert blocks; the same GEMMs and activation run with no weight fold;
    the gather applies the top-k weights and the routed scaling factor."""

    def __init__(self, rows, topk, w13, w13_scale, w2, w2_scale, align=128, fmt="f32",
                 routed_scaling_factor=1.0, device="cuda"):
        super().__init__(rows, topk, w13, w13_scale, w2, w2_scale, align, fmt, device)
        self.routed_scaling_factor = float(routed_scaling_factor)

    def layout(self, x, topk_ids, topk_weights, psum_recv_per_rank=None, stream=None):
        moe_expand_layout_bf16(x, self.fmt, topk_ids, topk_weights, psum_recv_per_rank,
                               self.E, self.align, self.capacity, self.ex, self.ex_scale,
                               self.psum, self.m_indices, self.src2dst, None, self.status,
                               self.workspace, stream)

    def experts(self, stream=None):
        moe_grouped_gemm_fp8(self.ex, self.ex_scale, self.fmt, self.w13, self.w13_scale,
                             self.psum, self.status, self.align, self.gate_up, stream)
        moe_act_quant(self.gate_up, self.m_indices, self.psum, self.status, self.E,
                      self.align, self.fmt, None, self.dq, self.ds, stream)
        moe_grouped_gemm_fp8(self.dq, self.ds, self.fmt, self.w2, self.w2_scale,
                             self.psum, self.status, self.align, self.down, stream)

    def gather(self, topk_weights, psum_recv_per_rank, out, stream=None):
        moe_gather(self.down, self.src2dst, topk_weights, psum_recv_per_rank, out, stream,
                   routed_scaling_factor=self.routed_scaling_factor)

    def __call__(self, x, topk_ids, topk_weights, psum_recv_per_rank=None, out=None,
                 stream=None):
        import torch
        if out is None:
            out = torch.empty((self.rows, self.H), dtype=torch.bfloat16, device=x.device)
        self.layout(x, topk_ids, topk_weights, psum_recv_per_rank, stream)
        self.experts(stream)
        self.gather(topk_weights, psum_recv_per_rank, out, stream)
        return out


class MaskedMoE(ExpandedMoE):
    """The decode path: the expanded layout, then the bridge into a
    fixed-height slab [E, max_m, H] with masked_m live rows per expert, the
    masked GEMMs and activation on the slab, the bridge back with the top-k
    weights, and the combine with weight 1."""

    def __init__(self, rows, topk, w13, w13_scale, w2, w2_scale, align, max_m, fmt="f32",
                 device="cuda"):
        import torch
        super().__init__(rows, topk, w13, w13_scale, w2, w2_scale, align, fmt, device)
        self.max_m = max_m
        E, H, I = self.E, self.H, self.I
        sdt = torch.float32 if fmt == "f32" else torch.uint8
        n = E * max_m
        self.slab = torch.empty((n, H), dtype=torch.uint8, device=device)
        self.slab_scale = torch.empty((H // 128, n), dtype=sdt, device=device)
        self.masked_m = torch.empty(E, dtype=torch.int32, device=device)
        self.s_gate_up = torch.empty((n, 2 * I), dtype=torch.bfloat16, device=device)
        self.s_dq = torch.empty((n, I), dtype=torch.uint8, device=device)
        self.s_ds = torch.empty((I // 128, n), dtype=sdt, device=device)
        self.s_down = torch.empty((n, H), dtype=torch.bfloat16, device=device)

    def experts(self, stream=None):
        moe_expand_to_masked_slab(self.ex, self.ex_scale, self.fmt, self.psum, self.status,
                                  self.E, self.align, self.max_m, self.slab, self.slab_scale,
                                  self.masked_m, stream)
        moe_grouped_gemm_fp8_masked(self.slab, self.slab_scale, self.fmt, self.w13,
                                    self.w13_scale, self.masked_m, self.max_m, self.s_gate_up,
                                    stream)
        moe_act_quant_masked(self.s_gate_up, self.masked_m, self.max_m, self.E, self.fmt,
                             self.s_dq, self.s_ds, stream)
        moe_grouped_gemm_fp8_masked(self.s_dq, self.s_ds, self.fmt, self.w2, self.w2_scale,
                                    self.masked_m, self.max_m, self.s_down, stream)
        moe_masked_slab_to_expand(self.s_down, self.masked_m, self.max_m, self.psum,
                                  self.status, self.m_indices, self.row_weight, self.E,
                                  self.align, self.down, stream)

    def gather(self, topk_weights, psum_recv_per_rank, out, stream=None):
        moe_gather(self.down, self.src2dst, None, psum_recv_per_rank, out, stream)


class StandardBf16MoE:
    """The standard path with bf16 weights: bf16 token rows scattered as they
    are into the 128-aligned expert blocks, bf16 gate_up GEMM, SiLU*up to
    bf16, bf16 down GEMM, gather with the top-k weights and the routed
    scaling factor.  w13 [E, 2I, H], w2 [E, H, I] bf16."""

    def __init__(self, rows, topk, w13, w2, align=128, routed_scaling_factor=1.0,
                 device="cuda"):
        import torch
        self.w13, self.w2, self.align = w13, w2, align
        self.routed_scaling_factor = float(routed_scaling_factor)
        E, two_i, H = w13.shape
        self.E, self.I, self.H = E, two_i // 2, H
        self.rows, self.topk = rows, topk
        cap = moe_expand_capacity(rows, topk, E, align)
        self.capacity = cap
        bf, i32 = torch.bfloat16, torch.int32
        self.ex = torch.empty((cap, H), dtype=bf, device=device)
        self.psum = torch.empty(E, dtype=i32, device=device)
        self.m_indices = torch.empty(cap, dtype=i32, device=device)
        self.src2dst = torch.empty((rows, topk), dtype=i32, device=device)
        self.status = torch.empty(2, dtype=i32, device=device)
        wsb = moe_expand_workspace_bytes(rows, topk, E)
        self.workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=device)
        self.gate_up = torch.empty((cap, 2 * self.I), dtype=bf, device=device)
        self.y = torch.empty((cap, self.I), dtype=bf, device=device)
        self.down = torch.empty((cap, H), dtype=bf, device=device)

    def layout(self, x, topk_ids, topk_weights, psum_recv_per_rank=None, stream=None):
        moe_expand_layout_bf16(x, "none", topk_ids, topk_weights, psum_recv_per_rank, self.E,
                               self.align, self.capacity, self.ex, None, self.psum,
                               self.m_indices, self.src2dst, None, self.status,
                               self.workspace, stream)

    def experts(self, stream=None):
        moe_grouped_gemm_bf16(self.ex, self.w13, self.psum, self.status, self.align,
                              self.gate_up, stream)
        moe_silu_mul_bf16(self.gate_up, self.m_indices, self.psum, self.status, self.E,
                          self.align, self.y, stream)
        moe_grouped_gemm_bf16(self.y, self.w2, self.psum, self.status, self.align, self.down,
                              stream)

    def gather(self, topk_weights, psum_recv_per_rank, out, stream=None):
        moe_gather(self.down, self.src2dst, topk_weights, psum_recv_per_rank, out, stream,
                   routed_scaling_factor=self.routed_scaling_factor)

    def __call__(self, x, topk_ids, topk_weights, psum_recv_per_rank=None, out=None,
                 stream=None):
        import torch
        if out is None:
            out = torch.empty((self.rows, self.H), dtype=torch.bfloat16, device=x.device)
        self.layout(x, topk_ids, topk_weights, psum_recv_per_rank, stream)
        self.experts(stream)
        self.gather(topk_weights, psum_recv_per_rank, out, stream)
        return out
