"""Per-group fp8 quantisation (oracle; test infrastructure only).

The rule is the pages' per-token-group fp8 quantisation (SGLang
moe_runner/deep_gemm.py source, ``_situ_mul_quant_contig_kernel``, and the
``sglang_per_token_group_quant_fp8`` call in ``_run_contiguous_gemm``):

* fp32 scale format: per group, ``amax = max(|v|)`` clamped below at 1e-10,
  codes ``q = E4M3(v * (448 / amax))`` and scale ``s = amax / 448``, all in
  fp32 arithmetic, so that ``q * s`` reconstructs ``v``.
* UE8M0 scale format: the fp32 scale ``amax / 448`` is rounded UP to a power
  of two (``fp8.e8m0_round_up``) and the codes are ``E4M3(v / 2^(b-127))``;
  dividing by a power of two is exact, so the only rounding is the fp8 one.
  (Reading: the pages store the rounded-up byte as the GEMM scale; dividing
  by that same power of two keeps ``q * s`` a reconstruction of ``v``.)

Activations use 1x128 groups along the row; weights use 128x128 blocks.

MXFP8 format ('mxfp8'; SGLang moe_runner/deep_gemm.py source,
``DeepGemmMoeQuantInfo.__post_init__``: MXFP8 requires a [1, 32] block shape
and UE8M0 scales; ``_run_masked_gemm``: recipe (1, 32) for the weights):
both operands use 1x32 groups along K with UE8M0 scales - activations
[M, K/32], weights per row [E, N, K/32] - quantised with the UE8M0 rule.
"""

import numpy as np

from . import fp8

GROUP = 128
EPS = np.float32(1e-10)
F8_MAX = np.float32(448.0)


MX_GROUP = 32


def _codes_and_scales(v32: np.ndarray, amax: np.ndarray, fmt: str):
    """v32: values in fp32 with the group's amax broadcast against them."""
    amax = np.maximum(amax, EPS).astype(np.float32)
    if fmt == "mxfp8":
        fmt = "ue8m0"
    if fmt == "f32":
        s = (amax / F8_MAX).astype(np.float32)
        inv = (F8_MAX / amax).astype(np.float32)
        q = fp8.encode_e4m3((v32 * inv).astype(np.float32))
        return q, s
    if fmt == "ue8m0":
        b = fp8.e8m0_round_up((amax / F8_MAX).astype(np.float32))
        # Scaling by a power of two is exact in float32 down to 2^-126; any
        # value that small is far below the smallest fp8 step and encodes to 0.
        q = fp8.encode_e4m3(np.ldexp(v32, (127 - b.astype(np.int32))).astype(np.float32))
        return q, b
    raise ValueError(f"unknown scale format {fmt!r}")


def quantize_rows(v, fmt: str = "f32", group: int = GROUP):
    """[M, K] values -> (codes [M, K] uint8, scales [M, K/group]).

    Scales are float32 (fmt 'f32') or UE8M0 bytes (fmt 'ue8m0'; 'mxfp8':
    UE8M0 bytes of 1x32 groups)."""
    if fmt == "mxfp8":
        group = MX_GROUP
    v32 = np.asarray(v, dtype=np.float32)
    m, k = v32.shape
    assert k % group == 0
    g = v32.reshape(m, k // group, group)
    amax = np.max(np.abs(g), axis=2, keepdims=True)
    q, s = _codes_and_scales(g, amax, fmt)
    return q.reshape(m, k), s.reshape(m, k // group)


def quantize_blocks(w, fmt: str = "f32", block: int = GROUP):
    """[E, N, K] weights -> (codes [E, N, K] uint8, scales [E, N/blk, K/blk]).

    One scale per block x block tile of each expert's [N, K] matrix; for
    'mxfp8' one per 1x32 group of each row: scales [E, N, K/32]."""
    if fmt == "mxfp8":
        w32 = np.asarray(w, dtype=np.float32)
        e, n, k = w32.shape
        q, s = quantize_rows(w32.reshape(e * n, k), "mxfp8")
        return q.reshape(e, n, k), s.reshape(e, n, k // MX_GROUP)
    w32 = np.asarray(w, dtype=np.float32)
    e, n, k = w32.shape
    assert n % block == 0 and k % block == 0
    t = w32.reshape(e, n // block, block, k // block, block)
    amax = np.max(np.abs(t), axis=(2, 4), keepdims=True)
    q, s = _codes_and_scales(t, amax, fmt)
    return q.reshape(e, n, k), s.reshape(e, n // block, k // block)


def scale_values(s, fmt: str) -> np.ndarray:
    """Stored scales -> float64 multipliers."""
    if fmt == "f32":
        return np.asarray(s, dtype=np.float32).astype(np.float64)
    if fmt in ("ue8m0", "mxfp8"):
        return fp8.e8m0_value(s)
    raise ValueError(f"unknown scale format {fmt!r}")


def dequant_rows(q, s, fmt: str, group: int = GROUP) -> np.ndarray:
    """codes [M, K] and scales [M, K/group] -> float64 values q * s."""
    if fmt == "mxfp8":
        group = MX_GROUP
    vals = fp8.decode_e4m3(q)
    m, k = vals.shape
    sv = scale_values(s, fmt).reshape(m, k // group, 1)
    return (vals.reshape(m, k // group, group) * sv).reshape(m, k)


def dequant_block(q, s, fmt: str, block: int = GROUP) -> np.ndarray:
    """One expert's codes [N, K] and scales [N/blk, K/blk] (mxfp8: [N, K/32])
    -> float64."""
    if fmt == "mxfp8":
        return dequant_rows(q, s, "mxfp8")
    vals = fp8.decode_e4m3(q)
    n, k = vals.shape
    sv = scale_values(s, fmt).reshape(n // block, 1, k // block, 1)
    return (vals.reshape(n // block, block, k // block, block) * sv).reshape(n, k)
