"""Number formats used on the path (oracle; test infrastructure only).

* OCP 8-bit float E4M3 in its "fn" flavour: 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits, subnormals, no infinities, and the all-ones
  exponent+mantissa pattern (0x7F / 0xFF) as NaN.  Largest finite value 448.
  The pages quantise activations and weights to this format with 1x128 and
  128x128 fp32 scales (SGLang moe_runner/deep_gemm.py source,
  ``_run_contiguous_gemm`` and ``_situ_mul_quant_contig_kernel``).
* bfloat16 round-to-nearest-even from a wider float.
* UE8M0 scale bytes: an unsigned biased exponent, value 2**(b - 127).  The
  pages turn an fp32 scale into such a byte by rounding its magnitude UP to a
  power of two (SGLang moe_runner/deep_gemm.py source,
  ``_cast_to_e8m0_with_rounding_up``).
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def _decode_table() -> np.ndarray:
    """All 256 E4M3(fn) codes as float64, written from the format definition."""
    tab = np.empty(256, dtype=np.float64)
    for b in range(256):
        sign = -1.0 if (b >> 7) else 1.0
        e = (b >> 3) & 0xF
        m = b & 0x7
        if e == 0xF and m == 0x7:
            tab[b] = np.nan
        elif e == 0:
            tab[b] = sign * (m / 8.0) * 2.0 ** -6
        else:
            tab[b] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


E4M3_TABLE = _decode_table()


def decode_e4m3(codes) -> np.ndarray:
    """uint8 codes -> float64 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


_POS = E4M3_TABLE[:0x7F]                     # codes 0x00..0x7E, increasing
_MIDS = (_POS[:-1] + _POS[1:]) / 2.0          # exact in float64


def encode_e4m3(values) -> np.ndarray:
    """Float values -> uint8 E4M3(fn) codes: the nearest representable
    magnitude, ties to the even code (even mantissa), sign kept.

    Magnitudes above 464 (the midpoint between 448 and the NaN slot) become
    NaN (0x7F with the sign bit), as do NaN and +-inf: the format has no
    infinity and this encoder does not saturate.  -0.0 keeps its sign bit.

    float32 input is rounded on its bit pattern (round to nearest even at
    the third mantissa bit; subnormals as multiples of 2^-9); any other input
    is converted to float64 and matched against the table of midpoints."""
    v = np.asarray(values)
    if v.dtype == np.float32:
        a = np.abs(v)
        code = _encode_f32_magnitude(a)
    else:
        v = v.astype(np.float64)
        a = np.abs(v)
        code = np.searchsorted(_MIDS, a, side="left")     # midpoints below a
        tie = (code < len(_MIDS)) & (_MIDS[np.minimum(code, len(_MIDS) - 1)] == a)
        code = np.where(tie & (code % 2 == 1), code + 1, code)
    bad = ~(a <= 464.0)                                   # > 464, inf or NaN
    code = np.where(bad, E4M3_NAN, code).astype(np.uint8)
    return code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)


def _encode_f32_magnitude(a):
    """|v| as float32 -> E4M3 code (before the overflow check)."""
    bits = np.ascontiguousarray(a).view(np.uint32)
    # Normal range (>= 2^-6): round to nearest-even at the third mantissa bit;
    # the top 12 bits are then (float32 exponent, 3 mantissa bits), a carry
    # moving into the exponent.  Rebias the exponent from 127 to 7.
    top = (bits + np.uint32(0x7FFFF) + ((bits >> np.uint32(20)) & np.uint32(1))) \
        >> np.uint32(20)
    normal = top.astype(np.int32) - ((127 - 7) << 3)
    # Subnormal range: multiples of 2^-9, nearest-even (rint); 8 is 2^-6.
    sub = np.rint(a * np.float32(512.0)).astype(np.int32)
    code = np.where(a >= np.float32(2.0 ** -6), normal, sub)
    return np.minimum(code, 0x7F)


def round_bf16(values) -> np.ndarray:
    """Round float64/float32 values to bfloat16 (nearest, ties to even) with a
    single rounding from the float64 value; return them as float32.

    Only used on finite values inside the normal bf16 range."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
    bits = v.view(np.uint64)
    # bf16 keeps the top 7 of the 52 float64 mantissa bits: drop the low 45.
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    bits = bits + np.uint64((1 << 44) - 1) + lsb
    bits = bits & ~np.uint64((1 << 45) - 1)
    return bits.view(np.float64).astype(np.float32)


def bf16_bits(values_f32) -> np.ndarray:
    """float32 values that are exact bf16 numbers -> their uint16 bf16 bits."""
    v = np.ascontiguousarray(np.asarray(values_f32, dtype=np.float32))
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def e8m0_round_up(scale_f32) -> np.ndarray:
    """fp32 scale -> UE8M0 byte of the smallest power of two not below it.

    Follows the pages' bit rule on the fp32 pattern: take the biased exponent
    field; add one unless the mantissa is zero (already a power of two), the
    exponent field is 0xFE (adding one would give the NaN byte), or the value
    is a subnormal whose mantissa is at most half-scale (then 2^-127, byte 0,
    already bounds it from above).  Only non-negative inputs occur on the
    path (scales are max-abs / 448)."""
    s = np.ascontiguousarray(np.asarray(scale_f32, dtype=np.float32))
    bits = s.view(np.int32).astype(np.int64)
    exp = bits >> 23
    mant = bits & 0x7FFFFF
    bump = (mant > 0) & (exp != 0xFE) & ~((exp == 0) & (mant <= 0x400000))
    return (exp + bump.astype(np.int64)).astype(np.uint8)


def e8m0_value(byte) -> np.ndarray:
    """UE8M0 byte -> float64 2**(b-127)."""
    return np.ldexp(1.0, np.asarray(byte, dtype=np.int64) - 127)
