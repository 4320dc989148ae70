"""Low-bit weight formats, decoded the plain way in float64.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

MXFP4 is named as the native expert weight format on the page "Sovereign
gpt-oss-20B (MXFP4) on Apple Silicon" (section 1 Contribution, and section 3
Results: the MXFP4 reader is bit-exact, max_abs 0.0).  The page prints no bit
layout, so the encoding follows the OCP Microscaling Formats (MX) v1.0
specification:

* an element is FP4 E2M1 - 1 sign bit, 2 exponent bits with bias 1, 1 mantissa
  bit, exponent field 0 meaning a subnormal with value m * 2^-1;
* a block of 32 elements shares one E8M0 scale, an unsigned 8-bit biased
  exponent with value 2^(e-127); e = 255 encodes NaN.

Packed int4 with on-chip dequantisation is the weight format of the pages
"Single-stream int4 decode of a 30B MoE on Apple Silicon" (section 6) and the
TinyTitan tracker (entries D108, D110).  They print no formula either; the
reading taken is the usual asymmetric group quantisation: an unsigned code
q in [0, 15], one unsigned int4 zero point z and one fp16 scale s per group of
``group`` contiguous K-elements of a row, w = (q - z) * s.

Layout readings (the pages fix none of them):

* row-major, K contiguous: codes [n][k/2] bytes;
* two elements per byte, the LOW nibble holds the even K index;
* MXFP4 scales [n][k/32] bytes, one per 32 contiguous K-elements of a row;
* int4 scales [n][k/group] fp16, zeros [n][ceil(k/group/2)] bytes packed two
  per byte along the group axis, low nibble = even group.
"""

import numpy as np


def unpack_nibbles(packed, count=None):
    """Split each byte into (low, high) nibbles along the last axis.

    ``packed[..., j]`` yields elements 2j (low nibble) and 2j+1 (high nibble).
    ``count`` trims the result to the first ``count`` elements.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    if count is not None:
        out = out[..., :count]
    return out


def e2m1_value(code):
    """Value of FP4 E2M1 code(s) 0..15 in float64 (OCP MX v1.0, FP4 E2M1).

    sign = bit 3, exponent field = bits 2..1 (bias 1), mantissa = bit 0.
    Exponent field 0 is subnormal: m * 0.5.  Otherwise 2^(e-1) * (1 + m/2).
    Code 8 is negative zero.
    """
    code = np.asarray(code, dtype=np.int64)
    sign = (code >> 3) & 1
    exp_field = (code >> 1) & 3
    mant = code & 1
    normal = np.ldexp(1.0 + mant / 2.0, exp_field - 1)
    subnormal = mant * 0.5
    mag = np.where(exp_field == 0, subnormal, normal).astype(np.float64)
    return np.where(sign == 1, -mag, mag)


def e8m0_value(e):
    """Value of E8M0 scale byte(s) in float64: 2^(e-127), and NaN for 255."""
    e = np.asarray(e, dtype=np.int64)
    val = np.ldexp(np.ones(e.shape, dtype=np.float64), e - 127)
    return np.where(e == 255, np.nan, val)


def mxfp4_dequant64(codes, scales):
    """Dequantize an MXFP4 matrix to float64 (exact products, no rounding).

    codes  : uint8 [n][k/2]   (low nibble = even k)
    scales : uint8 [n][k/32]  (E8M0, one per 32 contiguous K-elements)
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    n, half_k = codes.shape
    k = 2 * half_k
    if k % 32 or scales.shape != (n, k // 32):
        raise ValueError("MXFP4 shapes: codes [n][k/2], scales [n][k/32]")
    values = e2m1_value(unpack_nibbles(codes))
    block_scale = np.repeat(e8m0_value(scales), 32, axis=1)
    return values * block_scale


def mxfp4_dequant(codes, scales):
    """Dequantized MXFP4 weights as fp32: the fp64 product rounded once.

    Every product of an E2M1 value (at most 2 significant bits) and a power of
    two is exactly representable in fp32 unless it overflows (-> +-inf, e >=
    253 with a large code) - subnormal results (e in {0, 1}) are kept.  So the
    rounding to fp32 is exact and the result is the bit pattern a correct IEEE
    fp32 multiply must give.
    """
    with np.errstate(over="ignore", invalid="ignore"):
        return mxfp4_dequant64(codes, scales).astype(np.float32)


def int4_group_count(k, group):
    if group <= 0 or k % group:
        raise ValueError("k must be a multiple of the group size")
    return k // group


def int4g_dequant64(codes, scales_f16, zeros, group):
    """Dequantize a group-quantized int4 matrix to float64: w = (q - z) * s.

    codes      : uint8 [n][k/2]                 (low nibble = even k)
    scales_f16 : float16 (or its uint16 bits) [n][k/group]
    zeros      : uint8 [n][ceil((k/group)/2)]   (low nibble = even group)
    """
    codes = np.asarray(codes, dtype=np.uint8)
    n, half_k = codes.shape
    k = 2 * half_k
    groups = int4_group_count(k, group)
    scales = np.asarray(scales_f16)
    if scales.dtype == np.uint16:
        scales = scales.view(np.float16)
    if scales.shape != (n, groups):
        raise ValueError("int4 scales must be [n][k/group]")
    zeros = np.asarray(zeros, dtype=np.uint8)
    if zeros.shape != (n, (groups + 1) // 2):
        raise ValueError("int4 zeros must be [n][ceil(k/group/2)]")
    q = unpack_nibbles(codes).astype(np.float64)
    z = unpack_nibbles(zeros, groups).astype(np.float64)
    s = scales.astype(np.float64)
    return (q - np.repeat(z, group, axis=1)) * np.repeat(s, group, axis=1)


def int4g_dequant(codes, scales_f16, zeros, group):
    """Dequantized int4 weights as fp32.

    |q - z| <= 15 needs 4 significant bits and an fp16 scale 11, so the fp64
    product has at most 15 significant bits and lies inside the fp32 range:
    the rounding to fp32 is exact.  An infinite scale gives +-inf, or NaN when
    q == z; a NaN scale gives NaN.
    """
    with np.errstate(invalid="ignore"):
        return int4g_dequant64(codes, scales_f16, zeros, group).astype(np.float32)
