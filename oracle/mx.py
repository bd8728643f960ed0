"""MXFP4 decoding (test infrastructure; see the package docstring).

The txtmix.com article, §1 and §3, says the expert weights ship as MXFP4: 4-bit
elements sharing one E8M0 scale.  The element code is OCP MX v1.0's E2M1 and a
scale block holds 32 consecutive elements along the reduction dimension.

E2M1 (OCP MX v1.0, FP4 element): bit 3 sign, bits 2..1 exponent (bias 1), bit 0
mantissa.  Exponent 0 is subnormal: value = mantissa * 2^(1-1) * 0.5.  There is
no infinity and no NaN.  E8M0 (OCP MX v1.0 scale): an unsigned biased exponent,
value 2^(s-127); s = 255 is NaN; there is no zero and no sign.
"""
from __future__ import annotations

import numpy as np

__all__ = ["e2m1_decode", "e8m0_decode", "dequant_mxfp4", "E2M1_VALUES"]


def e2m1_decode(codes) -> np.ndarray:
    """Decode E2M1 codes (0..15) to float64 from the sign/exponent/mantissa fields."""
    c = np.asarray(codes, dtype=np.int64)
    sign = (c >> 3) & 1
    exp = (c >> 1) & 3
    man = c & 1
    normal = (1.0 + 0.5 * man) * np.exp2(exp - 1.0)      # 1.m * 2^(exp - bias), bias 1
    subnormal = 0.5 * man                                 # 0.m * 2^(1 - bias)
    mag = np.where(exp == 0, subnormal, normal)
    return np.where(sign == 1, -mag, mag)


E2M1_VALUES = e2m1_decode(np.arange(16))


def e8m0_decode(scales) -> np.ndarray:
    """Decode E8M0 scale bytes to float64: 2^(s-127), NaN for s = 255."""
    s = np.asarray(scales, dtype=np.int64)
    return np.where(s == 255, np.nan, np.exp2(s - 127.0))


def dequant_mxfp4(codes_packed, scales) -> np.ndarray:
    """Dequantise packed MXFP4 rows.

    codes_packed: uint8 [..., K/2]; element 2i is the low nibble of byte i and
    element 2i+1 the high nibble.  scales: uint8 [..., K/32], scale b covers
    elements 32b .. 32b+31.  Returns float32 [..., K].  The product is formed in
    float64 (it is exact: an E2M1 value has at most two significant bits) and
    then stored as float32.
    """
    c = np.asarray(codes_packed, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8)
    K = c.shape[-1] * 2
    if s.shape[-1] * 32 != K:
        raise ValueError("scales must hold one byte per 32 elements")
    elems = np.empty(c.shape[:-1] + (K,), dtype=np.uint8)
    elems[..., 0::2] = c & 0x0F
    elems[..., 1::2] = c >> 4
    vals = e2m1_decode(elems)
    scale = np.repeat(e8m0_decode(s), 32, axis=-1)
    with np.errstate(invalid="ignore", over="ignore"):
        return (vals * scale).astype(np.float32)
