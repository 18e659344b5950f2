"""Weight formats, decoded by their closed forms in float64.  (Test infrastructure only.)

NVFP4 [README, "Everything it has"; "Why it's NVIDIA-only"]: a weight is an
E2M1 code times the E4M3 scale of its group of 16 along K times one fp32
global scale.  The pages name the formats but print no table; the readings
taken are the OCP ones (E2M1 with max 6, E4M3FN with max 448), which are the
only ones consistent with a group scale of amax/6 under a global scale of
amax/(448*6).

Affine 4-bit [ISSUE, "Why now"]: w = q * scale + bias with q in [0, 15] and
one bf16 scale and bias per 64 weights along K.  The value is taken exactly
(the float64 bound of the issue's "Gates"), not with a bf16 rounding after
each operation.
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code) -> np.ndarray:
    """E2M1 code (bit 3 sign, bits 2-1 exponent with bias 1, bit 0 mantissa) -> float64.

    exponent 0: 0.5 * m (zero or the subnormal 0.5); else 2^(e-1) * (1 + m/2).
    Pinned against a generic minifloat decoder validated on torch's fp8 types,
    the OCP table in tests/golden, and the max-6 consistency of the recipe.
    """
    c = np.asarray(code).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.exp2(e - 1.0) * (1.0 + m / 2.0))
    return np.where(s == 1, -mag, mag)


def e4m3_value(byte) -> np.ndarray:
    """OCP E4M3FN byte -> float64 (bias 7, no infinities, 0x7F/0xFF are NaN).

    exponent 0: (-1)^s * 2^-6 * m/8; else (-1)^s * 2^(e-7) * (1 + m/8).
    Pinned against torch.float8_e4m3fn for all 256 bytes.
    """
    b = np.asarray(byte).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, np.exp2(-6.0) * (m / 8.0), np.exp2(e - 7.0) * (1.0 + m / 8.0))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes; element 2j is the low nibble of byte j."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def nvfp4_dequant(codes: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    """NVFP4 [N][K/2] codes, [N][K/16] scales, fp32 g -> exact float64 weights [N][K].

    e2m1 * e4m3 has at most 6 significant bits and g at most 24, so the float64
    product is exact: this is the weight's true value.
    """
    q = unpack_nibbles(codes)
    N, K = q.shape
    s = e4m3_value(scales)
    if s.shape != (N, K // 16):
        raise ValueError("scales must be [N][K/16]")
    return e2m1_value(q) * np.repeat(s, 16, axis=1) * np.float64(np.float32(g))


def nvfp4_dequant_f32(codes, scales, g) -> np.ndarray:
    """The fp32 value of each weight: the exact value rounded once to nearest-even."""
    return nvfp4_dequant(codes, scales, g).astype(np.float32)


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of an fp32)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def affine_dequant(codes: np.ndarray, scale_bits: np.ndarray, bias_bits: np.ndarray) -> np.ndarray:
    """Affine 4-bit [N][K/2] codes with bf16 scale/bias [N][K/64] -> float64 q*s + b.

    q (4 bits) times a bf16 (8 significant bits) plus a bf16 is exact in
    float64 whenever the exponents of s and b are within ~40 binades of each
    other, which the callers assert (all finite synthetic inputs satisfy it).
    """
    q = unpack_nibbles(codes).astype(np.float64)
    N, K = q.shape
    s = bf16_value(scale_bits)
    b = bf16_value(bias_bits)
    if s.shape != (N, K // 64) or b.shape != (N, K // 64):
        raise ValueError("scale/bias must be [N][K/64]")
    return q * np.repeat(s, 64, axis=1) + np.repeat(b, 64, axis=1)


def affine_dequant_f32(codes, scale_bits, bias_bits) -> np.ndarray:
    """fp32 value of each affine weight: exact q*s + b rounded once (== fmaf(q, s, b))."""
    return affine_dequant(codes, scale_bits, bias_bits).astype(np.float32)


AFFINE_BITS = (2, 3, 4, 5, 6, 8)


def affine_dequant_bits(codes: np.ndarray, scale_bits: np.ndarray, bias_bits: np.ndarray, bits: int) -> np.ndarray:
    """Affine b-bit codes, one per byte [N][K] (values < 2^b), with bf16
    scale/bias [N][K/64] -> float64 q * s + b, per 64-value group.

    [ISSUE "Why now": qlinear's MLX affine paths at 4 bits and at 2, 3, 5, 6
    and 8 bits, in groups of 64; "Steps" 3 and 9: the other MLX widths].  Exact in float64 for the same reason as the
    4-bit form (q < 2^8 times an 8-significant-bit bf16, plus a bf16)."""
    if bits not in AFFINE_BITS:
        raise ValueError(f"bits must be one of {AFFINE_BITS}")
    q = np.asarray(codes)
    if np.any(q >= (1 << bits)):
        raise ValueError("code out of range for the bit width")
    q = q.astype(np.float64)
    N, K = q.shape
    s = bf16_value(scale_bits)
    b = bf16_value(bias_bits)
    if s.shape != (N, K // 64) or b.shape != (N, K // 64):
        raise ValueError("scale/bias must be [N][K/64]")
    return q * np.repeat(s, 64, axis=1) + np.repeat(b, 64, axis=1)
