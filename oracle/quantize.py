"""Oracle for the NVFP4 quantizer (float32 steps, as the GPU quantizer takes them).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: [README] gemma-cuda-hybrid README, the kernel list of its source
tree (an NVFP4 quantization kernel beside the FP4 GEMM) and "Why it's
NVIDIA-only" (NVFP4: E2M1 codes, E4M3 scale per 16 values, fp32 global
scale).  The recipe, as the workload states it: global scale g = tensor
amax / (448 * 6); group scale = E4M3(group amax / 6 / g), round to nearest
even, saturating at 448; codes = E2M1(w / (e4m3(s) * g)), round to nearest
even, saturating at 6; a group whose decoded scale is 0 gets +0 codes.

Reading taken: every step is one float32 operation in that order (amax,
amax / 2688, gamax / 6, / g, e4m3 * g, w / S), because the quantized codes
are integers decided by floating point and the GPU takes the decisions in
float32.  The encoders here are written from the format definitions (not
shared with the input generator); tests/test_oracle_quantize.py pins them by
exhaustive nearest-value search and against the input generator's float64
recipe.
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_value, e2m1_value

F32 = np.float32


def e4m3_encode_rne(t: np.ndarray) -> np.ndarray:
    """Non-negative finite float32 -> E4M3FN byte (0..0x7E), nearest value,
    ties to the even code; above 448 saturates to 0x7E (448)."""
    t = np.asarray(t, np.float64)       # float32 values are exact in float64
    if np.any(t < 0) or not np.all(np.isfinite(t)):
        raise ValueError("E4M3 encode wants finite non-negative values")
    vals = e4m3_value(np.arange(0x7F, dtype=np.uint8))      # 0 .. 448, increasing
    i = np.searchsorted(vals, t, side="left")                # vals[i-1] < t <= vals[i]
    i = np.clip(i, 1, 0x7E)
    lo, hi = vals[i - 1], vals[i]
    pick_hi = (t - lo > hi - t) | ((t - lo == hi - t) & (i % 2 == 0))   # tie: the even code
    code = np.where(pick_hi, i, i - 1)
    code = np.where(t >= 448.0, 0x7E, code)
    code = np.where(t == 0, 0, code)
    return code.astype(np.uint8)


def e2m1_encode_rne(x: np.ndarray) -> np.ndarray:
    """Float32 -> E2M1 code (bit 3 = sign, bits 0-2 = magnitude index):
    nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even index, beyond 6
    saturates to 6; the sign is the sign bit of x (so -0 gives code 8)."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    grid = e2m1_value(np.arange(8, dtype=np.uint8))          # 0 .. 6
    d = np.abs(a[..., None] - grid)                          # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # at a midpoint the two candidates are adjacent indices: take the even one
    even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    idx = np.where(a >= 6.0, 7, idx)
    sign = np.signbit(x).astype(np.uint8)
    return (idx.astype(np.uint8) | (sign << 3)).astype(np.uint8)


def nvfp4_global_scale_f32(w: np.ndarray) -> np.float32:
    """g = amax|w| / (448 * 6), one float32 division (0 for an all-zero w)."""
    w = np.asarray(w, F32)
    amax = np.max(np.abs(w)) if w.size else F32(0)
    return F32(F32(amax) / F32(2688.0))


def nvfp4_quantize_f32(w: np.ndarray, global_scale: float | None = None):
    """fp32 [N][K] (K % 16 == 0) -> (codes u8[N][K/2] low nibble = even k,
    scales u8[N][K/16], g float32), every step in float32."""
    w = np.ascontiguousarray(w, F32)
    N, K = w.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    if global_scale is None or global_scale <= 0:
        g = nvfp4_global_scale_f32(w)
    else:
        g = F32(global_scale)
    blk = w.reshape(N, K // 16, 16)
    gamax = np.max(np.abs(blk), axis=2).astype(F32)
    if g > 0:
        t = ((gamax / F32(6.0)).astype(F32) / g).astype(F32)
    else:
        t = np.zeros_like(gamax)
    s = e4m3_encode_rne(t)
    S = (e4m3_value(s).astype(F32) * g).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        x = np.where(S[..., None] > 0, (blk / S[..., None]).astype(F32), F32(0))
    q = e2m1_encode_rne(x)
    q = np.where(S[..., None] > 0, q, 0).astype(np.uint8)
    q = q.reshape(N, K)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return codes, s.astype(np.uint8), g
