"""Dequantize-then-matmul in float64.  (Test infrastructure only.)

The skinny GEMM of decode and speculative verify [README, "Everything it
has": the M <= 16 tensor-core GEMM over NVFP4 weights; ISSUE, "Why now":
qlinear's affine paths] computes y[m, n] = sum_k a[m, k] * w[n, k] with the
weight matrix stored row-per-output ([N][K], groups along K).

The pass criterion is per element: |y_gpu - y| <= 1e-3 * sum_k |a[m,k] w[n,k]|,
which ``gemm_abs_bound`` supplies (the sum of absolute products).
"""
from __future__ import annotations

import numpy as np

from .formats import nvfp4_dequant, affine_dequant, affine_dequant_bits, unpack_nibbles, bf16_value


def gemm_ref(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = a @ w^T in float64 (a [M][K], w [N][K])."""
    return np.asarray(a, np.float64) @ np.asarray(w, np.float64).T


def gemm_abs_bound(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """sum_k |a[m,k] * w[n,k]| for every output element, float64."""
    return np.abs(np.asarray(a, np.float64)) @ np.abs(np.asarray(w, np.float64)).T


def nvfp4_gemm_ref(codes, scales, g, a, want_bound: bool = True):
    """NVFP4 W4A16 GEMM: (y float64 [M][N], bound [M][N] or None).

    Rows of W are processed in chunks so that large N stays within memory.
    """
    a64 = np.asarray(a, np.float64)
    N = codes.shape[0]
    y = np.empty((a64.shape[0], N))
    bnd = np.empty_like(y) if want_bound else None
    step = 16384
    for r0 in range(0, N, step):
        r1 = min(N, r0 + step)
        w = nvfp4_dequant(codes[r0:r1], scales[r0:r1], g)
        y[:, r0:r1] = a64 @ w.T
        if want_bound:
            bnd[:, r0:r1] = np.abs(a64) @ np.abs(w).T
    return y, bnd


def affine_gemm_ref(codes, scale_bits, bias_bits, a_bits, want_bound: bool = True):
    """Affine 4-bit GEMM with bf16 activations (a given as bf16 bit patterns)."""
    a64 = bf16_value(a_bits)
    N = codes.shape[0]
    y = np.empty((a64.shape[0], N))
    bnd = np.empty_like(y) if want_bound else None
    step = 8192
    for r0 in range(0, N, step):
        r1 = min(N, r0 + step)
        w = affine_dequant(codes[r0:r1], scale_bits[r0:r1], bias_bits[r0:r1])
        y[:, r0:r1] = a64 @ w.T
        if want_bound:
            bnd[:, r0:r1] = np.abs(a64) @ np.abs(w).T
    return y, bnd


def affine_gemm_groupsum(codes, scale_bits, bias_bits, a_bits) -> np.ndarray:
    """The same product in the group-sum form of the issue's "activation rows with
    64-value group sums": y = sum_g s[n,g] * sum_{k in g} a[m,k] q[n,k]
                              + b[n,g] * sum_{k in g} a[m,k].
    Algebraically identical to ``affine_gemm_ref``; the tests check they agree.
    """
    a64 = bf16_value(a_bits)
    M, K = a64.shape
    q = unpack_nibbles(codes).astype(np.float64)      # [N][K]
    N = q.shape[0]
    G = K // 64
    s = bf16_value(scale_bits)                        # [N][G]
    b = bf16_value(bias_bits)
    ag = a64.reshape(M, G, 64)
    qg = q.reshape(N, G, 64)
    dot = np.einsum("mgk,ngk->mng", ag, qg)           # per-group sum of a*q
    asum = ag.sum(axis=2)                             # [M][G] group sums of a
    return np.einsum("mng,ng->mn", dot, s) + asum @ b.T


def argmax_ref(y) -> np.ndarray:
    """Per-row argmax taken on the fp32 logits (the kernel's decision precision):
    the exact value is rounded once to fp32, ties go to the lowest index
    (tree_round's argmax in the issue's "Why now" names only the operation)."""
    y32 = np.asarray(y, np.float64).astype(np.float32)
    return np.argmax(y32, axis=1).astype(np.int32)   # numpy returns the first maximum


def affine_bits_gemm_ref(codes, scale_bits, bias_bits, a_bits, bits: int, want_bound: bool = True):
    """Affine b-bit GEMM (codes one per byte [N][K]) with bf16 activations:
    (y float64 [M][N], sum_k |a w| or None)."""
    a64 = bf16_value(a_bits)
    N = codes.shape[0]
    y = np.empty((a64.shape[0], N))
    bnd = np.empty_like(y) if want_bound else None
    step = 4096
    for r0 in range(0, N, step):
        r1 = min(N, r0 + step)
        w = affine_dequant_bits(codes[r0:r1], scale_bits[r0:r1], bias_bits[r0:r1], bits)
        y[:, r0:r1] = a64 @ w.T
        if want_bound:
            bnd[:, r0:r1] = np.abs(a64) @ np.abs(w).T
    return y, bnd
