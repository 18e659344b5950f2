"""Pins of the oracle GEMM: exact rational arithmetic on tiny shapes with weights
decoded by an independent route (torch fp8 + the OCP E2M1 table), special
cases with closed-form results, and the affine group-sum identity."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import read_golden

E2 = {int(c, 16): Fraction(v) for c, v in read_golden("e2m1_table.txt")}
E4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _exact_nvfp4_w(codes, scales, g):
    N, Kh = codes.shape
    W = [[None] * (2 * Kh) for _ in range(N)]
    for n in range(N):
        for k in range(2 * Kh):
            byte = int(codes[n, k // 2])
            c = (byte >> 4) if k & 1 else (byte & 15)
            W[n][k] = E2[c] * Fraction(float(E4[scales[n, k // 16]])) * Fraction(float(np.float32(g)))
    return W


def _exact_gemm(a, W):
    M, K = len(a), len(a[0])
    return [[sum((a[m][k] * W[n][k] for k in range(K)), Fraction(0)) for n in range(len(W))]
            for m in range(M)]


def _frac_rows(a):
    return [[Fraction(float(v)) for v in row] for row in np.asarray(a, np.float64)]


@pytest.mark.parametrize("M,K,N,seed", [(1, 32, 5, 1), (2, 64, 8, 2), (3, 48, 3, 3)])
def test_nvfp4_gemm_vs_exact_rationals(M, K, N, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)
    g = np.float32(rng.uniform(1e-5, 1e-3))
    a = rng.standard_normal((M, K)).astype(np.float16)
    y, bnd = oracle.nvfp4_gemm_ref(codes, scales, g, a)
    ex = _exact_gemm(_frac_rows(a), _exact_nvfp4_w(codes, scales, g))
    for m in range(M):
        for n in range(N):
            # float64 summation: |error| <= K * 2^-52 * sum|a w|
            assert abs(Fraction(y[m, n]) - ex[m][n]) <= Fraction(K) * Fraction(2) ** -52 * Fraction(bnd[m, n])
            absum = sum(abs(v) for v in (x * w for x, w in zip(_frac_rows(a)[m],
                                                                 _exact_nvfp4_w(codes, scales, g)[n])))
            assert abs(Fraction(bnd[m, n]) - absum) <= Fraction(K) * Fraction(2) ** -52 * absum


def test_nvfp4_gemm_identity_weights():
    # W[n, k] = 1.0 iff k == n: code 0x2 (1.0), scale 0x38 (1.0), g = 1 -> y = a[:, :N] exactly
    N, K = 16, 64
    q = np.zeros((N, K), np.uint8)
    q[np.arange(N), np.arange(N)] = 0x2
    codes = synth.pack_nibbles(q)
    scales = np.full((N, K // 16), 0x38, np.uint8)
    a = np.random.default_rng(0).standard_normal((3, K)).astype(np.float16)
    y, _ = oracle.nvfp4_gemm_ref(codes, scales, np.float32(1.0), a)
    assert np.array_equal(y, a[:, :N].astype(np.float64))


def test_nvfp4_gemm_single_nonzero_and_zero():
    N, K = 4, 32
    q = np.zeros((N, K), np.uint8)
    q[2, 17] = 0xF                                    # -6.0
    scales = np.zeros((N, K // 16), np.uint8)
    scales[2, 1] = 0x39                               # 1.125
    g = np.float32(0.5)
    a = np.random.default_rng(1).standard_normal((2, K)).astype(np.float16)
    y, _ = oracle.nvfp4_gemm_ref(synth.pack_nibbles(q), scales, g, a)
    expect = np.zeros((2, N))
    expect[:, 2] = a[:, 17].astype(np.float64) * (-6.0 * 1.125 * 0.5)
    assert np.array_equal(y, expect)


def test_nvfp4_gemm_linearity_and_orientation():
    rng = np.random.default_rng(5)
    inp = synth.nvfp4_gemm(9, 2, 64, 24)
    a1 = rng.standard_normal((2, 64)).astype(np.float16)
    y1, _ = oracle.nvfp4_gemm_ref(inp.codes, inp.scales, inp.g, a1)
    y2, _ = oracle.nvfp4_gemm_ref(inp.codes, inp.scales, inp.g, (2 * a1.astype(np.float32)).astype(np.float16))
    assert np.array_equal(2 * y1, y2)
    # output column n depends only on weight row n
    c2 = inp.codes.copy()
    c2[7] ^= 0x11
    y3, _ = oracle.nvfp4_gemm_ref(c2, inp.scales, inp.g, a1)
    changed = np.nonzero(np.any(y3 != y1, axis=0))[0]
    assert list(changed) == [7]


def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_affine_gemm_vs_exact_rationals():
    rng = np.random.default_rng(21)
    M, K, N = 2, 128, 3
    codes, s, b = synth.affine_weights(77, N, K)
    a = _bf16(rng.standard_normal((M, K)))
    y, bnd = oracle.affine_gemm_ref(codes, s, b, a)
    av = oracle.bf16_value(a)
    q = oracle.unpack_nibbles(codes)
    sv, bv = oracle.bf16_value(s), oracle.bf16_value(b)
    for m in range(M):
        for n in range(N):
            ex = sum((Fraction(float(av[m, k])) * (int(q[n, k]) * Fraction(float(sv[n, k // 64]))
                                                  + Fraction(float(bv[n, k // 64])))
                      for k in range(K)), Fraction(0))
            assert abs(Fraction(y[m, n]) - ex) <= Fraction(K) * Fraction(2) ** -52 * Fraction(bnd[m, n])


def test_affine_groupsum_identity():
    inp = synth.affine_gemm(13, 4, 5 * 64, 40)
    y, bnd = oracle.affine_gemm_ref(inp.codes, inp.scale, inp.bias, inp.a)
    y2 = oracle.affine_gemm_groupsum(inp.codes, inp.scale, inp.bias, inp.a)
    assert np.all(np.abs(y - y2) <= 1e-12 * bnd)


def test_affine_zero_codes_gives_bias_times_group_sums():
    M, K, N = 3, 256, 5
    rng = np.random.default_rng(4)
    codes = np.zeros((N, K // 2), np.uint8)
    s = _bf16(np.abs(rng.normal(0, .003, (N, K // 64))))
    b = _bf16(rng.normal(0, .01, (N, K // 64)))
    a = _bf16(rng.standard_normal((M, K)))
    y, _ = oracle.affine_gemm_ref(codes, s, b, a)
    av = oracle.bf16_value(a).reshape(M, K // 64, 64)
    asum = np.array([[sum(Fraction(float(v)) for v in av[m, gi]) for gi in range(K // 64)] for m in range(M)])
    bv = oracle.bf16_value(b)
    for m in range(M):
        for n in range(N):
            ex = sum((asum[m, gi] * Fraction(float(bv[n, gi])) for gi in range(K // 64)), Fraction(0))
            assert abs(Fraction(y[m, n]) - ex) <= Fraction(2) ** -40 * (1 + abs(ex))


def test_argmax_ties_and_fp32_decision():
    y = np.array([[1.0, 3.0, 3.0, 2.0],
                  [5.0, 5.0 + 1e-12, 4.0, 0.0],     # equal in fp32 -> lower index
                  [-1.0, -2.0, -0.5, -0.5]])
    assert list(oracle.argmax_ref(y)) == [1, 0, 2]


def test_abs_bound_dominates():
    inp = synth.nvfp4_gemm(3, 4, 128, 32)
    y, bnd = oracle.nvfp4_gemm_ref(inp.codes, inp.scales, inp.g, inp.a)
    assert np.all(np.abs(y) <= bnd * (1 + 1e-12))
