"""Pins of the affine b-bit oracle (oracle.affine_dequant_bits / affine_bits_gemm_ref)."""
import numpy as np
import pytest

import oracle
import synth


def test_four_bits_equals_the_pinned_nibble_form():
    # at 4 bits the one-code-per-byte form must equal the (separately pinned)
    # packed-nibble dequant
    q, s, b = synth.affine_weights_bits(3, 32, 256, 4)
    packed = synth.pack_nibbles(q)
    assert np.array_equal(oracle.affine_dequant_bits(q, s, b, 4), oracle.affine_dequant(packed, s, b))


@pytest.mark.parametrize("bits", [2, 3, 5, 6, 8])
def test_group_structure_and_extremes(bits):
    q, s, b = synth.affine_weights_bits(4, 16, 128, bits)
    w = oracle.affine_dequant_bits(q, s, b, bits)
    sv, bv = oracle.bf16_value(s), oracle.bf16_value(b)
    # code 0 gives the bias, the top code gives bias + (2^b - 1) * scale, per group of 64
    z = np.zeros_like(q)
    assert np.array_equal(oracle.affine_dequant_bits(z, s, b, bits), np.repeat(bv, 64, axis=1))
    top = np.full_like(q, (1 << bits) - 1)
    assert np.array_equal(oracle.affine_dequant_bits(top, s, b, bits),
                          np.repeat(bv + ((1 << bits) - 1) * sv, 64, axis=1))
    # affine in q: w(q1) - w(q0) = (q1 - q0) * s
    d = oracle.affine_dequant_bits(q, s, b, bits) - oracle.affine_dequant_bits(z, s, b, bits)
    assert np.array_equal(d, q.astype(np.float64) * np.repeat(sv, 64, axis=1))
    with pytest.raises(ValueError):
        oracle.affine_dequant_bits(np.full_like(q, 1 << bits) if bits < 8 else q.astype(np.int32) + 256, s, b, bits)


@pytest.mark.parametrize("bits", [2, 6])
def test_gemm_exact_rational_small(bits):
    # a tiny product checked with exact rationals
    from fractions import Fraction
    q, s, b = synth.affine_weights_bits(5, 2, 64, bits)
    a = synth.act_bf16_bits(6, 3, 64)
    y, bnd = oracle.affine_bits_gemm_ref(q, s, b, a, bits)
    sv, bv, av = oracle.bf16_value(s), oracle.bf16_value(b), oracle.bf16_value(a)
    for m in range(3):
        for n in range(2):
            exact = sum(Fraction(float(av[m, k])) * (int(q[n, k]) * Fraction(float(sv[n, 0])) + Fraction(float(bv[n, 0])))
                        for k in range(64))
            assert abs(float(exact) - y[m, n]) <= 1e-12 * float(bnd[m, n])
