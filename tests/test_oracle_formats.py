"""Pins of the oracle's format decoders against things other than themselves:
torch's fp8 types (a library implementation), the OCP tables in tests/golden,
exact rational arithmetic and the recipe's 448*6 constant."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden


def _minifloat(bits, ebits, mbits, bias, top="fn"):
    """Generic sign/exponent/mantissa decoder returning a Fraction (or 'nan'/'inf').

    top='fn': only all-ones exponent AND mantissa is NaN (E4M3FN);
    top='ieee': all-ones exponent is inf/NaN (E5M2); top='none': no specials (E2M1).
    """
    sign = (bits >> (ebits + mbits)) & 1
    e = (bits >> mbits) & ((1 << ebits) - 1)
    m = bits & ((1 << mbits) - 1)
    emax = (1 << ebits) - 1
    if top == "ieee" and e == emax:
        return "inf" if m == 0 else "nan"
    if top == "fn" and e == emax and m == (1 << mbits) - 1:
        return "nan"
    if e == 0:
        v = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        v = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)
    return -v if sign else v


def _torch_fp8(dtype):
    return torch.arange(256, dtype=torch.uint8).view(dtype).to(torch.float64).numpy()


@pytest.mark.parametrize("dtype,ebits,mbits,bias,top", [
    (torch.float8_e4m3fn, 4, 3, 7, "fn"),
    (torch.float8_e5m2, 5, 2, 15, "ieee"),
])
def test_generic_minifloat_matches_torch(dtype, ebits, mbits, bias, top):
    ref = _torch_fp8(dtype)
    for b in range(256):
        v = _minifloat(b, ebits, mbits, bias, top)
        if v == "nan":
            assert np.isnan(ref[b])
        elif v == "inf":
            assert np.isinf(ref[b])
        else:
            assert ref[b] == float(v), hex(b)


def test_e4m3_matches_torch_all_256():
    ref = _torch_fp8(torch.float8_e4m3fn)
    got = oracle.e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))  # -0.0 at 0x80


def test_e4m3_golden_anchors():
    for byte, val in read_golden("e4m3_anchors.txt"):
        got = oracle.e4m3_value(int(byte, 16))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), byte


def test_e2m1_golden_table():
    rows = read_golden("e2m1_table.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = oracle.e2m1_value(int(code, 16))
        assert got == float(val), code
        assert np.signbit(got) == val.startswith("-"), code


def test_e2m1_generic_minifloat():
    # E2M1: 2 exponent bits with bias 1, 1 mantissa bit, no specials
    for c in range(16):
        v = _minifloat(c, 2, 1, 1, "none")
        assert oracle.e2m1_value(c) == float(v)


def test_recipe_constant_448_times_6():
    # the global-scale recipe divides amax by 448*6: the largest E4M3 times the largest E2M1
    e4 = oracle.e4m3_value(np.arange(256))
    e2 = oracle.e2m1_value(np.arange(16))
    assert np.nanmax(e4) == 448.0 and np.max(e2) == 6.0
    assert np.nanmax(e4) * np.max(e2) == 2688.0


def test_e2m1_times_e4m3_exact_in_f16():
    """Every finite (code, scale) product is exactly representable in f16, so a
    kernel may dequantize to f16 without rounding and apply g in fp32."""
    e2 = oracle.e2m1_value(np.arange(16))
    e4 = oracle.e4m3_value(np.arange(256))
    prod = np.outer(e2, e4[~np.isnan(e4)])
    assert np.array_equal(prod.astype(np.float16).astype(np.float64), prod)
    nz = np.abs(prod[prod != 0])
    assert nz.min() >= 2.0 ** -10 and nz.max() == 2688.0  # normal f16 range


def test_nibble_order():
    q = np.array([[1, 2, 3, 4, 15, 0]], np.uint8)
    packed = np.array([[0x21, 0x43, 0x0F]], np.uint8)
    assert np.array_equal(oracle.unpack_nibbles(packed), q)


def test_nvfp4_dequant_exact_rational():
    rng = np.random.default_rng(7)
    N, K = 3, 32
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)   # finite, non-negative
    g = np.float32(3.1e-5)
    got = oracle.nvfp4_dequant(codes, scales, g)
    e2 = {int(c, 16): Fraction(v) for c, v in read_golden("e2m1_table.txt")}
    e4 = _torch_fp8(torch.float8_e4m3fn)
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            code = (byte >> 4) if (k % 2) else (byte & 15)
            exact = e2[code] * Fraction(float(e4[scales[n, k // 16]])) * Fraction(float(g))
            assert Fraction(float(got[n, k])) == exact, (n, k)
            f32 = oracle.nvfp4_dequant_f32(codes, scales, g)[n, k]
            assert f32 == np.float32(float(exact))


def test_bf16_value_matches_torch():
    bits = np.random.default_rng(3).integers(0, 1 << 16, 4096, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]             # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_value(bits), ref)


def test_affine_dequant_exact_rational():
    rng = np.random.default_rng(11)
    N, K = 2, 128
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    s_bits = torch.tensor(np.abs(rng.normal(0, .003, (N, 2))), dtype=torch.float32).to(torch.bfloat16)
    b_bits = torch.tensor(rng.normal(0, .01, (N, 2)), dtype=torch.float32).to(torch.bfloat16)
    s = s_bits.view(torch.int16).numpy().view(np.uint16)
    b = b_bits.view(torch.int16).numpy().view(np.uint16)
    got = oracle.affine_dequant(codes, s, b)
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            q = (byte >> 4) if (k % 2) else (byte & 15)
            exact = q * Fraction(float(s_bits[n, k // 64])) + Fraction(float(b_bits[n, k // 64]))
            assert Fraction(float(got[n, k])) == exact
    # the fp32 value is that exact value rounded once, i.e. a fused multiply-add
    f32 = oracle.affine_dequant_f32(codes, s, b)
    q = oracle.unpack_nibbles(codes).astype(np.float32)
    sf = np.repeat(s_bits.float().numpy(), 64, axis=1)
    bf = np.repeat(b_bits.float().numpy(), 64, axis=1)
    fma = (q.astype(np.float64) * sf + bf).astype(np.float32)  # float64 product is exact here
    assert np.array_equal(f32, fma)
