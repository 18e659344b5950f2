"""Pins of the NVFP4 quantizer oracle (oracle/quantize.py) to things other than itself."""
import numpy as np
import pytest

import oracle
import synth
from oracle import quantize as Q


def test_e4m3_encode_exact_values_and_midpoints():
    vals = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    # every representable value encodes to its own byte
    assert np.array_equal(Q.e4m3_encode_rne(vals.astype(np.float32)), np.arange(0x7F, dtype=np.uint8))
    # midpoints go to the even byte; points just off a midpoint go to the nearer value
    mid = (vals[:-1] + vals[1:]) / 2
    codes = Q.e4m3_encode_rne(mid.astype(np.float32))
    even = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    exact = mid.astype(np.float32).astype(np.float64) == mid          # midpoints that float32 holds
    assert np.array_equal(codes[exact], even[exact])
    for b in range(1, 0x7E):
        lo, hi = vals[b], vals[b + 1]
        t = np.float32(lo + 0.3 * (hi - lo)), np.float32(lo + 0.7 * (hi - lo))
        assert Q.e4m3_encode_rne(np.array(t)).tolist() == [b, b + 1]
    # saturation at 448, zero, smallest subnormal
    assert Q.e4m3_encode_rne(np.array([448.0, 460.0, 1e30, 0.0, 2.0 ** -9, 2.0 ** -11], np.float32)).tolist() == \
        [0x7E, 0x7E, 0x7E, 0, 1, 0]


def test_e2m1_encode_is_the_nearest_grid_value():
    grid = oracle.e2m1_value(np.arange(8, dtype=np.uint8))
    x = np.random.default_rng(0).uniform(-8, 8, 20000).astype(np.float32)
    code = Q.e2m1_encode_rne(x)
    got = oracle.e2m1_value(code)
    best = np.min(np.abs(np.abs(x)[:, None].astype(np.float64) - grid), axis=1)
    inrange = np.abs(x) <= 6
    assert np.allclose(np.abs(np.abs(x[inrange]) - np.abs(got[inrange])), best[inrange], atol=0)
    assert np.all(np.abs(got[~inrange]) == 6)
    assert np.array_equal(np.signbit(got), np.signbit(x))
    # the midpoints, each way (ties to the even index)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert Q.e2m1_encode_rne(mids).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert Q.e2m1_encode_rne(-mids).tolist() == [8, 10, 10, 12, 12, 14, 14]
    assert Q.e2m1_encode_rne(np.array([0.0, -0.0], np.float32)).tolist() == [0, 8]


@pytest.mark.parametrize("N,K", [(32, 256), (48, 704), (16, 80)])
def test_quantize_matches_the_float64_recipe_of_the_input_generator(N, K):
    # same recipe, float64 steps in the generator vs float32 steps here: the
    # codes and scales agree except where a value sits on a rounding boundary
    w = synth.normal_f32(11, 7, N, K, 0.02)
    c64, s64, g64 = synth.quantize_nvfp4(w)
    c32, s32, g32 = Q.nvfp4_quantize_f32(w)
    assert g32 == g64
    assert np.mean(s32 == s64) > 0.999
    same = np.mean(c32 == c64)
    assert same > 0.999, same


def test_quantize_roundtrip_is_nearest_on_the_scaled_grid():
    w = synth.normal_f32(12, 7, 64, 512, 0.02)
    codes, scales, g = Q.nvfp4_quantize_f32(w)
    deq = oracle.nvfp4_dequant(codes, scales, g)
    S = (oracle.e4m3_value(scales) * np.float64(g)).repeat(16, axis=1)
    grid = oracle.e2m1_value(np.arange(8, dtype=np.uint8))
    # every element is within half a grid step of its dequantized value (grid steps 0.5, 1, 2 times S)
    x = np.abs(w / S)
    step = np.where(x < 2, 0.5, np.where(x < 4, 1.0, 2.0))
    assert np.all(np.abs(w - deq) <= 0.5 * step * S * (1 + 1e-6) + 1e-30)
    # and the group scales follow amax / 6: the largest element of each group maps near 6
    blk = np.abs(w).reshape(64, -1, 16).max(axis=2)
    t = blk / 6 / np.float64(g)
    sv = oracle.e4m3_value(scales)
    assert np.all(np.abs(sv - t) <= 0.0625 * t + 1e-12)       # E4M3 keeps 3 mantissa bits


def test_quantize_zero_matrix_and_given_scale():
    c, s, g = Q.nvfp4_quantize_f32(np.zeros((16, 64), np.float32))
    assert g == 0 and not c.any() and not s.any()
    w = synth.normal_f32(13, 7, 16, 64, 0.02)
    c1, s1, g1 = Q.nvfp4_quantize_f32(w, global_scale=1e-4)
    assert g1 == np.float32(1e-4)
    # with the scale given, large groups saturate at 448 instead of following amax
    assert np.all(s1 <= 0x7E)
