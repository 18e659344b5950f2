"""The seeded generators: determinism, the encoding recipe checked by brute force
against the oracle's decoders, and bf16 rounding against torch."""
import numpy as np
import torch

import oracle
import synth


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [0.0, -0.0, 1.00390625, 1.01171875]   # exact ties to even in bf16
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(x), ref)
    assert np.array_equal(synth.bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).float().numpy())


def test_e4m3_encoder_brute_force():
    vals = oracle.e4m3_value(np.arange(0x7F))          # the finite non-negative bytes
    t = np.concatenate([np.random.default_rng(1).uniform(0, 500, 20000),
                        np.random.default_rng(2).uniform(0, 2 ** -5, 20000),
                        (vals[1:] + vals[:-1]) / 2,    # exact midpoints
                        vals, [0.0, 448.0, 460.0, 470.0, 1e6]])
    got = synth.encode_e4m3_rne_satfinite(t)
    for ti, gi in zip(t, got):
        d = np.abs(vals - min(ti, 448.0))
        best = np.flatnonzero(d == d.min())
        # nearest, ties to the even mantissa (even byte)
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert gi == want, (ti, gi, want)


def test_e2m1_encoder_ties_and_saturation():
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 100.0, -0.1, -5.0, 0.2500001])
    want = [0x0, 0x2, 0x2, 0x4, 0x4, 0x6, 0x6, 0x7, 0x7, 0x8, 0xE, 0x1]
    assert list(synth.encode_e2m1_rne_satfinite(x)) == want
    # brute force nearest (ties to even code) on random values
    vals = oracle.e2m1_value(np.arange(8))
    r = np.random.default_rng(3).uniform(-7, 7, 20000)
    got = synth.encode_e2m1_rne_satfinite(r)
    for ri, gi in zip(r, got):
        d = np.abs(vals - min(abs(ri), 6.0))
        best = np.flatnonzero(d == d.min())
        mag = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert gi == (mag | (8 if ri < 0 else 0))


def test_quantizer_recipe_round_trip():
    w = synth.normal_f32(42, 1, 64, 256, 0.02)
    w[3, 16:32] = 0.0                                  # a zero group
    codes, scales, g = synth.quantize_nvfp4(w)
    assert g == np.float32(np.float32(np.max(np.abs(w))) / np.float32(2688.0))
    sv = oracle.e4m3_value(scales)
    amax = np.abs(w.astype(np.float64)).reshape(64, 16, 16).max(axis=2)
    # scale byte is the E4M3 nearest to amax/6/g
    assert np.array_equal(scales, synth.encode_e4m3_rne_satfinite(amax / 6.0 / np.float64(g)))
    assert np.all(sv[3, 1] == 0) and np.all(oracle.unpack_nibbles(codes)[3, 16:32] == 0)
    # every code is the nearest E2M1 value to w / S (checked through the oracle's decoder)
    q = oracle.unpack_nibbles(codes)
    S = np.repeat(sv, 16, axis=1) * np.float64(g)
    vals = oracle.e2m1_value(np.arange(16))
    nz = S > 0
    x = np.where(nz, w / np.where(nz, S, 1), 0)
    err = np.abs(vals[q] - np.clip(x, -6, 6))
    best = np.min(np.abs(vals[None, None, :] - np.clip(x, -6, 6)[..., None]), axis=2)
    assert np.array_equal(err, best)
    # group maxima land near the top of the E2M1 range (the point of amax/6)
    assert np.max(np.abs(vals[q])) == 6.0


def test_generators_deterministic_and_blocked():
    a = synth.nvfp4_gemm(7, 2, 128, 48)
    b = synth.nvfp4_gemm(7, 2, 128, 48)
    assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales)
    assert a.g == b.g and np.array_equal(a.a, b.a)
    c = synth.nvfp4_gemm(8, 2, 128, 48)
    assert not np.array_equal(a.codes, c.codes)
    # a matrix taller than one block: the first block equals a draw of that block alone
    big = synth.normal_f32(5, 1, synth.BLOCK_ROWS + 3, 16, 1.0)
    small = synth.normal_f32(5, 1, synth.BLOCK_ROWS, 16, 1.0)
    assert np.array_equal(big[:synth.BLOCK_ROWS], small)


def test_affine_generator_ranges():
    inp = synth.affine_gemm(105, 2, 256, 32)
    q = oracle.unpack_nibbles(inp.codes)
    assert q.min() >= 0 and q.max() <= 15
    s = oracle.bf16_value(inp.scale)
    assert np.all(s >= 0) and 0.001 < s.mean() < 0.005
    assert inp.a.dtype == np.uint16 and inp.a.shape == (2, 256)
