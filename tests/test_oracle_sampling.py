"""Pins of the sampling oracle (oracle/sampling.py) to things other than itself."""
import math

import numpy as np
import pytest

import oracle
from oracle import sampling as S


def _carry_inc(c):  # 4 x 64-bit counter + 1
    c = list(c)
    for i in range(4):
        c[i] = (c[i] + 1) % 2**64
        if c[i] != 0:
            break
    return c


@pytest.mark.parametrize("ctr,key", [(0, 0), (5, 12345), (2**64 - 1, 2**64 - 1), (7 + (3 << 64), 99 + (1 << 70))])
def test_philox_round_structure_matches_numpy_4x64(ctr, key):
    # NumPy's Philox bit generator is Philox4x64-10: the same rounds and key
    # schedule with 64-bit words.  It steps its 256-bit counter before each
    # block, so its first block comes from counter + 1.
    bg = np.random.Philox(counter=ctr, key=key)
    words = [(ctr >> (64 * i)) & (2**64 - 1) for i in range(4)]
    c = _carry_inc(words)
    k = (key & (2**64 - 1), key >> 64)
    for _ in range(3):
        raw = bg.random_raw(4)
        out = S.philox4(tuple(np.uint64(x) for x in c), (np.uint64(k[0]), np.uint64(k[1])), bits=64)
        assert [int(o) for o in out] == [int(r) for r in raw]
        c = _carry_inc(c)


def test_philox4x32_known_answers():
    # the published known-answer vectors of Philox4x32-10 (Random123 distribution)
    kat = [((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
           ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
           ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
            (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1))]
    for ctr, key, want in kat:
        got = S.philox4(ctr, key, bits=32)
        assert tuple(int(x) for x in got) == want


def test_uniform_map_range_and_exactness():
    x = np.array([0, 1, 511, 512, 2**31, 2**32 - 1], np.uint32)
    u = S.uniform_bits_to_f32(x)
    assert u.dtype == np.float32
    assert u[0] == u[1] == u[2] == np.float32(2.0 ** -24)      # low 9 bits dropped
    assert u[3] == np.float32(3 * 2.0 ** -24)
    assert u[4] == np.float32(0.5 + 2.0 ** -24)
    assert u[5] == np.float32(1.0 - 2.0 ** -24) and u[5] < 1.0
    xs = np.arange(0, 2**32, 2**9 * 997, dtype=np.uint64).astype(np.uint32)
    us = S.uniform_bits_to_f32(xs)
    exact = ((xs >> np.uint32(9)).astype(np.float64) * 2 + 1) * 2.0 ** -24
    assert np.array_equal(us.astype(np.float64), exact)       # no rounding anywhere
    assert np.all((us > 0) & (us < 1))


def test_sample_uniforms_layout():
    seed, off, M, N = 0x0123456789ABCDEF, 77, 6, 10
    u = S.sample_uniforms(seed, off, M, N)
    assert u.shape == (M, N)
    for m in range(M):
        for n in range(N):
            w = S.philox4((n, m // 4, off, 0), (seed & 0xFFFFFFFF, seed >> 32), bits=32)[m % 4]
            assert u[m, n] == S.uniform_bits_to_f32(np.array([int(w)], np.uint32))[0]
    assert not np.array_equal(u, S.sample_uniforms(seed, off + 1, M, N))
    assert not np.array_equal(u, S.sample_uniforms(seed + 1, off, M, N))


def test_gumbel_moments():
    # Gumbel(0, 1): mean = Euler-Mascheroni constant, variance = pi^2 / 6
    g = S.gumbel(S.sample_uniforms(5, 0, 1000, 1000)).ravel()
    assert abs(g.mean() - 0.5772156649015329) < 5 * math.sqrt(math.pi**2 / 6 / g.size)
    assert abs(g.var() - math.pi**2 / 6) < 0.02


@pytest.mark.parametrize("T", [0.7, 2.0])
def test_gumbel_max_frequencies_follow_softmax(T):
    # the Gumbel-max trick: P(token = i) = softmax(z / T)_i; rows are independent trials
    z = np.array([1.0, 0.5, -0.3, 2.0, 0.0, 2.0])
    R = 60000
    tok = S.sample_tokens(np.tile(z, (R, 1)), T, seed=1234, offset=9)
    freq = np.bincount(tok, minlength=z.size) / R
    p = np.exp(z / T - np.max(z / T))
    p /= p.sum()
    sd = np.sqrt(p * (1 - p) / R)
    assert np.all(np.abs(freq - p) < 5 * sd + 1e-12), (freq, p)


def test_temperature_zero_is_greedy():
    z = np.random.default_rng(3).normal(size=(7, 300))
    z[2, 40] = z[2, 17] = z[2].max() + 1.0      # tie: the lower index
    assert np.array_equal(S.sample_tokens(z, 0.0, 1, 2), oracle.argmax_ref(z))
    assert S.sample_tokens(z, 0.0, 1, 2)[2] == 17


def test_softcap_closed_forms():
    cap = 30.0
    y = np.array([0.0, 1e-3, -2.5, 29.0, 300.0, -1e6])
    z = S.softcap(y, cap)
    assert z[0] == 0.0
    assert np.all(np.abs(z) <= cap)                                   # (tanh rounds to 1 far out)
    assert np.allclose(S.softcap(-y, cap), -z)                         # odd
    small = np.array([1e-3, -0.02, 0.1])
    taylor = small - small**3 / (3 * cap**2) + 2 * small**5 / (15 * cap**4)   # tanh series to 5th order
    assert np.allclose(S.softcap(small, cap), taylor, rtol=0, atol=1e-15)
    assert abs(S.softcap(np.array([1e6]), cap)[0] - cap) < 1e-12
    assert np.array_equal(S.softcap(y, 0.0), y) and np.array_equal(S.softcap(y, -1.0), y)
