"""Oracle for the lm_head's fused sampling: logit softcap and Gumbel-max.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages:
  [DOC 4.8]  TensorSharp docs, Gemma 4, 4.8 "Logit softcap" (and the forward
             graph of section 3, where an optional tanh softcap follows the
             LM head): z = cap * tanh(y / cap) when the cap is positive.
  [README]   gemma-cuda-hybrid README, "Everything it has", server features:
             temperature sampling by the Gumbel-max trick, temperature 0 being
             exact greedy decoding.

The pages name no noise generator.  Reading taken: the uniform draws come
from Philox4x32-10, a counter-based generator with a published definition
(Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
3", SC 2011), so that the GPU can draw them inside the lm_head kernel and
the oracle can draw the very same bits:
  key     = (seed mod 2^32, seed >> 32)
  counter = (n, m // 4, offset, 0), word m % 4 of the output for row m
            (one generator call gives the noise of four rows of a column,
            the rows an MFMA accumulator lane holds)
  U       = (2 (x >> 9) + 1) 2^-24, in (0, 1), exact in float32
  G       = -ln(-ln U)
  token   = argmax_n (z[m, n] / T + G[m, n]) for T > 0, argmax_n z for T = 0,
            the lower index on ties.

Pins (tests/test_oracle_sampling.py): the round function and key schedule
against NumPy's Philox4x64-10 bit generator (same construction, 64-bit
words), the 32-bit variant on published known-answer vectors, the uniform
map's range and exactness, the empirical token frequencies of Gumbel-max
against softmax(z / T), and softcap closed forms.
"""
from __future__ import annotations

import numpy as np

# Philox constants, [Salmon et al. 2011, section 4]: multipliers and the Weyl
# key increments (golden ratio and sqrt(3) - 1 in fixed point)
PHILOX_CONSTS = {
    32: dict(M=(0xD2511F53, 0xCD9E8D57), W=(0x9E3779B9, 0xBB67AE85)),
    64: dict(M=(0xD2E7470EE14C6C93, 0xCA5A826395121157), W=(0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)),
}


def _mulhilo(a: np.ndarray, b: int, bits: int):
    """(high, low) words of the 2*bits-wide product a * b."""
    mask = (1 << bits) - 1
    if bits == 32:
        p = a.astype(np.uint64) * np.uint64(b)
        return (p >> np.uint64(32)).astype(np.uint32), (p & np.uint64(mask)).astype(np.uint32)
    # 64-bit words: split into 32-bit halves (Python ints would be slow for arrays)
    a = a.astype(np.uint64)
    a_lo, a_hi = a & np.uint64(0xFFFFFFFF), a >> np.uint64(32)
    b_lo, b_hi = np.uint64(b & 0xFFFFFFFF), np.uint64(b >> 32)
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> np.uint64(32)) + (lh & np.uint64(0xFFFFFFFF)) + (hl & np.uint64(0xFFFFFFFF))  # < 3 * 2^32
    lo = (ll & np.uint64(0xFFFFFFFF)) | ((mid & np.uint64(0xFFFFFFFF)) << np.uint64(32))
    hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4(ctr, key, bits: int = 32, rounds: int = 10):
    """Philox4x{bits}-{rounds}: four counter words (arrays), two key words
    (arrays or scalars) -> four output words.  Each round multiplies words 0
    and 2 by the two multipliers, and the new words are (hi(M1 c2) ^ c1 ^ k0,
    lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key is bumped by the Weyl
    increments between rounds."""
    dt = np.uint32 if bits == 32 else np.uint64
    mask = (1 << bits) - 1
    M0, M1 = PHILOX_CONSTS[bits]["M"]
    W0, W1 = PHILOX_CONSTS[bits]["W"]
    c0, c1, c2, c3 = (np.asarray(c, dtype=dt) for c in ctr)
    k0 = np.asarray(key[0], dtype=dt)
    k1 = np.asarray(key[1], dtype=dt)
    with np.errstate(over="ignore"):  # word arithmetic wraps modulo 2^bits
        for r in range(rounds):
            if r > 0:
                if bits == 32:
                    k0 = ((k0.astype(np.uint64) + np.uint64(W0)) & np.uint64(mask)).astype(dt)
                    k1 = ((k1.astype(np.uint64) + np.uint64(W1)) & np.uint64(mask)).astype(dt)
                else:
                    k0 = k0 + dt(W0)
                    k1 = k1 + dt(W1)
            hi0, lo0 = _mulhilo(c0, M0, bits)
            hi1, lo1 = _mulhilo(c2, M1, bits)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform_bits_to_f32(x: np.ndarray) -> np.ndarray:
    """32-bit word -> U = (2 (x >> 9) + 1) 2^-24: 2^23 equally spaced values
    strictly inside (0, 1), each exact in float32."""
    x = np.asarray(x, dtype=np.uint32)
    return (((x >> np.uint32(9)).astype(np.float64) * 2.0 + 1.0) * 2.0 ** -24).astype(np.float32)


def sample_uniforms(seed: int, offset: int, M: int, N: int) -> np.ndarray:
    """U[m][n] (float32) for the lm_head's noise, as read by the kernel."""
    M4 = (M + 3) // 4
    nn = np.arange(N, dtype=np.uint32)
    m4 = np.arange(M4, dtype=np.uint32)
    c0 = np.broadcast_to(nn[None, :], (M4, N))
    c1 = np.broadcast_to(m4[:, None], (M4, N))
    c2 = np.full((M4, N), offset & 0xFFFFFFFF, np.uint32)
    c3 = np.zeros((M4, N), np.uint32)
    key = (np.uint32(seed & 0xFFFFFFFF), np.uint32((seed >> 32) & 0xFFFFFFFF))
    x = philox4((c0, c1, c2, c3), key, bits=32)          # word r of block (m4, n) -> row 4 m4 + r
    words = np.stack(x, axis=1).reshape(4 * M4, N)[:M]
    return uniform_bits_to_f32(words)


def gumbel(u: np.ndarray) -> np.ndarray:
    """G = -ln(-ln U) in float64."""
    return -np.log(-np.log(np.asarray(u, np.float64)))


def softcap(y: np.ndarray, cap: float) -> np.ndarray:
    """[DOC 4.8] cap * tanh(y / cap) for cap > 0; y unchanged otherwise."""
    y = np.asarray(y, np.float64)
    if cap <= 0:
        return y
    return cap * np.tanh(y / cap)


def sample_scores(z: np.ndarray, temperature: float, seed: int, offset: int) -> np.ndarray:
    """[README] Gumbel-max scores z / T + G (float64); z itself for T = 0."""
    z = np.asarray(z, np.float64)
    if temperature <= 0:
        return z
    M, N = z.shape
    return z / temperature + gumbel(sample_uniforms(seed, offset, M, N))


def sample_tokens(z: np.ndarray, temperature: float, seed: int, offset: int) -> np.ndarray:
    """Per row, the index of the largest score (the first one on ties)."""
    return np.argmax(sample_scores(z, temperature, seed, offset), axis=1).astype(np.int32)
