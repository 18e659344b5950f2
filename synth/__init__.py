"""Seeded synthetic inputs for the W4A16 skinny GEMM and the top-8 MoE layer.

Both the HIP path (tests, benchmark) and the CPU oracle consume what this
module produces; it is the only code the two sides share.  It draws random
numbers and stores them in the input formats the path reads:

* NVFP4 weights (gemma-cuda-hybrid README, "Everything it has"): 4-bit E2M1
  codes, one E4M3 scale per 16 weights along K and one fp32 global scale.
  The float weights are drawn N(0, 0.02) and encoded by the workload recipe
  below; the hot path itself never quantizes, it only decodes.
* MLX-style affine 4-bit weights (TensorFold issue "Proposal: Gemma 4 on
  CUDA", "Why now": qlinear's affine paths in groups of 64): uint4 codes with
  a bf16 scale and a bf16 bias per 64 weights along K.
* f16 / bf16 activations N(0, 1) and an fp32 router matrix N(0, 0.02).

Nothing here dequantizes, multiplies, routes or reduces: that arithmetic
lives on the HIP side and, independently, in the oracle.

NVFP4 encoding recipe (the synthetic-weight recipe; the pages do not spell
out the rounding, the readings taken are listed with the design notes):

1. ``g = f32(max|W|) / f32(2688)`` as one fp32 division (2688 = 448 * 6:
   the largest E4M3 value times the largest E2M1 value).
2. For each group of 16 consecutive weights of a row: ``t = (amax/6)/g`` in
   float64, rounded to E4M3 (OCP E4M3FN) to nearest-even, saturating at 448.
3. ``S = E4M3(s) * g`` (exact in float64); if ``S == 0`` every code is +0,
   else each weight is encoded as the E2M1 value nearest to ``w / S``
   (ties to the even code, magnitudes above 6 saturate to 6, sign kept).
4. Codes are packed two per byte, the even-k element in the low nibble.

Every random stream is a ``numpy.random.Generator`` (PCG64) seeded with
``SeedSequence([seed, stream_tag, block])``; large matrices are drawn in
blocks of 16384 rows so they can be produced in parallel and in chunks.
"""
from __future__ import annotations

import concurrent.futures as _fut
import os
from dataclasses import dataclass

import numpy as np

BLOCK_ROWS = 16384

# stream tags (second word of the SeedSequence entropy)
TAG_WEIGHT = 1
TAG_ACT = 2
TAG_ROUTER = 3
TAG_EXPERT = 4
TAG_AFF_CODES = 5
TAG_AFF_SCALE = 6
TAG_AFF_BIAS = 7
TAG_BLOCK = 8

_E4M3_MAX = 448.0
_E2M1_MAX = 6.0


def _rng(seed: int, tag: int, block: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tag), int(block)]))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed: int, tag: int, rows: int, cols: int, std: float) -> np.ndarray:
    """fp32 matrix [rows][cols] drawn N(0, std^2), row blocks of 16384 seeded separately."""
    out = np.empty((rows, cols), np.float32)
    blocks = [(b, b * BLOCK_ROWS, min(rows, (b + 1) * BLOCK_ROWS))
              for b in range((rows + BLOCK_ROWS - 1) // BLOCK_ROWS)]

    def draw(job):
        b, r0, r1 = job
        x = _rng(seed, tag, b).standard_normal((r1 - r0, cols), dtype=np.float32)
        x *= np.float32(std)
        out[r0:r1] = x

    if len(blocks) == 1:
        draw(blocks[0])
    else:
        with _fut.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(draw, blocks))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even) and return the 16-bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# NVFP4 encoding (input recipe)
# --------------------------------------------------------------------------

def encode_e4m3_rne_satfinite(t: np.ndarray) -> np.ndarray:
    """Encode non-negative float64 values as OCP E4M3FN bytes.

    Round to nearest, ties to even; values beyond 448 saturate to 0x7E; values
    below the smallest subnormal (2^-9) may round to +0.
    """
    t = np.asarray(t, np.float64)
    if np.any(t < 0) or not np.all(np.isfinite(t)):
        raise ValueError("E4M3 scale targets must be finite and non-negative")
    _, ex = np.frexp(t)                      # t = f * 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1              # t in [2^e, 2^(e+1))
    e = np.where(t == 0, -6, np.maximum(e, -6))  # subnormals share the 2^-6 binade's quantum
    quantum = np.ldexp(1.0, (e - 3).astype(np.int32))
    m = np.rint(t / quantum).astype(np.int64)  # exact scaling by a power of two, then RNE
    # normal binade: m in [8, 16], code = exponent field << 3 | (m - 8); m == 16
    # carries into the exponent field.  Subnormal binade (e == -6 and t < 2^-6):
    # m in [0, 8] and the same expression reduces to code == m.
    code = ((e + 7) << 3) + (m - 8)
    code = np.minimum(code, 0x7E)            # satfinite: never emit NaN (0x7F)
    return code.astype(np.uint8)


# magnitude thresholds of the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}; at a midpoint
# the even code wins: ties at .25, 1.25, 2.5, 5 go down, at .75, 1.75, 3.5 go up.
_E2M1_UP_STRICT = (0.25, 1.25, 2.5, 5.0)     # count when x >  threshold
_E2M1_UP_TIE = (0.75, 1.75, 3.5)             # count when x >= threshold


def encode_e2m1_rne_satfinite(x: np.ndarray) -> np.ndarray:
    """Encode float64 values as E2M1 codes (sign bit 3, magnitude index bits 0-2)."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    mag = np.zeros(a.shape, np.uint8)
    for th in _E2M1_UP_STRICT:
        mag += (a > th)
    for th in _E2M1_UP_TIE:
        mag += (a >= th)
    sign = np.signbit(x).astype(np.uint8)
    return (mag | (sign << 3)).astype(np.uint8)


_E4M3_SCALE_CACHE: dict = {}


def _e4m3_byte_values() -> np.ndarray:
    # the values of the 127 finite non-negative E4M3 bytes, used only to turn an
    # encoded scale back into the divisor of step 3 of the recipe.
    if "v" not in _E4M3_SCALE_CACHE:
        b = np.arange(128, dtype=np.int64)
        ex, mt = (b >> 3) & 15, b & 7
        v = np.where(ex == 0, mt / 8.0 * 2.0 ** -6, (1 + mt / 8.0) * np.exp2(ex - 7.0))
        v[0x7F] = np.nan
        _E4M3_SCALE_CACHE["v"] = v
    return _E4M3_SCALE_CACHE["v"]


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """[..., K] codes 0..15 -> [..., K/2] bytes, element 2j in the low nibble."""
    q = np.asarray(q, np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def nvfp4_global_scale(w: np.ndarray) -> np.float32:
    amax = np.float32(np.max(np.abs(w))) if w.size else np.float32(0)
    return np.float32(amax / np.float32(_E4M3_MAX * _E2M1_MAX))


def quantize_nvfp4(w: np.ndarray, g: np.float32 | None = None):
    """Encode fp32 weights [N][K] (K % 16 == 0) -> (codes u8[N][K/2], scales u8[N][K/16], g f32)."""
    w = np.ascontiguousarray(w, np.float32)
    N, K = w.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    if g is None:
        g = nvfp4_global_scale(w)
    g = np.float32(g)
    codes = np.empty((N, K // 2), np.uint8)
    scales = np.empty((N, K // 16), np.uint8)
    svals = _e4m3_byte_values()

    def enc(r0, r1):
        blk = w[r0:r1].astype(np.float64).reshape(r1 - r0, K // 16, 16)
        amax = np.max(np.abs(blk), axis=2)
        if g > 0:
            t = (amax / 6.0) / np.float64(g)
        else:
            t = np.zeros_like(amax)
        s = encode_e4m3_rne_satfinite(t)
        S = svals[s] * np.float64(g)
        with np.errstate(divide="ignore", invalid="ignore"):
            x = np.where(S[..., None] > 0, blk / S[..., None], 0.0)
        q = encode_e2m1_rne_satfinite(x)
        q = np.where(S[..., None] > 0, q, 0).astype(np.uint8)  # zero group -> all +0
        codes[r0:r1] = pack_nibbles(q.reshape(r1 - r0, K))
        scales[r0:r1] = s

    step = 2048
    jobs = [(r, min(N, r + step)) for r in range(0, N, step)]
    if len(jobs) <= 1:
        for j in jobs:
            enc(*j)
    else:
        with _fut.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda j: enc(*j), jobs))
    return codes, scales, g


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

@dataclass
class NvGemmInputs:
    codes: np.ndarray     # u8 [N][K/2]
    scales: np.ndarray    # u8 [N][K/16]
    g: np.float32
    a: np.ndarray         # f16 [M][K]

    @property
    def shape(self):
        return self.a.shape[0], self.a.shape[1], self.codes.shape[0]


@dataclass
class AffineGemmInputs:
    codes: np.ndarray     # u8 [N][K/2]
    scale: np.ndarray     # u16 bf16 bits [N][K/64]
    bias: np.ndarray      # u16 bf16 bits [N][K/64]
    a: np.ndarray         # u16 bf16 bits [M][K]

    @property
    def shape(self):
        return self.a.shape[0], self.a.shape[1], self.codes.shape[0]


@dataclass
class MoeInputs:
    x: np.ndarray           # f16 [T][D]
    w_router: np.ndarray    # f32 [D][E]
    gate: list              # per expert (codes [F][D/2], scales [F][D/16], g)
    up: list
    down: list              # per expert (codes [D][F/2], scales [D][F/16], g)
    E: int
    k: int
    has_shared: bool

    @property
    def T(self):
        return self.x.shape[0]

    @property
    def D(self):
        return self.x.shape[1]

    @property
    def F(self):
        return self.gate[0][0].shape[0]


@dataclass
class MoeBlockInputs:
    """A Gemma-4 MoE block: routed experts (no shared one), a dense gated FFN
    branch, the router with its learned per-expert scale, the per-expert down
    scale and five RMSNorm weight vectors; residual fp32 [T][D]."""
    residual: np.ndarray    # f32 [T][D]
    w_router: np.ndarray    # f32 [D][E]
    router_scale: np.ndarray  # f32 [E]
    down_scale: np.ndarray    # f32 [E]
    gate: list
    up: list
    down: list
    dense_gate: tuple       # (codes [Fd][D/2], scales [Fd][D/16], g)
    dense_up: tuple
    dense_down: tuple       # (codes [D][Fd/2], scales [D][Fd/16], g)
    ffn_norm: np.ndarray    # f32 [D] each
    post_ffw_norm_1: np.ndarray
    pre_ffw_norm_2: np.ndarray
    post_ffw_norm_2: np.ndarray
    post_ffw_norm: np.ndarray
    E: int
    k: int

    @property
    def T(self):
        return self.residual.shape[0]

    @property
    def D(self):
        return self.residual.shape[1]


def act_f16(seed: int, M: int, K: int) -> np.ndarray:
    return _rng(seed, TAG_ACT).standard_normal((M, K), dtype=np.float32).astype(np.float16)


def act_bf16_bits(seed: int, M: int, K: int) -> np.ndarray:
    return f32_to_bf16_bits(_rng(seed, TAG_ACT).standard_normal((M, K), dtype=np.float32))


def nvfp4_weights(seed: int, N: int, K: int, std: float = 0.02, tag: int = TAG_WEIGHT):
    w = normal_f32(seed, tag, N, K, std)
    return quantize_nvfp4(w)


def nvfp4_gemm(seed: int, M: int, K: int, N: int) -> NvGemmInputs:
    """NVFP4 W4A16 GEMM inputs: W N(0,0.02) encoded by the recipe, a f16 N(0,1)."""
    codes, scales, g = nvfp4_weights(seed, N, K)
    return NvGemmInputs(codes, scales, g, act_f16(seed, M, K))


def affine_weights(seed: int, N: int, K: int):
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    q = _rng(seed, TAG_AFF_CODES).integers(0, 16, size=(N, K), dtype=np.uint8)
    s = np.abs(_rng(seed, TAG_AFF_SCALE).standard_normal((N, K // 64), dtype=np.float32)) * np.float32(0.003)
    b = _rng(seed, TAG_AFF_BIAS).standard_normal((N, K // 64), dtype=np.float32) * np.float32(0.01)
    return pack_nibbles(q), f32_to_bf16_bits(s), f32_to_bf16_bits(b)


def affine_weights_bits(seed: int, N: int, K: int, bits: int):
    """MLX-style affine b-bit weights, codes one per byte [N][K] uniform in
    0..2^b - 1, scale bf16(|N(0, .003)| * 15 / (2^b - 1)) (the 4-bit recipe's
    weight range at every width), bias bf16(N(0, .01)) [N][K/64]."""
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    q = _rng(seed, TAG_AFF_CODES).integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    s = np.abs(_rng(seed, TAG_AFF_SCALE).standard_normal((N, K // 64), dtype=np.float32)) \
        * np.float32(0.003 * 15.0 / ((1 << bits) - 1))
    b = _rng(seed, TAG_AFF_BIAS).standard_normal((N, K // 64), dtype=np.float32) * np.float32(0.01)
    return q, f32_to_bf16_bits(s), f32_to_bf16_bits(b)


def affine_gemm(seed: int, M: int, K: int, N: int) -> AffineGemmInputs:
    """MLX-style affine 4-bit inputs: codes U[0,15], scale bf16(|N(0,.003)|), bias bf16(N(0,.01)), a bf16 N(0,1)."""
    codes, s, b = affine_weights(seed, N, K)
    return AffineGemmInputs(codes, s, b, act_bf16_bits(seed, M, K))


def moe_layer(seed: int, T: int = 16, D: int = 2816, E: int = 128, F: int = 704,
              k: int = 8, has_shared: bool = True) -> MoeInputs:
    """Gemma-4-MoE-shaped layer: x f16 N(0,1) [T][D], W_r fp32 N(0,.02) [D][E], and
    per expert (routed 0..E-1, then the shared one) gate/up [F][D] and down [D][F]
    drawn N(0,.02) and NVFP4-encoded, each matrix with its own global scale."""
    x = act_f16(seed, T, D)
    w_router = _rng(seed, TAG_ROUTER).standard_normal((D, E), dtype=np.float32) * np.float32(0.02)
    n_exp = E + (1 if has_shared else 0)

    def one(e):
        base = TAG_EXPERT * 1_000_000 + 3 * e
        return (nvfp4_weights(seed, F, D, tag=base + 0),
                nvfp4_weights(seed, F, D, tag=base + 1),
                nvfp4_weights(seed, D, F, tag=base + 2))

    if n_exp > 4:
        with _fut.ThreadPoolExecutor(_threads()) as ex:
            mats = list(ex.map(one, range(n_exp)))
    else:
        mats = [one(e) for e in range(n_exp)]
    return MoeInputs(x, w_router, [m[0] for m in mats], [m[1] for m in mats],
                     [m[2] for m in mats], E, k, has_shared)


def moe_block(seed: int, T: int = 16, D: int = 2816, E: int = 128, F: int = 704, F_dense: int = 2112,
              k: int = 8) -> MoeBlockInputs:
    """The MoE layer of moe_layer (routed experts only) plus: residual fp32
    N(0, 1); the dense branch's gate/up [F_dense][D] and down [D][F_dense]
    N(0, .02) NVFP4; router_scale, down_scale and the five norm weights
    drawn 1 + N(0, .1) in fp32."""
    layer = moe_layer(seed, T=T, D=D, E=E, F=F, k=k, has_shared=False)
    residual = _rng(seed, TAG_BLOCK).standard_normal((T, D), dtype=np.float32)
    base = TAG_BLOCK * 1_000_000
    dg = nvfp4_weights(seed, F_dense, D, tag=base + 1)
    du = nvfp4_weights(seed, F_dense, D, tag=base + 2)
    dd = nvfp4_weights(seed, D, F_dense, tag=base + 3)
    r = _rng(seed, TAG_BLOCK, 1)
    one = lambda n: (1.0 + 0.1 * r.standard_normal(n)).astype(np.float32)
    return MoeBlockInputs(residual, layer.w_router, one(E), one(E), layer.gate, layer.up, layer.down,
                          dg, du, dd, one(D), one(D), one(D), one(D), one(D), E, k)


# named workloads: sizes of the decode / speculative-verify shapes on the pages
WORKLOADS = {
    "nvfp4_m1_k1024_n1024": dict(kind="nvfp4", seed=101, M=1, K=1024, N=1024, out="f32"),
    "nvfp4_verify_m16_k4096_n8192": dict(kind="nvfp4", seed=102, M=16, K=4096, N=8192, out="f16"),
    "nvfp4_lmhead_m16_k2816_n262144": dict(kind="nvfp4", seed=103, M=16, K=2816, N=262144,
                                           out="f32", argmax=True),
    # the same lm_head with fused sampling: softcap 30, temperature 1, only the tokens kept
    "nvfp4_lmhead_sample_m16_k2816_n262144": dict(kind="nvfp4", seed=103, M=16, K=2816, N=262144,
                                                  out="none", sample=dict(softcap=30.0, temperature=1.0)),
    "moe_t16_d2816_e128s1_f704_top8": dict(kind="moe", seed=104, T=16, D=2816, E=128, F=704, k=8,
                                           has_shared=True),
    # the whole Gemma-4 MoE block: dense branch (width 2112) + 128 routed experts top-8, norms
    "moe_block_t16_d2816_e128_f704_fd2112_top8": dict(kind="moe_block", seed=108, T=16, D=2816, E=128, F=704,
                                                      F_dense=2112, k=8),
    # a prefill chunk of 512 rows through the verify-shaped weights (M > 16: the matrix-core regime)
    "nvfp4_prefill_m512_k4096_n8192": dict(kind="nvfp4", seed=106, M=512, K=4096, N=8192, out="f32"),
    "nvfp4_prefill_m2048_k4096_n8192": dict(kind="nvfp4", seed=107, M=2048, K=4096, N=8192, out="f32"),
    # the tied embedding in fp32, N(0, 0.02), for the device quantizer
    "nvfp4_quantize_n262144_k2816": dict(kind="quant", seed=103, N=262144, K=2816, std=0.02),
    # the other MLX affine widths at the affine workload's shape
    "affine2_m16_k5120_n15360": dict(kind="affine_bits", bits=2, seed=109, M=16, K=5120, N=15360, out="f32"),
    "affine8_m16_k5120_n15360": dict(kind="affine_bits", bits=8, seed=110, M=16, K=5120, N=15360, out="f32"),
    "affine4_m1_k5120_n15360": dict(kind="affine", seed=105, M=1, K=5120, N=15360, out="f32"),
    "affine4_m16_k5120_n15360": dict(kind="affine", seed=105, M=16, K=5120, N=15360, out="f32"),
}
