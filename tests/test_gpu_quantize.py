"""GPU parity of the NVFP4 quantizer (q4_nvfp4_quantize) against the oracle.

Bar: bit-exact.  The packed bytes equal the host repack of the oracle's codes
and scales (the oracle takes every decision in float32, as the kernel does),
and the global scale equals the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def q4():
    import moe_w4a16_skinny_amd as m
    return m


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def note(*a):
    print(*a, flush=True)


def expect_packed(w, global_scale=None):
    codes, scales, g = oracle.nvfp4_quantize_f32(w, global_scale)
    return q4().q4_nvfp4_repack(codes, scales), np.float32(g)


def run(w, global_scale=0.0):
    packed, g = q4().q4_nvfp4_quantize(dev(w), global_scale)
    torch.cuda.synchronize()
    return packed.cpu().numpy(), np.float32(g.cpu().numpy()[0])


@pytest.mark.parametrize("N,K", [(16, 16), (32, 80), (48, 704), (16, 128), (64, 2816), (1024, 2816), (256, 4096),
                                 (96, 1088)])
def test_quantize_matches_oracle(N, K):
    # 16/80/704/1088: K ends inside a 64-k half tile or pads a tile with zero groups
    note(f"quantize N={N} K={K}")
    w = synth.normal_f32(500 + N + K, synth.TAG_WEIGHT, N, K, 0.02)
    got, g = run(w)
    ref, g_ref = expect_packed(w)
    assert g.view(np.uint32) == g_ref.view(np.uint32)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


def test_quantize_given_global_scale_and_saturation():
    # a given g: groups far above 448 * 6 * g saturate their scale (0x7E) and codes (+-6)
    w = synth.normal_f32(7, synth.TAG_WEIGHT, 64, 512, 1.0)
    for gs in (1e-4, 1e-3, 0.05, 3.0):
        got, g = run(w, gs)
        ref, g_ref = expect_packed(w, gs)
        assert g == np.float32(gs) and g_ref == np.float32(gs)
        assert np.array_equal(got, ref), gs
    _, scales = q4().q4_nvfp4_unpack(run(w, 1e-4)[0], 64, 512)
    assert np.all(scales == 0x7E)


def tie_matrix():
    """Groups that land on rounding midpoints, with g = 1: the E2M1 midpoints
    (group amax 6 gives scale 1), the 126 E4M3 midpoints (group amax 6 * mid
    gives target mid exactly), E4M3 subnormal targets and targets that round
    to a zero scale."""
    e4 = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = (e4[:-1] + e4[1:]) / 2
    rng = np.random.default_rng(11)
    groups = []
    e2 = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -0.0]
    groups.append(np.array(e2))
    groups.append(-np.array(e2))
    for m in mids:
        amax = 6.0 * m
        v = rng.uniform(-amax, amax, 16)
        v[rng.integers(16)] = amax if rng.integers(2) else -amax
        groups.append(v)
    for t in (2.0 ** -7, 3 * 2.0 ** -10, 2.0 ** -10, 2.0 ** -11, 2.0 ** -12, 1e-30):
        v = rng.uniform(-6 * t, 6 * t, 16)
        v[0] = 6 * t
        groups.append(v)
    groups.append(np.zeros(16))
    while len(groups) % 16:
        groups.append(rng.standard_normal(16))
    w = np.concatenate(groups).astype(np.float32)
    return w.reshape(16, -1)


def test_quantize_rounding_ties():
    w = tie_matrix()
    assert w.shape[1] % 16 == 0
    got, _ = run(w, 1.0)
    ref, _ = expect_packed(w, 1.0)
    assert np.array_equal(got, ref)


F32 = np.float32
E2M1_DECISIONS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)   # the magnitudes where the E2M1 code steps


def as_matrix(groups, seed):
    """groups of 16 values -> a [16][K] matrix (padding groups of noise)"""
    rng = np.random.default_rng(seed)
    groups = list(groups)
    while len(groups) % 16:
        groups.append(rng.standard_normal(16))
    return np.concatenate(groups).astype(F32).reshape(16, -1)


def test_quantize_encoder_near_every_decision():
    # g = 1 and a group amax of 6 give S = 1, so the codes are those of the
    # values themselves: every float within 2048 ulps of each E2M1 decision
    # point, both signs, signed zeros and the smallest subnormals
    vals = []
    for t in E2M1_DECISIONS:
        b = np.array([t], F32).view(np.uint32)[0]
        vals.append((b + np.arange(-2048, 2049, dtype=np.int64)).astype(np.uint32).view(F32))
    vals.append(np.array([0.0, 1e-45, 1e-40, 2.0 ** -126, 6.0, 5.999999], F32))
    v = np.concatenate(vals)
    v = np.concatenate([v, -v])
    groups = [np.concatenate([[6.0 if i % 2 else -6.0], v[i:i + 15]]) for i in range(0, len(v), 15)]
    groups[-1] = np.concatenate([groups[-1], np.zeros(16 - len(groups[-1]))])
    w = as_matrix(groups, 3)
    got, _ = run(w, 1.0)
    ref, _ = expect_packed(w, 1.0)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("g", [1.0, 0.0123456789, 3.3e-7, 2.0 ** -70, 7.7e5])
def test_quantize_quotients_near_every_decision(g):
    # a full-precision S = RN(e4m3(s) * g) and values a few ulps either side of
    # S times each decision point: the quotients w / S must round exactly as
    # the IEEE division does
    g = F32(g)
    rng = np.random.default_rng(int(g.view(np.uint32)))
    groups = []
    for _ in range(512):
        A = F32(6.0 * float(g) * 2.0 ** rng.uniform(-5.5, 8.7))
        if not np.isfinite(A) or A == 0:
            continue
        _, sc, _ = oracle.nvfp4_quantize_f32(np.array([[A] + [0.0] * 15], F32), g)
        S = F32(float(oracle.e4m3_value(sc[0, 0])) * float(g))
        xs = [A]
        for _ in range(15):
            c = F32(float(rng.choice(E2M1_DECISIONS)) * float(S)).view(np.uint32)
            x = np.array([c + rng.integers(-6, 7)], np.uint32).view(F32)[0]
            x = min(x, A) * (1 if rng.integers(2) else -1)
            xs.append(x)
        groups.append(np.array(xs, F32))
    w = as_matrix(groups, 4)
    got, _ = run(w, float(g))
    ref, _ = expect_packed(w, float(g))
    assert np.array_equal(got, ref)


def test_quantize_zero_matrix_and_all_equal():
    got, g = run(np.zeros((32, 256), np.float32))
    assert g == 0.0 and not got.any()
    # every value equal: amax / 6 / g = 448 exactly, scale 0x7E, codes +-6
    w = np.full((16, 128), -0.5, np.float32)
    got, g = run(w)
    ref, g_ref = expect_packed(w)
    assert g.view(np.uint32) == g_ref.view(np.uint32) and np.array_equal(got, ref)
    codes, scales = q4().q4_nvfp4_unpack(got, 16, 128)
    assert np.all(scales == 0x7E) and np.all(codes == 0xFF)


def test_quantize_amax_planted_everywhere():
    # the tensor amax is found wherever it sits: 4096 x 2816 values take the
    # amax pass's steady double-buffered loop, its first batch and its
    # remainder loop; one planted maximum (either sign) at a time, at the
    # ends, inside each range, and at float4 and grid-pass boundaries.  g is
    # amax / 2688 in float32, as the oracle forms it.
    N, K = 4096, 2816
    base = synth.normal_f32(57, synth.TAG_WEIGHT, N, K, 0.02)
    big = np.float32(7.25)
    assert np.max(np.abs(base)) < big
    n = N * K
    stride = 4 * 256 * 256  # values one grid pass covers
    at = [0, 3, stride - 1, 8 * stride + 5, n // 2 + 1, n - stride + 2, n - 4, n - 1]
    want = np.float32(big / np.float32(2688.0))
    _, _, g_oracle = oracle.nvfp4_quantize_f32(np.array([[big] + [0.0] * 15] * 16, np.float32))
    assert np.float32(g_oracle).view(np.uint32) == want.view(np.uint32)
    m = q4()
    tw = dev(base)
    for i, pos in enumerate(at):
        r, c = divmod(pos, K)
        tw[r, c] = float(big if i % 2 else -big)
        _, g = m.q4_nvfp4_quantize(tw)
        torch.cuda.synchronize()
        tw[r, c] = float(base[r, c])
        assert np.float32(g.cpu().numpy()[0]).view(np.uint32) == want.view(np.uint32), f"planted at {pos}"


def test_quantize_then_gemm():
    # the quantized matrix feeds the GEMM directly: the product matches the
    # oracle GEMM on the oracle's codes within the GEMM bound
    m = q4()
    M, K, N = 16, 2816, 1024
    w = synth.normal_f32(31, synth.TAG_WEIGHT, N, K, 0.02)
    a = synth.act_f16(32, M, K)
    packed, g = m.q4_nvfp4_quantize(dev(w))
    y = m.qgemm_nvfp4(packed, float(g.cpu().numpy()[0]), dev(a), N)
    torch.cuda.synchronize()
    codes, scales, g_ref = oracle.nvfp4_quantize_f32(w)
    ref, bnd = oracle.nvfp4_gemm_ref(codes, scales, g_ref, a)
    assert np.all(np.abs(y.cpu().numpy() - ref) <= 1e-3 * bnd)


def test_quantize_repeat_and_reused_workspace():
    # two calls in a row (the amax word is reused), the second on a smaller matrix
    w1 = synth.normal_f32(41, synth.TAG_WEIGHT, 256, 1024, 0.5)
    w2 = synth.normal_f32(42, synth.TAG_WEIGHT, 32, 256, 0.01)
    run(w1)
    got, g = run(w2)
    ref, g_ref = expect_packed(w2)
    assert g.view(np.uint32) == g_ref.view(np.uint32) and np.array_equal(got, ref)


def test_quantize_tied_embedding_full_size_sampled():
    # the tied embedding (262144 x 2816 fp32, N(0, 0.02)): g bit-exact over
    # the whole matrix; 64 sampled 16-row panels bit-exact
    m = q4()
    wl = synth.WORKLOADS["nvfp4_quantize_n262144_k2816"]
    N, K = wl["N"], wl["K"]
    w = synth.normal_f32(wl["seed"], synth.TAG_WEIGHT, N, K, wl["std"])
    note(f"quantize full size N={N} K={K}")
    wd = dev(w)
    packed, g = m.q4_nvfp4_quantize(wd)
    torch.cuda.synchronize()
    del wd
    g = np.float32(g.cpu().numpy()[0])
    g_ref = oracle.nvfp4_global_scale_f32(w)
    assert g.view(np.uint32) == g_ref.view(np.uint32)
    pb = m.q4_nvfp4_packed_bytes(16, K)
    panels = np.random.default_rng(5).choice(N // 16, 64, replace=False)
    panels[:2] = (0, N // 16 - 1)
    got = packed.cpu().numpy()
    for p in panels:
        ref, _ = expect_packed(w[16 * p:16 * p + 16], g_ref)
        assert np.array_equal(got[p * pb:(p + 1) * pb], ref[:pb]), p


def test_quantize_rejects_bad_arguments():
    m = q4()
    w = torch.zeros((16, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(m.Q4Error):
        m.q4_nvfp4_quantize(torch.zeros((15, 64), dtype=torch.float32, device="cuda"))
    with pytest.raises(m.Q4Error):
        m.q4_nvfp4_quantize(torch.zeros((16, 24), dtype=torch.float32, device="cuda"))
    with pytest.raises(m.Q4Error):
        m.q4_nvfp4_quantize(w, float("inf"))
    with pytest.raises(m.Q4Error):
        m.q4_nvfp4_quantize(w, packed=torch.empty((100,), dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        m.q4_nvfp4_quantize(w.half())
