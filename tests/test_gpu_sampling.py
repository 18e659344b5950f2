"""GPU parity of the lm_head's fused sampling (qgemm_nvfp4_sample) against the oracle.

Bars: the generator's uniforms bit-exact; softcapped logits within the GEMM
bound (1e-3 * sum_k |a w|, through tanh' <= 1) plus 4e-7 * cap for the
kernel's tanh; tokens equal to the argmax of the oracle's float64 scores
z / T + G computed from the kernel's own logits, except where the two best
scores are closer than the fp32 score error (then the kernel's token must
score within it of the best); token frequencies of Gumbel-max follow
softmax(z / T)."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SCORE_TOL = 2e-5   # fp32 score vs float64 oracle score: logit rounding / T + noise (two hardware logs)


def q4():
    import moe_w4a16_skinny_amd as m
    return m


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def note(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("seed,offset,M,N", [(0, 0, 1, 16), (0x0123456789ABCDEF, 77, 6, 1000), (2**64 - 1, 2**32 - 1, 16, 4096),
                                            (5, 3, 13, 262144)])
def test_uniforms_bit_exact(seed, offset, M, N):
    u = q4().q4_sample_uniforms(seed, offset, M, N).cpu().numpy()
    ref = oracle.sample_uniforms(seed, offset, M, N)
    assert np.array_equal(u.view(np.uint32), ref.view(np.uint32))


def check_tokens(z_gpu, tok, T, seed, offset, what):
    """tokens vs the oracle's scores from the kernel's own (fp32) logits"""
    sc = oracle.sample_scores(z_gpu.astype(np.float64), T, seed, offset)
    best = sc.max(axis=1)
    ref = np.argmax(sc, axis=1)
    mine = sc[np.arange(sc.shape[0]), tok]
    assert np.all(tok >= 0) and np.all(tok < sc.shape[1]), what
    assert np.all(mine >= best - SCORE_TOL), f"{what}: a token scores below the best by more than the tolerance"
    second = np.partition(sc, -2, axis=1)[:, -2]
    clear = best - second > SCORE_TOL
    assert np.array_equal(tok[clear], ref[clear]), what
    if (~clear).any():
        note(f"{what}: {int((~clear).sum())} row(s) with a near-tie, checked against the tolerance only")


CASES = [  # (M, K, N, config or None): in-stream keys (one k-range, one k-split wave), epilogue keys
    (16, 2816, 4096, "2,8,4,1,1,16"),     # keys taken during the stream
    (16, 2816, 4096, None),               # default (the ring, 8 k-split waves): keys in the epilogue
    (7, 704, 1024, "2,8,4,1,1,16"),       # half tile: keys in the epilogue
    (5, 1024, 2048, "2,8,4,2,1,16"),      # two k-ranges: keys in the last workgroup
    (1, 1024, 1024, None),
]


@pytest.mark.parametrize("M,K,N,cfg", CASES)
@pytest.mark.parametrize("softcap,T", [(0.0, 0.0), (30.0, 0.0), (0.0, 1.0), (30.0, 0.7), (5.0, 2.5)])
def test_sample_parity(M, K, N, cfg, softcap, T, monkeypatch):
    m = q4()
    if cfg:
        monkeypatch.setenv("Q4MI_GEMM_CFG", cfg)
    note(f"sample M={M} K={K} N={N} cfg={cfg} softcap={softcap} T={T}")
    inp = synth.nvfp4_gemm(3000 + M + K + N, M, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    seed, offset = 0xC0FFEE + M, 11
    z, tok = m.qgemm_nvfp4_sample(w, float(inp.g), dev(inp.a), N, softcap=softcap, temperature=T, seed=seed,
                                  offset=offset)
    torch.cuda.synchronize()
    z = z.cpu().numpy()
    tok = tok.cpu().numpy()
    # logits: softcap of the oracle GEMM, within the GEMM bound plus the tanh's error
    y_ref, bnd = oracle.nvfp4_gemm_ref(inp.codes, inp.scales, inp.g, inp.a)
    z_ref = oracle.softcap(y_ref, softcap)
    tol = 1e-3 * bnd + (4e-7 * softcap if softcap > 0 else 0.0) + np.abs(z_ref) * 2.0 ** -23
    err = np.abs(z.astype(np.float64) - z_ref)
    assert np.all(err <= tol), f"worst err/tol {np.max(err / tol):.3e}"
    check_tokens(z, tok, T, seed, offset, f"M={M} K={K} N={N} cfg={cfg} cap={softcap} T={T}")
    # without the logits stored: the same tokens
    _, tok2 = m.qgemm_nvfp4_sample(w, float(inp.g), dev(inp.a), N, softcap=softcap, temperature=T, seed=seed,
                                   offset=offset, want_logits=False)
    torch.cuda.synchronize()
    assert np.array_equal(tok2.cpu().numpy(), tok)


def test_sample_greedy_matches_fused_argmax():
    m = q4()
    M, K, N = 16, 2816, 8192
    inp = synth.nvfp4_gemm(41, M, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    a = dev(inp.a)
    y, am = m.qgemm_nvfp4(w, float(inp.g), a, N, want_argmax=True)
    z, tok = m.qgemm_nvfp4_sample(w, float(inp.g), a, N)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), z.view(torch.int32))
    assert torch.equal(am, tok)


def test_sample_lm_head_shape_and_offsets():
    # the lm_head shape (262144 vocab rows, keys taken in the stream): tokens
    # against the oracle's scores; successive offsets draw different tokens
    m = q4()
    M, K, N = 16, 2816, 262144
    inp = synth.nvfp4_gemm(synth.WORKLOADS["nvfp4_lmhead_m16_k2816_n262144"]["seed"], M, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    a = dev(inp.a)
    toks = []
    for off in (0, 1, 2):
        z, tok = m.qgemm_nvfp4_sample(w, float(inp.g), a, N, softcap=30.0, temperature=1.0, seed=1234, offset=off)
        torch.cuda.synchronize()
        check_tokens(z.cpu().numpy(), tok.cpu().numpy(), 1.0, 1234, off, f"lm_head offset {off}")
        toks.append(tok.cpu().numpy())
    assert not np.array_equal(toks[0], toks[1]) and not np.array_equal(toks[1], toks[2])
    # repeated call: bitwise the same
    z2, tok2 = m.qgemm_nvfp4_sample(w, float(inp.g), a, N, softcap=30.0, temperature=1.0, seed=1234, offset=2)
    torch.cuda.synchronize()
    assert np.array_equal(tok2.cpu().numpy(), toks[2])


def test_sample_frequencies_follow_softmax():
    # 16 rows x 300 offsets of one 16-column vocab: P(token) = softmax(z / T)
    m = q4()
    M, K, N, T = 16, 256, 16, 0.8
    inp = synth.nvfp4_gemm(77, M, K, N)
    a = inp.a.copy()
    a[:] = a[0]                                   # every row the same logits
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    ad = dev(a)
    counts = np.zeros(N)
    z = None
    for off in range(300):
        z, tok = m.qgemm_nvfp4_sample(w, float(inp.g), ad, N, temperature=T, seed=99, offset=off)
        counts += np.bincount(tok.cpu().numpy(), minlength=N)
    torch.cuda.synchronize()
    zz = z.cpu().numpy()[0].astype(np.float64)
    p = np.exp(zz / T - np.max(zz / T))
    p /= p.sum()
    R = counts.sum()
    sd = np.sqrt(p * (1 - p) / R)
    assert np.all(np.abs(counts / R - p) < 5 * sd + 1e-9), (counts / R, p)


def test_sample_rejects_bad_arguments():
    m = q4()
    inp = synth.nvfp4_gemm(5, 2, 128, 32)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    a = dev(inp.a)
    for kw in (dict(temperature=-1.0), dict(temperature=float("nan")), dict(softcap=float("inf"))):
        with pytest.raises(m.Q4Error):
            m.qgemm_nvfp4_sample(w, float(inp.g), a, 32, **kw)
