"""GPU parity of the dequantization and the two skinny GEMMs against the oracle.

Bars: dequantized weights bit-exact (fp32 patterns, -0.0 and NaN included);
GEMM outputs within 1e-3 * sum_k |a w| per element; argmax bit-exact (the
lowest index among equal stored values), with near-ties of the oracle
reported, not failed; repeated calls bitwise identical."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

REL = 1e-3
# "P,W,D,KS,KW,PB[,RING]": panels per wave group, waves, loads in flight, k-ranges, k-split waves,
# panels per workgroup, activations moved per wave into an LDS ring (1) or staged per workgroup
CFGS = ["1,4,4,1,1,4", "1,4,4,3,1,8", "2,4,4,1,1,8", "2,4,4,4,1,8", "2,8,4,1,1,16", "2,8,4,2,1,48", "4,4,4,1,1,16",
        "4,8,4,5,1,32", "2,4,8,1,1,8", "2,8,8,7,1,16", "4,4,6,2,1,64", "2,8,4,1,8,2", "2,8,4,2,4,4", "1,4,4,3,2,2",
        "4,8,4,1,2,16",
        # activations moved by each wave into its own LDS ring
        "2,8,4,1,8,2,1", "2,8,4,2,4,4,1", "1,4,4,3,2,2,1", "4,8,4,1,2,8,1", "2,4,8,1,1,8,1", "4,4,6,2,1,16,1",
        "2,4,4,1,1,16,1",
        # two tiles in flight
        "2,8,2,1,4,4", "2,8,2,2,2,8", "2,8,2,1,1,16"]


def q4():
    import moe_w4a16_skinny_amd as m
    return m


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def check_gemm(y_gpu, y_ref, bnd, what):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    err = np.abs(y - y_ref)
    worst = np.max(err / np.maximum(bnd, 1e-300))
    assert np.all(np.isfinite(y)), what
    assert np.all(err <= REL * bnd), f"{what}: worst err/bound {worst:.3e} > {REL}"
    return worst


# ---------------------------------------------------------------- dequant

def test_dequant_nvfp4_all_code_scale_pairs():
    m = q4()
    # row n uses scale byte n in every group; codes cycle 0..15 along k -> all 4096 pairs
    N, K = 256, 256
    q = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    scales = np.tile(np.arange(256, dtype=np.uint8)[:, None], (1, K // 16))
    codes = synth.pack_nibbles(q)
    for g in (np.float32(1.0), np.float32(3.7e-5)):
        w = dev(m.q4_nvfp4_repack(codes, scales))
        got = m.q4_dequant_nvfp4(w, float(g), N, K).cpu().numpy()
        ref = oracle.nvfp4_dequant_f32(codes, scales, g)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # incl. -0.0


@pytest.mark.parametrize("N,K", [(64, 1024), (48, 704), (16, 80), (32, 176), (16, 2816)])
def test_dequant_nvfp4_shapes(N, K):
    m = q4()
    inp = synth.nvfp4_gemm(300 + K, 1, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    got = m.q4_dequant_nvfp4(w, float(inp.g), N, K).cpu().numpy()
    ref = oracle.nvfp4_dequant_f32(inp.codes, inp.scales, inp.g)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("N,K", [(32, 128), (16, 64), (48, 704), (16, 5120)])
def test_dequant_affine_bit_exact(N, K):
    m = q4()
    codes, s, b = synth.affine_weights(400 + K, N, K)
    w = dev(m.q4_affine4_repack(codes, s, b))
    got = m.q4_dequant_affine4(w, N, K).cpu().numpy()
    ref = oracle.affine_dequant_f32(codes, s, b)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- NVFP4 GEMM

NV_SHAPES = [  # (M, K, N): tile edges, tails, ragged M, the decode / verify shapes
    (1, 1024, 1024), (16, 4096, 8192), (2, 704, 48), (15, 2816, 64), (16, 80, 32),
    (3, 176, 16), (16, 128, 16), (7, 4096, 272), (1, 64, 16), (4, 2816, 1408), (16, 5120, 160),
    (16, 65536, 1024), (12, 131072, 1024),  # long K (512 and 1024 tiles a row)
]


@pytest.mark.parametrize("M,K,N", NV_SHAPES)
@pytest.mark.parametrize("out_dtype", ["f32", "f16"])
def test_qgemm_nvfp4_parity(M, K, N, out_dtype):
    m = q4()
    note(f"nvfp4 M={M} K={K} N={N} out={out_dtype}")
    inp = synth.nvfp4_gemm(1000 + M * 7 + K + N, M, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    a = dev(inp.a)
    dt = torch.float32 if out_dtype == "f32" else torch.float16
    y = m.qgemm_nvfp4(w, float(inp.g), a, N, out_dtype=dt)
    torch.cuda.synchronize()
    ref, bnd = oracle.nvfp4_gemm_ref(inp.codes, inp.scales, inp.g, inp.a)
    check_gemm(y, ref, bnd, f"nvfp4 {M}x{K}x{N} {out_dtype}")


@pytest.mark.parametrize("cfg", CFGS)
def test_qgemm_nvfp4_every_config(cfg, monkeypatch):
    m = q4()
    monkeypatch.setenv("Q4MI_GEMM_CFG", cfg)
    for (M, K, N) in [(16, 2816, 400), (5, 704, 96), (1, 1024, 48), (16, 80, 32)]:
        inp = synth.nvfp4_gemm(77 + K + N, M, K, N)
        w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
        y, am = m.qgemm_nvfp4(w, float(inp.g), dev(inp.a), N, want_argmax=True)
        torch.cuda.synchronize()
        ref, bnd = oracle.nvfp4_gemm_ref(inp.codes, inp.scales, inp.g, inp.a)
        check_gemm(y, ref, bnd, f"cfg {cfg} {M}x{K}x{N}")
        yc = y.cpu().numpy()
        assert np.array_equal(am.cpu().numpy(), np.argmax(yc, axis=1).astype(np.int32))


def test_qgemm_nvfp4_deterministic():
    m = q4()
    inp = synth.nvfp4_gemm(5, 16, 4096, 8192)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    a = dev(inp.a)
    y1 = m.qgemm_nvfp4(w, float(inp.g), a, 8192).clone()
    y2 = m.qgemm_nvfp4(w, float(inp.g), a, 8192)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_argmax_planted_ties():
    m = q4()
    M, K, N = 16, 256, 512
    inp = synth.nvfp4_gemm(11, M, K, N)
    codes, scales = inp.codes.copy(), inp.scales.copy()
    # duplicate rows 100 -> 7 and 300 -> 200: equal weights give bitwise-equal logits
    codes[7], scales[7] = codes[100], scales[100]
    codes[300], scales[300] = codes[200], scales[200]
    a = inp.a.copy()
    # make row 0 favour column 100 strongly (and therefore its twin 7)
    w64 = oracle.nvfp4_dequant(codes, scales, inp.g)
    a[0] = (np.sign(w64[100]) * 2.0).astype(np.float16)
    w = dev(m.q4_nvfp4_repack(codes, scales))
    y, am = m.qgemm_nvfp4(w, float(inp.g), dev(a), N, want_argmax=True)
    torch.cuda.synchronize()
    yc, amc = y.cpu().numpy(), am.cpu().numpy()
    assert np.array_equal(yc[:, 7], yc[:, 100]) and np.array_equal(yc[:, 200], yc[:, 300])
    assert amc[0] == 7                                   # tie with 100 -> lower index
    assert np.array_equal(amc, np.argmax(yc, axis=1))    # numpy picks the first maximum
    ref, bnd = oracle.nvfp4_gemm_ref(codes, scales, inp.g, a)
    check_gemm(y, ref, bnd, "ties")
    assert oracle.argmax_ref(ref)[0] == 7


def test_argmax_f16_output_and_repeat():
    m = q4()
    M, K, N = 9, 704, 4096
    inp = synth.nvfp4_gemm(12, M, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    a = dev(inp.a)
    for _ in range(3):  # the workspace is left clean for the next call
        y, am = m.qgemm_nvfp4(w, float(inp.g), a, N, out_dtype=torch.float16, want_argmax=True)
        torch.cuda.synchronize()
        yc = y.float().cpu().numpy()
        assert np.array_equal(am.cpu().numpy(), np.argmax(yc, axis=1))


def test_lm_head_tied_embedding_full_shape():
    """The tied NVFP4 lm_head at its own shape, M = 16, K = 2816, N = 262,144,
    in the configuration the library picks for it (f32 logits and the fused
    argmax): every logit within 1e-3 * sum|a w| of the oracle; each row's
    argmax equal to the oracle's (argmax_ref, on fp32-rounded exact logits),
    except on a row whose oracle top-two margin is within twice the observed
    error of the two candidates, where the device's index must be one of the
    two; the argmax equal to that of the stored logits; the sampler at
    temperature 0 and no softcap returning the same tokens."""
    m = q4()
    M, K, N = 16, 2816, 262144
    note("lm_head: generating the 262144 x 2816 tied embedding (seed of the lm_head workload)")
    inp = synth.nvfp4_gemm(103, M, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    a = dev(inp.a)
    y, am = m.qgemm_nvfp4(w, float(inp.g), a, N, want_argmax=True)
    _, tok = m.qgemm_nvfp4_sample(w, float(inp.g), a, N, softcap=0.0, temperature=0.0, want_logits=False)
    torch.cuda.synchronize()
    yc, amc, tkc = y.cpu().numpy().astype(np.float64), am.cpu().numpy(), tok.cpu().numpy()
    del w
    ref = np.empty((M, N))
    err = np.empty((M, N))
    step = 16384
    for c0 in range(0, N, step):
        r, b = oracle.nvfp4_gemm_ref(inp.codes[c0:c0 + step], inp.scales[c0:c0 + step], inp.g, inp.a)
        e = np.abs(yc[:, c0:c0 + step] - r)
        assert np.all(e <= REL * b), f"columns {c0}..: worst err/bound {np.max(e / b):.3e}"
        ref[:, c0:c0 + step] = r
        err[:, c0:c0 + step] = e
        if c0 % (8 * step) == 0:
            note(f"lm_head: oracle columns up to {c0 + step}")
    assert np.array_equal(amc, np.argmax(yc, axis=1).astype(np.int32))
    assert np.array_equal(tkc, amc)
    oref = oracle.argmax_ref(ref)
    near = 0
    for r_ in range(M):
        if amc[r_] != oref[r_]:
            i, j = int(oref[r_]), int(amc[r_])
            margin = ref[r_, i] - ref[r_, j]
            assert margin <= 2 * max(err[r_, i], err[r_, j]), f"row {r_}: argmax {j} vs oracle {i}, margin {margin}"
            near += 1
    note(f"lm_head: argmax equal to the oracle's on {M - near} of {M} rows ({near} near-tie)")
    assert near <= 1


# ---------------------------------------------------------------- affine GEMM

AF_SHAPES = [(1, 5120, 15360), (16, 5120, 15360), (2, 64, 16), (16, 128, 32), (5, 704, 48), (16, 4096, 272),
             (1, 192, 1024), (16, 65536, 1024), (1, 65536, 1024)]


@pytest.mark.parametrize("M,K,N", AF_SHAPES)
def test_qgemm_affine_parity(M, K, N):
    m = q4()
    note(f"affine M={M} K={K} N={N}")
    inp = synth.affine_gemm(2000 + M + K + N, M, K, N)
    w = dev(m.q4_affine4_repack(inp.codes, inp.scale, inp.bias))
    a = dev(inp.a.view(np.int16)).view(torch.bfloat16)
    y = m.qgemm_affine4(w, a, N)
    torch.cuda.synchronize()
    ref, bnd = oracle.affine_gemm_ref(inp.codes, inp.scale, inp.bias, inp.a)
    check_gemm(y, ref, bnd, f"affine {M}x{K}x{N}")


@pytest.mark.parametrize("cfg", CFGS)
def test_qgemm_affine_every_config(cfg, monkeypatch):
    m = q4()
    monkeypatch.setenv("Q4MI_GEMM_CFG", cfg)
    for (M, K, N) in [(16, 1344, 400), (3, 704, 96), (1, 64, 48)]:
        inp = synth.affine_gemm(99 + K + N, M, K, N)
        w = dev(m.q4_affine4_repack(inp.codes, inp.scale, inp.bias))
        a = dev(inp.a.view(np.int16)).view(torch.bfloat16)
        for dt in (torch.float32, torch.bfloat16):
            y = m.qgemm_affine4(w, a, N, out_dtype=dt)
            torch.cuda.synchronize()
            ref, bnd = oracle.affine_gemm_ref(inp.codes, inp.scale, inp.bias, inp.a)
            if dt == torch.bfloat16:
                bnd = bnd + np.abs(ref) * 2.0 ** -8 / REL  # bf16 output rounding on top
            check_gemm(y, ref, bnd, f"cfg {cfg} {M}x{K}x{N} {dt}")
