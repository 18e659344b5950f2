"""GPU parity of the NVFP4 GEMM for more than 16 activation rows (prefill
chunks, large verify blocks) against the oracle: |err| <= 1e-3 * sum_k |a w|
per element (plus the output rounding for bf16)."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

REL = 1e-3


def q4():
    import moe_w4a16_skinny_amd as m
    return m


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def note(*a):
    print(*a, flush=True)


def check(y_gpu, ref, bnd, what, extra_rel=0.0):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y)), what
    tol = REL * bnd + extra_rel * np.abs(ref)
    err = np.abs(y - ref)
    assert np.all(err <= tol), f"{what}: worst err/tol {np.max(err / np.maximum(tol, 1e-300)):.3e}"


SHAPES = [  # (M, K, N): one row past the skinny limit, ragged blocks in M and N, K tails and half tiles;
    # more than 8 row blocks (the workgroup order's bands of 8: 8 + 2, and 8 + 8 + 2 with a ragged last block)
    (17, 128, 16), (32, 80, 48), (100, 704, 272), (128, 4096, 256), (129, 64, 144), (257, 1024, 1040),
    (512, 2816, 512), (64, 4096, 8192), (300, 1088, 2000), (600, 512, 272), (1100, 320, 1040),
    (65536, 64, 16),  # the most rows the entry point takes: 1024 row blocks, 128 bands
]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_prefill_parity(M, K, N):
    m = q4()
    note(f"prefill M={M} K={K} N={N}")
    inp = synth.nvfp4_gemm(7000 + M + K + N, M, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    y = m.qgemm_nvfp4(w, float(inp.g), dev(inp.a), N)
    torch.cuda.synchronize()
    ref, bnd = oracle.nvfp4_gemm_ref(inp.codes, inp.scales, inp.g, inp.a)
    check(y, ref, bnd, f"{M}x{K}x{N}")


@pytest.mark.parametrize("out_dtype", ["f16", "bf16"])
def test_prefill_low_precision_outputs(out_dtype):
    m = q4()
    M, K, N = 200, 2816, 384
    inp = synth.nvfp4_gemm(71, M, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    dt = torch.float16 if out_dtype == "f16" else torch.bfloat16
    y = m.qgemm_nvfp4(w, float(inp.g), dev(inp.a), N, out_dtype=dt)
    torch.cuda.synchronize()
    assert y.dtype == dt
    ref, bnd = oracle.nvfp4_gemm_ref(inp.codes, inp.scales, inp.g, inp.a)
    check(y, ref, bnd, out_dtype, extra_rel=2.0 ** -11 if out_dtype == "f16" else 2.0 ** -8)


def test_prefill_rows_match_the_skinny_kernel_bound():
    # rows 0..15 of an M = 48 product and the same 16 rows through the
    # skinny kernel: both within the bound of the same oracle values
    m = q4()
    M, K, N = 48, 4096, 1024
    inp = synth.nvfp4_gemm(72, M, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    a = dev(inp.a)
    y = m.qgemm_nvfp4(w, float(inp.g), a, N)
    y16 = m.qgemm_nvfp4(w, float(inp.g), a[:16].contiguous(), N)
    torch.cuda.synchronize()
    ref, bnd = oracle.nvfp4_gemm_ref(inp.codes, inp.scales, inp.g, inp.a)
    check(y, ref, bnd, "M=48")
    check(y16, ref[:16], bnd[:16], "first 16 rows, skinny kernel")


def test_prefill_deterministic_and_special_inputs():
    m = q4()
    M, K, N = 160, 1024, 272
    inp = synth.nvfp4_gemm(73, M, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    a = inp.a.copy()
    a[5] = 0                     # a zero row
    a[77, :] = 0
    a[77, 100] = 1.0             # a unit row picks one column of W (times g)
    y1 = m.qgemm_nvfp4(w, float(inp.g), dev(a), N)
    y2 = m.qgemm_nvfp4(w, float(inp.g), dev(a), N)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y = y1.cpu().numpy()
    assert np.all(y[5] == 0)
    wd = oracle.nvfp4_dequant(inp.codes, inp.scales, inp.g)
    assert np.array_equal(y[77].astype(np.float64), wd[:, 100].astype(np.float32).astype(np.float64))
    ref, bnd = oracle.nvfp4_gemm_ref(inp.codes, inp.scales, inp.g, a)
    check(y1, ref, bnd, "special rows")


def test_prefill_workload_size():
    # the prefill workload: 512 rows x K 4096 x N 8192, every element
    m = q4()
    wl = synth.WORKLOADS["nvfp4_prefill_m512_k4096_n8192"]
    M, K, N = wl["M"], wl["K"], wl["N"]
    inp = synth.nvfp4_gemm(wl["seed"], M, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    y = m.qgemm_nvfp4(w, float(inp.g), dev(inp.a), N)
    torch.cuda.synchronize()
    ref, bnd = oracle.nvfp4_gemm_ref(inp.codes, inp.scales, inp.g, inp.a)
    check(y, ref, bnd, "prefill workload")


def test_prefill_workload_2048_rows():
    # the 2048-row prefill workload (four bands of 8 row blocks), every element
    m = q4()
    wl = synth.WORKLOADS["nvfp4_prefill_m2048_k4096_n8192"]
    M, K, N = wl["M"], wl["K"], wl["N"]
    note(f"prefill workload M={M} K={K} N={N}")
    inp = synth.nvfp4_gemm(wl["seed"], M, K, N)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    y = m.qgemm_nvfp4(w, float(inp.g), dev(inp.a), N)
    torch.cuda.synchronize()
    ref, bnd = oracle.nvfp4_gemm_ref(inp.codes, inp.scales, inp.g, inp.a)
    check(y, ref, bnd, "prefill 2048-row workload")


def test_prefill_refusals():
    m = q4()
    inp = synth.nvfp4_gemm(74, 17, 128, 32)
    w = dev(m.q4_nvfp4_repack(inp.codes, inp.scales))
    with pytest.raises(m.Q4Error):
        m.qgemm_nvfp4(w, float(inp.g), dev(inp.a), 32, want_argmax=True)
    with pytest.raises(m.Q4Error):
        m.qgemm_nvfp4_sample(w, float(inp.g), dev(inp.a), 32)
