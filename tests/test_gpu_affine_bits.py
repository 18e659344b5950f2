"""GPU parity of the affine 2/3/5/6/8-bit GEMM (qgemm_affine_bits) against the
oracle: |err| <= 1e-3 * sum_k |a w| per element (plus the output rounding for
bf16)."""
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


def run(bits, M, K, N, seed, out_dtype=None):
    m = q4()
    q, s, b = synth.affine_weights_bits(seed, N, K, bits)
    a = synth.act_bf16_bits(seed + 1, M, K)
    w = dev(m.q4_affine_bits_repack(q, s, b, bits))
    y = m.qgemm_affine_bits(w, dev(a.view(np.int16)).view(torch.bfloat16), N, bits, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, bnd = oracle.affine_bits_gemm_ref(q, s, b, a, bits)
    return y.float().cpu().numpy().astype(np.float64), ref, bnd


@pytest.mark.parametrize("bits", [2, 3, 5, 6, 8])
@pytest.mark.parametrize("M,K,N", [(1, 64, 16), (3, 192, 48), (16, 128, 16), (7, 640, 272), (16, 5120, 1024),
                                   (16, 2816, 3088), (16, 65536, 512)])
def test_affine_bits_parity(bits, M, K, N):
    print(f"affine bits={bits} M={M} K={K} N={N}", flush=True)
    y, ref, bnd = run(bits, M, K, N, 300 + bits + M + K + N)
    assert np.all(np.isfinite(y))
    err = np.abs(y - ref)
    assert np.all(err <= REL * bnd), f"worst err/bound {np.max(err / np.maximum(bnd, 1e-300)):.3e}"


@pytest.mark.parametrize("bits", [2, 8])
def test_affine_bits_workload_size(bits):
    y, ref, bnd = run(bits, 16, 5120, 15360, 40 + bits)
    assert np.all(np.abs(y - ref) <= REL * bnd)


def test_affine_bits_bf16_output_and_extreme_codes():
    m = q4()
    M, K, N, bits = 5, 256, 32, 8
    q, s, b = synth.affine_weights_bits(61, N, K, bits)
    q[:, :64] = 255                      # top codes in the first group
    q[:, 64:128] = 0
    a = synth.act_bf16_bits(62, M, K)
    w = dev(m.q4_affine_bits_repack(q, s, b, bits))
    y = m.qgemm_affine_bits(w, dev(a.view(np.int16)).view(torch.bfloat16), N, bits, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, bnd = oracle.affine_bits_gemm_ref(q, s, b, a, bits)
    yy = y.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(yy - ref) <= REL * bnd + 2.0 ** -8 * np.abs(ref))


def test_affine_bits_refusals():
    m = q4()
    w = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    a = torch.zeros((17, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.Q4Error):
        m.qgemm_affine_bits(w, a, 16, 2)
    with pytest.raises(m.Q4Error):
        m.qgemm_affine_bits(w, a[:2], 16, 4)
