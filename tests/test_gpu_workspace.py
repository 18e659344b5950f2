"""Regression: entry points of different kinds and shapes share one workspace
in stream order (router partials, split-K partials of several block counts,
MoE scratch, argmax keys); every call must still match the oracle, which
requires every call to leave the counter region at zero."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def test_shared_workspace_interleaved_calls():
    import moe_w4a16_skinny_amd as q4
    q4.workspace(64 << 20)  # one buffer, large enough for every call below: no regrowth
    moe = synth.moe_layer(31, T=8, D=512, E=16, F=192, k=4, has_shared=True)
    mw = q4.moe_pack_experts(moe.gate, moe.up, moe.down, moe.E, moe.has_shared)
    _, iref, wref = oracle.route_topk(moe.x, moe.w_router, moe.k)

    aff = synth.affine_gemm(32, 1, 5120, 15360)
    waff = dev(q4.q4_affine4_repack(aff.codes, aff.scale, aff.bias))
    aaff = dev(aff.a.view(np.int16)).view(torch.bfloat16)
    ref_aff, bnd_aff = oracle.affine_gemm_ref(aff.codes, aff.scale, aff.bias, aff.a)

    # K % 64 != 0: activations staged in LDS, K split over two workgroups per block
    nv = synth.nvfp4_gemm(33, 16, 5136, 1024)
    assert q4.raw().qgemm_nvfp4_workspace_bytes(16, 5136, 1024, 1) > 32768
    wnv = dev(q4.q4_nvfp4_repack(nv.codes, nv.scales))
    ref_nv, bnd_nv = oracle.nvfp4_gemm_ref(nv.codes, nv.scales, nv.g, nv.a)

    for rep in range(2):
        _, idx, w = q4.moe_route_topk(dev(moe.x), dev(moe.w_router), moe.k)
        y_aff = q4.qgemm_affine4(waff, aaff, 15360)
        y_nv, am = q4.qgemm_nvfp4(wnv, float(nv.g), dev(nv.a), 1024, want_argmax=True)
        y_moe = q4.moe_grouped_qgemm(mw, dev(moe.x), dev(iref), dev(wref.astype(np.float32)))
        y_aff2 = q4.qgemm_affine4(waff, aaff, 15360)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), iref)
        for y in (y_aff, y_aff2):
            assert np.all(np.abs(y.cpu().numpy() - ref_aff) <= 1e-3 * bnd_aff), f"affine after sharing (rep {rep})"
        ync = y_nv.cpu().numpy()
        assert np.all(np.abs(ync - ref_nv) <= 1e-3 * bnd_nv), f"nvfp4 after sharing (rep {rep})"
        assert np.array_equal(am.cpu().numpy(), np.argmax(ync, axis=1))
        w32 = wref.astype(np.float32).astype(np.float64)
        ref_m, _ = oracle.moe_ref_grouped(moe, iref, w32)
        assert np.all(np.abs(y_moe.cpu().numpy() - ref_m) <= oracle.moe_abs_bound(moe, iref, w32))
    # the counter region is back to zero
    ws = q4.workspace(0)
    assert int(torch.count_nonzero(ws[:32768])) == 0
