"""GPU parity of moe_route_grouped_qgemm (the router writes partial logits;
the gate/up launch sums them and takes the top-k itself) against the two-call
path (moe_route_topk, then moe_grouped_qgemm) and the oracle.

Bars: logits bit-exact to moe_route_topk's (the same partial sums added in
the same order); indices bit-exact to moe_route_topk's (an exact top-k of the
same bits, ties to the lower index), so also to the oracle's except on its
near-ties; weights within 1e-6 of moe_route_topk's (the softmax sums are
added in another order); y within oracle.moe_abs_bound at the GPU's routing
and within 1e-5 relative L2 of the two-call path's y; repeated calls bitwise
identical."""
import sys

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


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


_CACHE = {}


def layer(seed, **kw):
    key = (seed, tuple(sorted(kw.items())))
    if key not in _CACHE:
        moe = synth.moe_layer(seed, **kw)
        _CACHE.clear()
        _CACHE[key] = (moe, q4().moe_pack_experts(moe.gate, moe.up, moe.down, moe.E, moe.has_shared))
    return _CACHE[key]


def check_routed(moe, mw, k, renormalize=False, wr=None, what=""):
    m = q4()
    wr = moe.w_router if wr is None else wr
    x, wrd = dev(moe.x), dev(wr)
    note(f"routed {what}: T={moe.T} D={moe.D} E={moe.E} F={moe.F} k={k} shared={moe.has_shared}")
    y, lg, idx, w = m.moe_route_grouped_qgemm(mw, x, wrd, k, renormalize=renormalize, want_logits=True)
    lg2, idx2, w2 = m.moe_route_topk(x, wrd, k, renormalize=renormalize)
    y2 = m.moe_grouped_qgemm(mw, x, idx2, w2)
    ya, _, idxa, wa = m.moe_route_grouped_qgemm(mw, x, wrd, k, renormalize=renormalize)
    torch.cuda.synchronize()
    lg, lg2 = lg.cpu().numpy(), lg2.cpu().numpy()
    ig, ig2 = idx.cpu().numpy(), idx2.cpu().numpy()
    wg, wg2 = w.cpu().numpy(), w2.cpu().numpy()
    assert np.array_equal(lg.view(np.uint32), lg2.view(np.uint32)), f"{what}: logits differ from the router's"
    assert np.array_equal(ig, ig2), f"{what}: indices differ from the router's"
    assert np.max(np.abs(wg.astype(np.float64) - wg2)) <= 1e-6, f"{what}: weights differ from the router's"
    yg = y.cpu().numpy().astype(np.float64)
    assert np.array_equal(yg, ya.cpu().numpy().astype(np.float64)), f"{what}: repeated call differs"
    assert np.array_equal(ig, idxa.cpu().numpy()) and np.array_equal(wg, wa.cpu().numpy())
    # the oracle's routing (near-ties aside) and the layer at the GPU's routing
    _, iref, wref = oracle.route_topk(moe.x, wr, k, renormalize=renormalize)
    same = np.all(ig == iref, axis=1)
    assert np.max(np.abs(wg[same].astype(np.float64) - wref[same]), initial=0.0) <= 1e-6
    if not np.all(same):
        note(f"routed {what}: {int((~same).sum())} token(s) route differently from the oracle (near-ties)")
    w64 = wg.astype(np.float64)
    ref, _ = oracle.moe_ref_grouped(moe, ig, w64)
    bnd = oracle.moe_abs_bound(moe, ig, w64)
    err = np.abs(yg - ref)
    assert np.all(np.isfinite(yg)) and np.all(err <= bnd), f"{what}: worst err/bound {np.max(err / bnd):.3e}"
    y2g = y2.cpu().numpy().astype(np.float64)
    nrm = np.maximum(np.linalg.norm(y2g, axis=1), 1e-30)
    rel = np.linalg.norm(yg - y2g, axis=1) / nrm
    note(f"routed {what}: worst err/bound {np.max(err / bnd):.3e}; vs two calls {rel.max():.2e}")
    assert np.all(rel <= 1e-5), f"{what}: relative L2 vs the two-call path {rel.max():.3e}"
    return ig, wg


def test_routed_gemma_layer():
    moe, mw = layer(104)
    check_routed(moe, mw, moe.k, what="gemma T=16 E=128+1 top-8")
    check_routed(moe, mw, moe.k, renormalize=True, what="renormalized")


@pytest.mark.parametrize("T,D,E,F,k,shared", [(7, 256, 32, 128, 4, True), (3, 192, 64, 64, 8, False),
                                               (4, 128, 256, 64, 8, True), (16, 128, 200, 64, 16, False),
                                               (1, 64, 4, 64, 1, True), (5, 128, 30, 64, 3, True),
                                               (16, 512, 128, 128, 8, True)])
def test_routed_shapes(T, D, E, F, k, shared):
    # E = 30 (not a multiple of 4) takes the router's own top-k
    moe, mw = layer(1300 + T + D + E + F + k, T=T, D=D, E=E, F=F, k=k, has_shared=shared)
    check_routed(moe, mw, k, what=f"T={T} E={E} k={k}")


def test_routed_zero_router_and_ties():
    moe, mw = layer(1500, T=4, D=256, E=128, F=64, k=8, has_shared=True)
    m = q4()
    _, _, idx, w = m.moe_route_grouped_qgemm(mw, dev(moe.x), dev(np.zeros((256, 128), np.float32)), 8)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(8, dtype=np.int32), (4, 1)))
    assert np.all(w.cpu().numpy() == np.float32(1.0 / 128))
    wr = (np.random.default_rng(1).standard_normal((256, 128)) * 0.02).astype(np.float32)
    wr[:, 3] = 0.05               # duplicate columns with the largest logits ->
    wr[:, 100] = 0.05             # bitwise-equal logits at the top
    moe_p = synth.moe_layer(1500, T=4, D=256, E=128, F=64, k=8, has_shared=True)
    moe_p.x = np.abs(moe_p.x)
    ig, _ = check_routed(moe_p, mw, 8, wr=wr, what="tied top")
    assert np.all(ig[:, 0] == 3) and np.all(ig[:, 1] == 100)   # lower index first


def test_routed_workspace_and_refusals():
    m = q4()
    moe, mw = layer(1501, T=2, D=64, E=8, F=64, k=2, has_shared=False)
    d = mw.desc()
    import ctypes as C
    need = m.raw().moe_route_grouped_workspace_bytes(C.byref(d), 2, 2)
    assert need >= m.raw().moe_workspace_bytes(C.byref(d), 2, 2) > 0
    x = dev(moe.x)
    wr = dev(moe.w_router)
    small = torch.zeros(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(m.Q4Error):
        m.moe_route_grouped_qgemm(mw, x, wr, 2, ws=small)
    with pytest.raises(m.Q4Error):
        m.moe_route_grouped_qgemm(mw, x, wr, 9)       # k > E
