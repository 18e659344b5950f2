"""GPU parity of the whole Gemma-4 MoE block (moe_block_forward) against the oracle.

Every token is checked, at the routing the device chose (moe_block_forward
returns it):

* router: the device's experts are a valid top-k of the oracle's scores z
  within their rigorous error (oracle.route_normed_bound: the f16 h2 and the
  fp32 sums), in decreasing device order, distinct; its weights within
  oracle.routing_weight_bound of softmax(z)[idx] * down_scale[idx];
* output against the oracle evaluated at that routing:
  - the W4A16 oracle (every activation that enters a 4-bit GEMM rounded to
    f16, as the pages' W4A16 fixes): relative L2 of the update per token
    <= 2e-4.  What remains between the two is fp32 accumulation and the
    elements whose fp32 value (the device's norms are a few ulps from the
    exact ones) and float64 value round to different f16 neighbours: each
    such h1/h2 element moves the update by about 2^-10 / sqrt(D), a few of
    them per token (9e-5 measured at the full shape).  The f16 roundings
    themselves move the update by ~4e-4, so a device that skipped or
    misplaced them fails;
  - the exact float64 oracle: relative L2 <= 2 x (the A16 roundings' own
    effect, as the oracle measures it) + 1e-4;
  - elementwise within oracle.moe_block_bound, the per-GEMM 1e-3 sum|a w|
    criterion composed rigorously through the FFNs and norms.  That
    composition is infinite where the criterion lets a branch's error reach
    its own size (every row of the full shape): there the contract alone
    constrains nothing and the two checks above carry the verdict.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TIGHT_REL_L2 = 2e-4


def q4():
    import moe_w4a16_skinny_amd as m
    return m


def note(*a):
    print(*a, flush=True)


def run_block(blk, eps=1e-6):
    m = q4()
    bw = m.moe_block_pack(blk, eps=eps)
    res = torch.from_numpy(np.ascontiguousarray(blk.residual)).cuda()
    _, idx, w = m.moe_block_forward(bw, res, blk.k, want_routing=True)
    torch.cuda.synchronize()
    return (res.cpu().numpy().astype(np.float64), idx.cpu().numpy(), w.cpu().numpy().astype(np.float64))


def check_router(blk, parts, idx, w, what):
    z = parts["z"]
    zb = oracle.route_normed_bound(blk, parts["h2"])
    T, E = z.shape
    k = blk.k
    assert idx.shape == (T, k) and np.all((idx >= 0) & (idx < E)), what
    ntie = 0
    for t in range(T):
        sel = idx[t]
        assert len(set(sel.tolist())) == k, f"{what}: token {t} names an expert twice"
        rest = np.setdiff1d(np.arange(E), sel)
        lo = np.min(z[t, sel] + zb[t, sel])          # the weakest chosen expert, at its best
        if rest.size:
            hi = np.max(z[t, rest] - zb[t, rest])    # the strongest unchosen one, at its worst
            assert lo >= hi, f"{what}: token {t}: expert set not a top-{k} within the score error"
        # decreasing device order: consecutive picks may only swap within their errors
        zs = z[t, sel]
        assert np.all(zs[:-1] + zb[t, sel[:-1]] >= zs[1:] - zb[t, sel[1:]]), f"{what}: token {t} order"
        ntie += int(not np.array_equal(sel, parts["idx"][t]))
    wb = oracle.routing_weight_bound(z, zb, idx, blk.down_scale)
    p = oracle.softmax(z)
    ds = np.ones(E) if blk.down_scale is None else np.asarray(blk.down_scale, np.float64)
    wref = np.take_along_axis(p, idx.astype(np.int64), axis=1) * ds[idx]
    assert np.all(np.abs(w - wref) <= wb), f"{what}: routing weights outside their bound"
    if ntie:
        note(f"{what}: {ntie} token(s) routed differently from the oracle, within the score error")


def check_block(blk, what):
    note(f"{what}: device")
    out, idx, w = run_block(blk)
    assert np.all(np.isfinite(out)), what
    note(f"{what}: oracle at the device's routing")
    ref, parts = oracle.moe_block_ref(blk, blk.residual, want_parts=True)
    check_router(blk, parts, idx, w, what)
    at = (idx, w)
    ref_d, parts_d = oracle.moe_block_ref(blk, blk.residual, want_parts=True, routing=at)
    ref16 = oracle.moe_block_ref(blk, blk.residual, routing=at, a16_inputs=True)
    res = np.asarray(blk.residual, np.float64)
    c_gpu, c_ref, c16 = out - res, ref_d - res, ref16 - res
    nrm = np.linalg.norm(c_ref, axis=1)
    tight = np.linalg.norm(c_gpu - c16, axis=1) / nrm
    a16_effect = np.linalg.norm(c16 - c_ref, axis=1) / nrm
    exact = np.linalg.norm(c_gpu - c_ref, axis=1) / nrm
    note(f"{what}: update vs W4A16 oracle {tight.max():.2e}, vs exact {exact.max():.2e} "
         f"(A16 roundings alone {a16_effect.max():.2e})")
    assert np.all(tight <= TIGHT_REL_L2), f"{what}: relative L2 vs the W4A16 oracle {tight.max():.3e}"
    assert np.all(exact <= 2 * a16_effect + 1e-4), f"{what}: relative L2 vs the exact oracle {exact.max():.3e}"
    note(f"{what}: composed contract bound")
    bnd = oracle.moe_block_bound(blk, blk.residual, parts_d)
    err = np.abs(out - ref_d)
    assert np.all(err <= bnd), f"{what}: worst err/bound {np.max(err / bnd):.3e}"
    fin = np.isfinite(bnd).all(axis=1)
    note(f"{what}: {int(fin.sum())} of {len(fin)} token(s) with a finite contract bound")
    return out


# the experts and the dense branch share each grouped launch, the grid split
# by their tile-items: the last two shapes put the split at its extremes (a
# dense branch 32x the routed work; a dense branch of one 64-wide tile, which
# gets a single workgroup), with K = F of one half tile in down
@pytest.mark.parametrize("T,D,E,F,Fd,k", [(4, 256, 8, 128, 192, 2), (1, 512, 16, 64, 64, 4), (7, 1024, 32, 256, 320, 8),
                                          (16, 2816, 128, 704, 2112, 8), (1, 1024, 2, 64, 2048, 1),
                                          (16, 512, 64, 256, 64, 8)])
def test_block_parity(T, D, E, F, Fd, k):
    note(f"block T={T} D={D} E={E} F={F} Fd={Fd} k={k}")
    blk = synth.moe_block(900 + T + E, T=T, D=D, E=E, F=F, F_dense=Fd, k=k)
    check_block(blk, f"T={T} D={D} E={E}")


def test_block_without_down_scale_and_repeat():
    m = q4()
    blk = synth.moe_block(77, T=5, D=256, E=16, F=64, F_dense=128, k=4)
    blk.down_scale = None
    bw = m.moe_block_pack(blk)
    outs = []
    for _ in range(2):
        res = torch.from_numpy(np.ascontiguousarray(blk.residual)).cuda()
        m.moe_block_forward(bw, res, blk.k)
        torch.cuda.synchronize()
        outs.append(res.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]), "two runs differ"
    blk.down_scale = np.ones(16, np.float32)
    out = check_block(blk, "no down scale")
    assert np.array_equal(out, outs[0].astype(np.float64))


def test_block_silent_experts_is_the_dense_branch():
    # down_scale = 0: the MoE branch adds nothing, the update is the normed dense branch
    blk = synth.moe_block(78, T=3, D=512, E=8, F=128, F_dense=256, k=2)
    blk.down_scale = np.zeros(8, np.float32)
    check_block(blk, "silent experts")


def test_block_refusals():
    m = q4()
    blk = synth.moe_block(79, T=2, D=256, E=8, F=64, F_dense=64, k=2)
    bw = m.moe_block_pack(blk)
    res = torch.from_numpy(np.ascontiguousarray(blk.residual)).cuda()
    before = res.clone()
    with pytest.raises(m.Q4Error):
        m.moe_block_forward(m.MoeBlockWeights(bw.experts, bw.dense, bw.w_router, bw.router_scale, bw.down_scale,
                                              bw.norms, eps=0.0), res, 2)
    with pytest.raises(m.Q4Error):
        m.moe_block_forward(bw, res, 17)      # k beyond the router's 16
    with pytest.raises(m.Q4Error):
        m.moe_block_forward(bw, res, 9)       # k beyond E
    big = torch.zeros((17, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(m.Q4Error):
        m.moe_block_forward(bw, big, 2)       # T beyond 16
    with pytest.raises(ValueError):
        m.moe_block_forward(bw, res.double(), 2)
    torch.cuda.synchronize()
    assert torch.equal(res, before), "a refused call changed the residual"


def test_block_scratch_needs_no_zero_fill():
    # Only the workspace's first 32 KiB (counters) must start at zero; the
    # scratch above them may hold anything (here: NaN bit patterns and junk
    # left from other calls), and the result is the same as on a zeroed one.
    import ctypes as C
    m = q4()
    blk = synth.moe_block(81, T=6, D=512, E=16, F=128, F_dense=192, k=4)
    bw = m.moe_block_pack(blk)
    d = bw.desc()
    lib = m.raw()
    T, k = blk.T, blk.k
    wsb = lib.moe_block_workspace_bytes(C.byref(d), T, k)
    outs = []
    for fill in (0, 0xFF, 0x7F):
        ws = torch.full((wsb,), fill, dtype=torch.uint8, device="cuda")
        ws[:32768].zero_()
        res = torch.from_numpy(np.ascontiguousarray(blk.residual)).cuda()
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        vp = C.c_void_p
        rc = lib.moe_block_forward(C.byref(d), vp(res.data_ptr()), T, k, vp(idx.data_ptr()), vp(w.data_ptr()),
                                   vp(ws.data_ptr()), C.c_size_t(wsb), vp(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, lib.q4_last_error().decode() if hasattr(lib, "q4_last_error") else rc
        torch.cuda.synchronize()
        assert torch.count_nonzero(ws[:32768]).item() == 0, "counters not left at zero"
        outs.append((res.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b), "result depends on the scratch's prior contents"
