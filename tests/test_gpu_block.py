"""GPU parity of the whole Gemma-4 MoE block (moe_block_forward) against the oracle.

Bars: every output element within the composed first-order bound
(oracle.moe_block_bound: the per-GEMM 1e-3 * sum|a w| carried through the
gated FFNs, the post-norms, the sum and the final norm); the update added to
the residual within 5e-3 relative (L2 per token; the f16 inputs of the
GEMMs, 2^-11 relative, dominate the real error).  A token whose k-th and
(k+1)-th normalized router scores are closer than the bound of those scores
may pick another expert on the GPU: it is only checked for finiteness and
reported."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

REL_L2 = 5e-3


def q4():
    import moe_w4a16_skinny_amd as m
    return m


def note(*a):
    print(*a, flush=True)


def near_tie_tokens(blk, parts):
    """tokens whose top-k boundary is within the error of the normalized scores"""
    h2 = parts["h2"]
    logits = h2 @ np.asarray(blk.w_router, np.float64)
    r = 1.0 / np.sqrt(np.mean(logits * logits, axis=1, keepdims=True) + 1e-6)
    zb = (2.0 ** -10 * (np.abs(h2) @ np.abs(np.asarray(blk.w_router, np.float64))) + 1e-6 * np.abs(logits)) \
        * r * np.abs(blk.router_scale)
    z = parts["z"]
    srt = -np.sort(-z, axis=1)
    k = blk.k
    gap = srt[:, k - 1] - srt[:, k] if k < z.shape[1] else np.full(z.shape[0], np.inf)
    return gap <= 2 * zb.max(axis=1) + 1e-7


def run_block(blk, eps=1e-6):
    m = q4()
    bw = m.moe_block_pack(blk, eps=eps)
    res = torch.from_numpy(np.ascontiguousarray(blk.residual)).cuda()
    m.moe_block_forward(bw, res, blk.k)
    torch.cuda.synchronize()
    return res.cpu().numpy().astype(np.float64), bw


def check_block(blk, what):
    out, _ = run_block(blk)
    ref, parts = oracle.moe_block_ref(blk, blk.residual, want_parts=True)
    bnd = oracle.moe_block_bound(blk, blk.residual, parts)
    assert np.all(np.isfinite(out)), what
    tie = near_tie_tokens(blk, parts)
    ok = ~tie
    if tie.any():
        note(f"{what}: {int(tie.sum())} token(s) with a near-tie at the top-k boundary, checked for finiteness only")
    err = np.abs(out - ref)
    assert np.all(err[ok] <= bnd[ok]), f"{what}: worst err/bound {np.max(err[ok] / bnd[ok]):.3e}"
    c_gpu = out - np.asarray(blk.residual, np.float64)
    c_ref = parts["c"]
    rel = np.linalg.norm(c_gpu - c_ref, axis=1) / np.linalg.norm(c_ref, axis=1)
    assert np.all(rel[ok] <= REL_L2), f"{what}: relative L2 error of the update {rel.max():.3e}"
    note(f"{what}: max relative L2 error of the update {rel[ok].max():.2e}")
    return out


@pytest.mark.parametrize("T,D,E,F,Fd,k", [(4, 256, 8, 128, 192, 2), (1, 512, 16, 64, 64, 4), (7, 1024, 32, 256, 320, 8),
                                          (16, 2816, 128, 704, 2112, 8)])
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
    ref, parts = oracle.moe_block_ref(blk, blk.residual, want_parts=True)
    bnd = oracle.moe_block_bound(blk, blk.residual, parts)
    ok = ~near_tie_tokens(blk, parts)
    assert np.all(np.abs(outs[0] - ref)[ok] <= bnd[ok])


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
    with pytest.raises(m.Q4Error):
        m.moe_block_forward(m.MoeBlockWeights(bw.experts, bw.dense, bw.w_router, bw.router_scale, bw.down_scale,
                                              bw.norms, eps=0.0), res, 2)
    with pytest.raises(m.Q4Error):
        m.moe_block_forward(bw, res, 17)      # k beyond the router's 16
    big = torch.zeros((17, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(m.Q4Error):
        m.moe_block_forward(bw, big, 2)       # T beyond 16
    with pytest.raises(ValueError):
        m.moe_block_forward(bw, res.double(), 2)
