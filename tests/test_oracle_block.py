"""Pins of the MoE-block oracle (oracle/block.py) to things other than itself."""
import numpy as np
import pytest

import oracle
import synth
from perturb import perturbed_block


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(0)
    v = rng.standard_normal((5, 64))
    # unit weights, no eps: every row has root mean square 1
    y = oracle.rmsnorm(v, None, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    # scale invariance (eps = 0) and sign
    assert np.allclose(oracle.rmsnorm(3.5 * v, None, eps=0.0), y, rtol=1e-14)
    assert np.allclose(oracle.rmsnorm(-v, None, eps=0.0), -y, rtol=1e-14)
    # a constant row c: c / sqrt(c^2 + eps) times the weights
    w = rng.standard_normal(64)
    c = 0.25
    got = oracle.rmsnorm(np.full((1, 64), c), w, eps=1e-6)
    assert np.allclose(got, c / np.sqrt(c * c + 1e-6) * w, rtol=1e-14)
    # eps keeps a zero row at zero
    assert np.all(oracle.rmsnorm(np.zeros((1, 8)), np.ones(8)) == 0)


def test_rmsnorm_bound_dominates_perturbations():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((4, 128))
    w = 1 + 0.1 * rng.standard_normal(128)
    B = 1e-4 * np.abs(rng.standard_normal((4, 128)))
    bnd = oracle.rmsnorm_bound(v, w, B)
    y = oracle.rmsnorm(v, w)
    worst = 0.0
    for s in range(20):
        dv = B * rng.choice([-1.0, 1.0], size=B.shape) * rng.uniform(0, 1, B.shape)
        dev = np.abs(oracle.rmsnorm(v + dv, w) - y)
        assert np.all(dev <= bnd)
        worst = max(worst, float(np.max(dev / bnd)))
    # the largest permitted change of one element: dv = +-B everywhere, signed with v there
    for i in range(3):
        dv = B * np.where(np.arange(128) == i, 1.0, -np.sign(v) * np.sign(v[:, i:i + 1]))
        dev = np.abs(oracle.rmsnorm(v + dv, w) - y)
        assert np.all(dev <= bnd)
        worst = max(worst, float(np.max(dev[:, i] / bnd[:, i])))
    assert worst > 0.5
    # a perturbation as large as the row itself: no finite bound
    assert np.all(np.isinf(oracle.rmsnorm_bound(v, w, 2 * np.abs(v))))


def test_router_normalization_is_scale_invariant():
    # the unweighted RMSNorm of the logits makes routing independent of the
    # scale of W_r (eps negligible); the learned scale then changes it
    blk = synth.moe_block(5, T=6, D=128, E=16, F=64, F_dense=64, k=4)
    h2 = oracle.rmsnorm(blk.residual, blk.pre_ffw_norm_2)
    z1, i1, w1 = oracle.route_normed(h2, blk.w_router, blk.router_scale, blk.down_scale, 4, eps=0.0)
    z2, i2, w2 = oracle.route_normed(h2, blk.w_router * 7.0, blk.router_scale, blk.down_scale, 4, eps=0.0)
    assert np.array_equal(i1, i2) and np.allclose(w1, w2, rtol=1e-12)
    # unit scales: the routing weights are the softmax of the normalized
    # logits, which have root mean square 1 per token
    z, idx, w = oracle.route_normed(h2, blk.w_router, np.ones(16), np.ones(16), 16, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(z * z, axis=1)), 1.0)
    assert np.allclose(w.sum(axis=1), 1.0)
    assert np.all(np.diff(np.take_along_axis(z, idx, axis=1), axis=1) <= 0)
    # the down scale multiplies each kept expert's weight
    _, idx3, w3 = oracle.route_normed(h2, blk.w_router, blk.router_scale, 2 * blk.down_scale, 4, eps=0.0)
    assert np.array_equal(idx3, i1) and np.allclose(w3, 2 * w1)


def test_block_reduces_to_the_dense_branch_without_experts():
    # down_scale = 0 silences the MoE branch: the block adds
    # RMSNorm(RMSNorm(b1; post1); post) with b1 the dense FFN of RMSNorm(res; ffn_norm)
    blk = synth.moe_block(6, T=3, D=128, E=8, F=64, F_dense=128, k=2)
    blk.down_scale = np.zeros(8, np.float32)
    out, parts = oracle.moe_block_ref(blk, blk.residual, want_parts=True)
    assert np.all(parts["b2"] == 0) and np.all(parts["b2n"] == 0)
    # the dense FFN written out by hand from the dequantized matrices
    wg = oracle.nvfp4_dequant(*blk.dense_gate)
    wu = oracle.nvfp4_dequant(*blk.dense_up)
    wd = oracle.nvfp4_dequant(*blk.dense_down)
    h1 = parts["h1"]
    b1 = (oracle.gelu_tanh(h1 @ wg.T) * (h1 @ wu.T)) @ wd.T
    assert np.allclose(parts["b1"], b1, rtol=1e-12, atol=1e-14)
    r1 = np.sqrt(np.mean(b1 * b1, axis=1, keepdims=True) + 1e-6)
    s = b1 / r1 * blk.post_ffw_norm_1
    r = np.sqrt(np.mean(s * s, axis=1, keepdims=True) + 1e-6)
    assert np.allclose(out - blk.residual, s / r * blk.post_ffw_norm, rtol=1e-12, atol=1e-14)


def test_block_output_is_residual_plus_unit_rms_update():
    # with unit post-norm weights the update added to the residual has root
    # mean square sqrt(m / (m + eps)) ~ 1 per token
    blk = synth.moe_block(7, T=4, D=128, E=8, F=64, F_dense=64, k=2)
    blk.post_ffw_norm = np.ones(128, np.float32)
    out = oracle.moe_block_ref(blk, blk.residual)
    c = out - blk.residual
    assert np.allclose(np.sqrt(np.mean(c * c, axis=1)), 1.0, atol=1e-4)


@pytest.mark.parametrize("T,D,E,F,Fd,k", [(3, 128, 8, 64, 64, 2), (2, 256, 6, 64, 128, 3)])
def test_block_bound_dominates_contract_limit_errors(T, D, E, F, Fd, k):
    blk = synth.moe_block(60 + D, T=T, D=D, E=E, F=F, F_dense=Fd, k=k)
    rng = np.random.default_rng(D)
    worst = 0.0
    for target in (None, None, 3, 17, D - 1):
        out, ref, parts = perturbed_block(blk, rng, target=target)
        bnd = oracle.moe_block_bound(blk, blk.residual, parts)
        assert np.all(np.isfinite(bnd))
        dev = np.abs(out - ref)
        assert np.all(dev <= bnd), f"dev/bound {np.max(dev / bnd):.3f}"
        worst = max(worst, float(np.max(dev / bnd)))
    assert worst >= 1 / 20, f"bound {1 / worst:.1f}x the largest deviation"


def test_block_bound_fails_without_the_h_error_term(monkeypatch):
    blk = synth.moe_block(64, T=3, D=128, E=8, F=64, F_dense=64, k=2)
    rng = np.random.default_rng(5)
    out, ref, parts = perturbed_block(blk, rng, target=7)
    full = oracle.moe_block_bound(blk, blk.residual, parts)

    def h_error_rounding_only(g, u, rg, ru, act_rel):
        return (act_rel + oracle.moe.F16_REL) * np.abs(oracle.gelu_tanh(g) * u) + oracle.moe.F16_ABS

    monkeypatch.setattr(oracle.moe, "_h_error", h_error_rounding_only)
    cut = oracle.moe_block_bound(blk, blk.residual, parts)
    assert np.all(cut < full)
    assert np.any(np.abs(out - ref) > cut)


def test_block_at_a_given_routing():
    # evaluated at its own routing the block is unchanged; at another one the
    # expert branch follows that routing and the dense branch does not move
    blk = synth.moe_block(65, T=3, D=128, E=8, F=64, F_dense=64, k=2)
    out, parts = oracle.moe_block_ref(blk, blk.residual, want_parts=True)
    same, p2 = oracle.moe_block_ref(blk, blk.residual, want_parts=True, routing=(parts["idx"], parts["w"]))
    assert np.array_equal(out, same)
    idx = parts["idx"][:, ::-1].copy()
    w = parts["w"][:, ::-1].copy() * 0.5
    _, p3 = oracle.moe_block_ref(blk, blk.residual, want_parts=True, routing=(idx, w))
    assert np.array_equal(p3["b1"], parts["b1"]) and np.array_equal(p3["idx"], idx)
    assert np.allclose(p3["b2"], 0.5 * parts["b2"], rtol=1e-12, atol=1e-15)


def test_router_score_bound_dominates_f16_inputs_and_fp32_sums():
    # the device's scores come from the f16 h2 and fp32 accumulation: z from
    # h2 rounded to f16 (and its neighbours one f16 step away), with fp32
    # products summed in fp32 four at a time, must lie within route_normed_bound
    blk = synth.moe_block(66, T=4, D=512, E=16, F=64, F_dense=64, k=4)
    res = np.asarray(blk.residual, np.float64)
    h2 = oracle.rmsnorm(res, blk.pre_ffw_norm_2)
    z, _, _ = oracle.route_normed(h2, blk.w_router, blk.router_scale, blk.down_scale, 4)
    zb = oracle.route_normed_bound(blk, h2)
    wr32 = np.asarray(blk.w_router, np.float32)
    rng = np.random.default_rng(2)
    for trial in range(3):
        h16 = h2.astype(np.float16)
        if trial:
            up = np.nextafter(h16, np.float16(np.inf) * np.sign(rng.standard_normal(h16.shape)).astype(np.float16))
            h16 = np.where(rng.uniform(size=h16.shape) < 0.5, up, h16)
        acc = np.zeros((4, 16), np.float32)
        for d0 in range(0, 512, 4):
            acc = (acc + (h16[:, d0:d0 + 4].astype(np.float32) @ wr32[d0:d0 + 4])).astype(np.float32)
        zd = oracle.rmsnorm(acc.astype(np.float64), blk.router_scale)
        assert np.all(np.abs(zd - z) <= zb)


def test_a16_block_within_the_rounding_only_bound():
    # rounding h1, h2 and h to f16 at a fixed routing moves the block by at
    # most the bound with no GEMM error (gemm_rel = 0) and exact norms
    blk = synth.moe_block(67, T=3, D=128, E=8, F=64, F_dense=64, k=2)
    out, parts = oracle.moe_block_ref(blk, blk.residual, want_parts=True)
    o16 = oracle.moe_block_ref(blk, blk.residual, routing=(parts["idx"], parts["w"]), a16_inputs=True)
    bnd = oracle.moe_block_bound(blk, blk.residual, parts, gemm_rel=0.0, f32_rel=0.0)
    assert np.all(np.isfinite(bnd)) and np.all(np.abs(o16 - out) <= bnd) and np.max(np.abs(o16 - out)) > 0
