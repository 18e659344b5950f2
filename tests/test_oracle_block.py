"""Pins of the MoE-block oracle (oracle/block.py) to things other than itself."""
import numpy as np

import oracle
import synth


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
    for s in range(20):
        dv = B * rng.choice([-1.0, 1.0], size=B.shape) * rng.uniform(0, 1, B.shape)
        assert np.all(np.abs(oracle.rmsnorm(v + dv, w) - y) <= bnd * 1.01 + 1e-15)


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
