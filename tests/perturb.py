"""Device errors at their contracts' limits, injected into float64 forward
passes of the expert layer and the block: the CPU pins of the composed
bounds (oracle.moe_abs_bound, oracle.moe_block_bound) check that these stay
within them."""
import numpy as np

import oracle


def perturbed_ffn(x, wg, wu, wd, we, sx, sg, su, sh, so, gemm_rel=1e-3, act_rel=1e-4, in_rel=0.0, in_abs=0.0):
    """we * FFN(x) of one token through one expert, every step moved by its
    limit with the given signs: the GEMM input by in_rel |x| + in_abs, each
    GEMM output by gemm_rel * sum|a w| of its own inputs, h by its fp32
    evaluation (act_rel) and its f16 store (2^-11 |h| + 2^-25)."""
    xt = x + sx * (in_rel * np.abs(x) + in_abs)
    gt = wg @ xt + sg * gemm_rel * (np.abs(wg) @ np.abs(xt))
    ut = wu @ xt + su * gemm_rel * (np.abs(wu) @ np.abs(xt))
    ht = oracle.gelu_tanh(gt) * ut
    ht = ht * (1 + sh * act_rel)
    hb = ht + sh * (oracle.moe.F16_REL * np.abs(ht) + oracle.moe.F16_ABS)
    return we * (wd @ hb + so * gemm_rel * (np.abs(wd) @ np.abs(hb)))


def perturbed_layer(moe, idx, w, rng, target=None, gemm_rel=1e-3, act_rel=1e-4, in_rel=0.0, in_abs=0.0, x=None,
                    direction=1.0):
    """The expert layer (x = moe.x unless given) in float64 with every device
    error at its contract's limit (perturbed_ffn per token and expert, then
    the combine's (k + 3) 2^-24 sum|w o|).  Signs are random, or, with
    target = n, aligned so that every FFN error pushes y[t][n] the same way
    (up for direction = 1, down for -1)."""
    x = np.asarray(moe.x if x is None else x, np.float64)
    T, D = x.shape
    k = idx.shape[1]
    y = np.zeros((T, D))
    for t in range(T):
        sel = [(int(idx[t, j]), float(w[t, j])) for j in range(k)]
        if moe.has_shared:
            sel.append((moe.E, 1.0))
        mag = np.zeros(D)
        sx = rng.choice([-1.0, 1.0], size=D)
        for e, we in sel:
            wg, wu, wd = oracle.moe._expert_mats(moe, e)
            g, u = wg @ x[t], wu @ x[t]
            if target is None:
                sg, su, sh, so = (rng.choice([-1.0, 1.0], size=n) for n in (len(g), len(g), len(g), D))
            else:
                dn = direction * we * wd[target]
                sg = np.sign(dn * oracle.gelu_tanh_deriv(g) * u)
                su = np.sign(dn * oracle.gelu_tanh(g))
                sh = np.sign(dn * oracle.gelu_tanh(g) * u)
                so = np.full(D, np.sign(we))
            o = perturbed_ffn(x[t], wg, wu, wd, we, sx, sg, su, sh, so, gemm_rel, act_rel, in_rel, in_abs)
            y[t] += o
            mag += np.abs(o)
        s = rng.choice([-1.0, 1.0], size=D) if target is None else np.full(D, direction)
        y[t] += s * (k + 3) * 2.0 ** -24 * mag
    return y


def perturbed_block(blk, rng, gemm_rel=1e-3, f32_rel=1e-5, target=None):
    """The MoE block in float64 at the oracle's routing with every device
    error at its limit: fp32 norms within f32_rel, h1 and h2 rounded to f16,
    both branches through perturbed_layer, fp32 sums.  Signs are random, or,
    with target = n, the FFN errors of both branches are aligned to move the
    output's element n of every token the same way (through the signs of the
    post-norm weights at n)."""
    from oracle.block import _Layer
    res = np.asarray(blk.residual, np.float64)
    T, D = res.shape
    sgn = lambda *shape: rng.choice([-1.0, 1.0], size=shape)
    in_rel = oracle.moe.F16_REL * (1 + f32_rel) + f32_rel
    ref, parts = oracle.moe_block_ref(blk, res, want_parts=True)
    dense = _Layer(parts["h1"], [blk.dense_gate], [blk.dense_up], [blk.dense_down], 1)
    d1 = d2 = 1.0
    if target is not None:
        d1 = float(np.sign(blk.post_ffw_norm[target] * blk.post_ffw_norm_1[target]))
        d2 = float(np.sign(blk.post_ffw_norm[target] * blk.post_ffw_norm_2[target]))
    b1 = perturbed_layer(dense, np.zeros((T, 1), np.int32), np.ones((T, 1)), rng, target=target, gemm_rel=gemm_rel,
                         in_rel=in_rel, in_abs=oracle.moe.F16_ABS, direction=d1)
    experts = _Layer(parts["h2"], blk.gate, blk.up, blk.down, blk.E)
    b2 = perturbed_layer(experts, parts["idx"], parts["w"], rng, target=target, gemm_rel=gemm_rel, in_rel=in_rel,
                         in_abs=oracle.moe.F16_ABS, direction=d2)
    b1n = oracle.rmsnorm(b1, blk.post_ffw_norm_1) * (1 + f32_rel * sgn(T, D))
    b2n = oracle.rmsnorm(b2, blk.post_ffw_norm_2) * (1 + f32_rel * sgn(T, D))
    s = (b1n + b2n) * (1 + 2.0 ** -24 * sgn(T, D))
    c = oracle.rmsnorm(s, blk.post_ffw_norm) * (1 + f32_rel * sgn(T, D))
    return (res + c) * (1 + 2.0 ** -24 * sgn(T, D)), ref, parts
