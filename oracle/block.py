"""The whole Gemma-4 MoE block around the expert FFNs, in float64.  (Test infrastructure only.)

[DOC 3.2 "Per-layer (MoE)"] and [DOC 4.6 "MoE"]: from the residual stream,
a dense MLP branch (RMSNorm with ffn_norm, the gated FFN, RMSNorm with
post_ffw_norm_1) and a MoE branch (RMSNorm with pre_ffw_norm_2; router
logits, an unweighted RMSNorm of the logits times the learned
ffn_gate_inp.scale, softmax, top-k; the kept experts' FFNs summed with the
routing weights; RMSNorm with post_ffw_norm_2) are added, normalized with
post_ffw_norm and added to the residual.  [DOC 14 "Completed", expert-
batched FFN]: the per-expert ffn_down_exps.scale factor is folded into the
routing weights.

Readings where the pages leave a step open (listed with the design notes):
* RMSNorm(v; w) = v / sqrt(mean(v^2) + eps) * w over the row, eps = 1e-6;
  the unweighted norm of the logits is the same with w = 1, over the E
  logits of the token;
* ffn_gate_inp.scale is one learned factor per expert (a vector of E);
* the FFN is the gated GELU-tanh FFN of the expert layer (oracle/moe.py),
  for the dense branch too, with its own width;
* no renormalization of the kept probabilities; top-k by decreasing value,
  ties to the lower expert index.
"""
from __future__ import annotations

import numpy as np

from .moe import F16_ABS, F16_REL, F32_ULP, _expert_mats, _ffn, a16, moe_abs_bound, moe_ref, softmax

EPS = 1e-6


def rmsnorm(v, w=None, eps: float = EPS):
    """v / sqrt(mean(v^2) + eps) * w, row by row (last axis)."""
    v = np.asarray(v, np.float64)
    r = np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    y = v / r
    return y if w is None else y * np.asarray(w, np.float64)


def rmsnorm_bound(v, w, B, eps: float = EPS):
    """Bound on |RMSNorm(v + dv; w) - RMSNorm(v; w)| for every |dv| <= B
    (elementwise), row by row.  With r = sqrt(mean(v^2) + eps) and
    q = sqrt(mean(B^2)): r is a Euclidean norm (of v and sqrt(D eps), over
    sqrt(D)), so |r' - r| <= q and r' >= r - q; then
      y'_i - y_i = w_i (dv_i / r' + v_i (r - r') / (r r'))
    gives |w_i| (B_i / (r - q) + |v_i| q / (r (r - q))).  Infinite where
    q >= r (the perturbation may reach a zero row)."""
    v = np.asarray(v, np.float64)
    B = np.asarray(B, np.float64)
    r = np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    q = np.sqrt(np.mean(B * B, axis=-1, keepdims=True))
    lo = r - q
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.abs(np.asarray(w, np.float64)) * (B / lo + np.abs(v) * q / (r * lo))
    return np.where(lo > 0, out, np.inf)


class _Layer:
    """the fields of synth.MoeInputs that oracle/moe.py reads, with another x"""

    def __init__(self, x, gate, up, down, E, has_shared=False):
        self.x, self.gate, self.up, self.down, self.E, self.has_shared = x, gate, up, down, E, has_shared


def route_normed(h2, w_router, router_scale, down_scale, k: int, eps: float = EPS):
    """Router of the block: (z = RMSNorm(h2 . W_r) * scale [T][E], idx [T][k], w [T][k]).
    Top-k by decreasing z (softmax is monotone), ties to the lower index;
    w = softmax(z)[idx] * down_scale[idx]."""
    logits = np.asarray(h2, np.float64) @ np.asarray(w_router, np.float64)
    z = rmsnorm(logits, router_scale, eps)
    p = softmax(z)
    T, E = z.shape
    idx = np.zeros((T, k), np.int32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-z[t, e], e))
        idx[t] = order[:k]
    w = np.take_along_axis(p, idx, axis=1) * np.asarray(down_scale, np.float64)[idx]
    return z, idx, w


def route_normed_bound(blk, h2, gemm_rel: float = 0.0, f32_rel: float = 1e-5):
    """Rigorous bound [T][E] on |z_device - z| for the block's router scores
    z = RMSNorm(h2 . W_r) * router_scale, when the device multiplies the f16
    h2 (|h2~ - h2| <= (2^-11 (1 + f32_rel) + f32_rel) |h2| + 2^-25) by the
    fp32 W_r with fp32 accumulation: D/4 sequential fp32 accumulations of
    4-term products (the 16x16x4 fp32 matrix step) add at most
    (D/4 + 1) 2^-24 of sum|h2~ W_r|, plus gemm_rel of it if given; the fp32
    norm adds f32_rel of its result, the scale one rounding."""
    h2 = np.asarray(h2, np.float64)
    wr = np.abs(np.asarray(blk.w_router, np.float64))
    D = h2.shape[1]
    in_rel = F16_REL * (1.0 + f32_rel) + f32_rel
    acc_rel = (D / 4 + 1) * F32_ULP + gemm_rel
    ah = np.abs(h2)
    S = ah @ wr
    A = wr.sum(axis=0)
    Bl = in_rel * S + F16_ABS * A + acc_rel * ((1 + in_rel) * S + F16_ABS * A)
    logits = h2 @ np.asarray(blk.w_router, np.float64)
    sc = np.asarray(blk.router_scale, np.float64)
    Rz = rmsnorm_bound(logits, sc, Bl)
    z = rmsnorm(logits, sc)
    return Rz + (f32_rel + F32_ULP) * (np.abs(z) + Rz)


def routing_weight_bound(z, zb, idx, down_scale=None, f32_rel: float = 1e-5):
    """Rigorous bound [T][k] on |w_device - w| for w = softmax(z)[idx] *
    down_scale[idx] when the device's scores are within zb of z: log p_e moves
    by at most zb_e + max_j zb_j (log-sum-exp is 1-Lipschitz in the max
    norm), so p~ is within p (exp(zb_e + max zb) - 1) of p; the fp32 softmax
    and the product with the down scale add f32_rel."""
    z = np.asarray(z, np.float64)
    p = softmax(z)
    zi = np.take_along_axis(zb, idx.astype(np.int64), axis=1)
    m = zb.max(axis=1, keepdims=True)
    pi = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    ds = np.ones(z.shape[1]) if down_scale is None else np.asarray(down_scale, np.float64)
    dsi = np.abs(ds[idx])
    dp = pi * np.expm1(zi + m)
    return dsi * (dp + f32_rel * (pi + dp))


def moe_block_ref(blk, residual, want_parts: bool = False, routing=None, a16_inputs: bool = False):
    """residual [T][D] -> residual + RMSNorm(b1 + b2; post_ffw_norm).

    ``blk`` is a ``synth.MoeBlockInputs``.  Returns the new residual (and the
    intermediates if want_parts).  ``routing`` = (idx [T][k], w [T][k])
    replaces the router's choice and weights (to evaluate the block at a
    routing taken elsewhere, where several are valid); z is still the
    oracle's.  a16_inputs: every activation that enters a 4-bit GEMM (h1 and
    h2 into the FFNs and the router, h into the down projections) is the
    16-bit activation of W4A16 (oracle.a16); the router's matrix is fp32 and
    its product exact."""
    res = np.asarray(residual, np.float64)
    h1 = rmsnorm(res, blk.ffn_norm)
    h2 = rmsnorm(res, blk.pre_ffw_norm_2)
    x1, x2 = (a16(h1), a16(h2)) if a16_inputs else (h1, h2)
    dense = _Layer(x1, [blk.dense_gate], [blk.dense_up], [blk.dense_down], 1)
    T = res.shape[0]
    b1 = moe_ref(dense, np.zeros((T, 1), np.int32), np.ones((T, 1)), a16_h=a16_inputs)
    z, idx, w = route_normed(x2, blk.w_router, blk.router_scale, blk.down_scale, blk.k)
    if routing is not None:
        idx = np.asarray(routing[0], np.int32)
        w = np.asarray(routing[1], np.float64)
    experts = _Layer(x2, blk.gate, blk.up, blk.down, blk.E)
    b2 = moe_ref(experts, idx, w, a16_h=a16_inputs)
    b1n = rmsnorm(b1, blk.post_ffw_norm_1)
    b2n = rmsnorm(b2, blk.post_ffw_norm_2)
    c = rmsnorm(b1n + b2n, blk.post_ffw_norm)
    out = res + c
    if want_parts:
        return out, dict(h1=h1, h2=h2, b1=b1, b2=b2, z=z, idx=idx, w=w, b1n=b1n, b2n=b2n, c=c)
    return out


def moe_block_bound(blk, residual, parts, gemm_rel: float = 1e-3, f32_rel: float = 1e-5, w_rel: float = 0.0):
    """Rigorous elementwise tolerance of the block's output [T][D], for the
    routing in ``parts`` (idx, w).

    The device computes each norm in fp32 (within f32_rel of the exact norm
    of its own input) and rounds h1, h2 to f16 before the GEMMs, so the
    branches' FFN inputs carry in_rel = 2^-11 (1 + f32_rel) + f32_rel and
    in_abs = 2^-25; each branch's FFN output is then within
    oracle.moe_abs_bound of the exact one (every GEMM within gemm_rel *
    sum|a w|; for the experts, the device's routing weights within w_rel of
    those in ``parts``: 0 when ``parts`` was computed at the device's own
    routing, see moe_block_ref).  rmsnorm_bound carries these through the
    post-norms, the sum and the final norm (each fp32 norm adding f32_rel of
    its result), and the residual add one fp32 rounding."""
    res = np.asarray(residual, np.float64)
    T = res.shape[0]
    in_rel = F16_REL * (1.0 + f32_rel) + f32_rel
    dense = _Layer(parts["h1"], [blk.dense_gate], [blk.dense_up], [blk.dense_down], 1)
    B1 = moe_abs_bound(dense, np.zeros((T, 1), np.int32), np.ones((T, 1)), gemm_rel=gemm_rel, in_rel=in_rel,
                       in_abs=F16_ABS)
    experts = _Layer(parts["h2"], blk.gate, blk.up, blk.down, blk.E)
    B2 = moe_abs_bound(experts, parts["idx"], parts["w"], gemm_rel=gemm_rel, in_rel=in_rel, in_abs=F16_ABS,
                       w_rel=w_rel)
    R1 = rmsnorm_bound(parts["b1"], blk.post_ffw_norm_1, B1)
    R2 = rmsnorm_bound(parts["b2"], blk.post_ffw_norm_2, B2)
    B1n = R1 + f32_rel * (np.abs(parts["b1n"]) + R1)
    B2n = R2 + f32_rel * (np.abs(parts["b2n"]) + R2)
    s = parts["b1n"] + parts["b2n"]
    Bs = B1n + B2n + F32_ULP * (np.abs(s) + B1n + B2n)
    Bc = rmsnorm_bound(s, blk.post_ffw_norm, Bs) + f32_rel * (np.abs(parts["c"]) + Bs)
    return Bc + F32_ULP * (np.abs(res + parts["c"]) + Bc)
