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

from .moe import _expert_mats, _ffn, moe_abs_bound, moe_ref, softmax

EPS = 1e-6


def rmsnorm(v, w=None, eps: float = EPS):
    """v / sqrt(mean(v^2) + eps) * w, row by row (last axis)."""
    v = np.asarray(v, np.float64)
    r = np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    y = v / r
    return y if w is None else y * np.asarray(w, np.float64)


def rmsnorm_bound(v, w, B, eps: float = EPS):
    """First-order bound on |RMSNorm(v + dv; w) - RMSNorm(v; w)| for |dv| <= B
    (elementwise), row by row: with r = sqrt(mean(v^2) + eps),
    d y_i = w_i (dv_i / r - v_i (v . dv) / (D r^3))."""
    v = np.asarray(v, np.float64)
    D = v.shape[-1]
    r = np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    proj = np.sum(np.abs(v) * B, axis=-1, keepdims=True)
    return np.abs(np.asarray(w, np.float64)) * (B / r + np.abs(v) * proj / (D * r ** 3))


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


def moe_block_ref(blk, residual, want_parts: bool = False):
    """residual [T][D] -> residual + RMSNorm(b1 + b2; post_ffw_norm).

    ``blk`` is a ``synth.MoeBlockInputs``.  Returns the new residual (and the
    intermediates if want_parts)."""
    res = np.asarray(residual, np.float64)
    h1 = rmsnorm(res, blk.ffn_norm)
    h2 = rmsnorm(res, blk.pre_ffw_norm_2)
    dense = _Layer(h1, [blk.dense_gate], [blk.dense_up], [blk.dense_down], 1)
    T = res.shape[0]
    b1 = moe_ref(dense, np.zeros((T, 1), np.int32), np.ones((T, 1)))
    z, idx, w = route_normed(h2, blk.w_router, blk.router_scale, blk.down_scale, blk.k)
    experts = _Layer(h2, blk.gate, blk.up, blk.down, blk.E)
    b2 = moe_ref(experts, idx, w)
    b1n = rmsnorm(b1, blk.post_ffw_norm_1)
    b2n = rmsnorm(b2, blk.post_ffw_norm_2)
    c = rmsnorm(b1n + b2n, blk.post_ffw_norm)
    out = res + c
    if want_parts:
        return out, dict(h1=h1, h2=h2, b1=b1, b2=b2, z=z, idx=idx, w=w, b1n=b1n, b2n=b2n, c=c)
    return out


def moe_block_bound(blk, residual, parts, gemm_rel: float = 1e-3, f32_rel: float = 1e-5):
    """First-order elementwise tolerance of the block's output [T][D].

    The branches' FFN outputs may err by the composed expert-layer bound
    (oracle.moe_abs_bound: each GEMM within gemm_rel * sum|a w|, which also
    covers the f16 rounding of the normalized inputs); the bound is carried
    through the post-norms, the sum and the final norm by rmsnorm_bound; each
    fp32 norm and the residual add add f32_rel of their result."""
    res = np.asarray(residual, np.float64)
    T = res.shape[0]
    dense = _Layer(parts["h1"], [blk.dense_gate], [blk.dense_up], [blk.dense_down], 1)
    B1 = moe_abs_bound(dense, np.zeros((T, 1), np.int32), np.ones((T, 1)), gemm_rel=gemm_rel)
    experts = _Layer(parts["h2"], blk.gate, blk.up, blk.down, blk.E)
    B2 = moe_abs_bound(experts, parts["idx"], parts["w"], gemm_rel=gemm_rel)
    B2 = B2 + f32_rel * np.abs(parts["b2"])                    # routing weights in fp32
    B1n = rmsnorm_bound(parts["b1"], blk.post_ffw_norm_1, B1) + f32_rel * np.abs(parts["b1n"])
    B2n = rmsnorm_bound(parts["b2"], blk.post_ffw_norm_2, B2) + f32_rel * np.abs(parts["b2n"])
    s = parts["b1n"] + parts["b2n"]
    Bc = rmsnorm_bound(s, blk.post_ffw_norm, B1n + B2n) + f32_rel * np.abs(parts["c"])
    return Bc + f32_rel * np.abs(res + parts["c"])
