"""Router, gated GELU-tanh expert FFN and weighted combine, in float64.  (Test infrastructure only.)

[DOC 3.2 "Per-layer (MoE)" and 4.6 "MoE"]: the router multiplies the
hidden row by the router matrix, a softmax turns the logits into
probabilities and the top-k experts are kept; each kept expert runs its
gated FFN and the outputs are summed with the routing weights.  [README,
"What it is" / "Everything it has"]: 128 experts, top-8, plus one shared
expert that every token uses.  [DOC 3.1 and 14 "Completed: Expert-batched FFN
(GEGLU)"]: the gate half goes through GELU and multiplies the up half, then
the down projection.

Readings where the pages are silent or disagree (listed with the design notes):
* the router's RMSNorm and learned scale of DOC 3.2 are not applied: the
  logits are x . W_r with W_r stored [D][E];
* no renormalization of the kept probabilities (a flag selects it);
* top-k order is by decreasing fp32 logit, ties to the lower expert index;
* the activation is GELU with the tanh approximation on the gate half (the
  README's SwiGLU and the doc's GeGLU disagree; GeGLU is taken);
* the shared expert has the same shape as a routed one and weight 1.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import nvfp4_dequant

_C = math.sqrt(2.0 / math.pi)
_A = 0.044715


def gelu_tanh(u):
    """0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))).  Pinned against torch's
    gelu(approximate='tanh') in float64 and its odd-part identity."""
    u = np.asarray(u, np.float64)
    return 0.5 * u * (1.0 + np.tanh(_C * (u + _A * u ** 3)))


def gelu_tanh_deriv(u):
    """Analytic derivative of ``gelu_tanh`` (used only by the error bound)."""
    u = np.asarray(u, np.float64)
    th = np.tanh(_C * (u + _A * u ** 3))
    return 0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * _C * (1.0 + 3.0 * _A * u * u)


def softmax(l, axis=-1):
    """exp(l - max l) / sum exp(l - max l) along ``axis``, float64."""
    l = np.asarray(l, np.float64)
    z = np.exp(l - np.max(l, axis=axis, keepdims=True))
    return z / np.sum(z, axis=axis, keepdims=True)


def route_topk(x, w_router, k: int, renormalize: bool = False):
    """Router: (logits float64 [T][E], idx int32 [T][k], weights float64 [T][k]).

    logits = x . W_r (x [T][D], W_r [D][E]).  The choice of the k experts is an
    integer decision taken, as on the GPU, on fp32 logits: the exact logit is
    rounded once to fp32 and the experts are ordered by decreasing value, ties
    to the lower index.  The weights are the float64 softmax probabilities of
    the chosen experts (renormalized to sum 1 over the k if asked).
    """
    logits = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64)
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    p = softmax(logits, axis=1)
    l32 = logits.astype(np.float32)
    idx = np.empty((T, k), np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -l32[t].astype(np.float64)))  # value desc, index asc
        idx[t] = order[:k]
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return logits, idx, w


def _expert_mats(moe, e):
    gc, gs, gg = moe.gate[e]
    uc, us, ug = moe.up[e]
    dc, ds, dg = moe.down[e]
    return nvfp4_dequant(gc, gs, gg), nvfp4_dequant(uc, us, ug), nvfp4_dequant(dc, ds, dg)


def _ffn(x_rows, wg, wu, wd):
    g = x_rows @ wg.T
    u = x_rows @ wu.T
    h = gelu_tanh(g) * u
    return g, u, h, h @ wd.T


def moe_ref(moe, idx, w) -> np.ndarray:
    """Per-token form: y[t] = sum_{j<k} w[t,j] * FFN_{idx[t,j]}(x[t]) + FFN_shared(x[t]).

    ``moe`` is a ``synth.MoeInputs``; idx/w are the routing (from ``route_topk``).
    """
    x = np.asarray(moe.x, np.float64)
    T, D = x.shape
    y = np.zeros((T, D))
    cache = {}

    def mats(e):
        if e not in cache:
            cache[e] = _expert_mats(moe, e)
        return cache[e]

    for t in range(T):
        for j in range(idx.shape[1]):
            wg, wu, wd = mats(int(idx[t, j]))
            y[t] += float(w[t, j]) * _ffn(x[t:t + 1], wg, wu, wd)[3][0]
        if moe.has_shared:
            wg, wu, wd = mats(moe.E)
            y[t] += _ffn(x[t:t + 1], wg, wu, wd)[3][0]
    return y


def moe_ref_grouped(moe, idx, w):
    """Expert-grouped form (each expert's weights visited once, as in the README's
    grouped MoE and the doc's expert-batched FFN): pairs (token, slot) are
    sorted by expert, each expert runs once on its batch of rows, and the
    outputs are combined per token.  Returns (y, active experts in order).
    Must equal ``moe_ref`` up to float64 rounding; a test checks it.
    """
    x = np.asarray(moe.x, np.float64)
    T, D = x.shape
    k = idx.shape[1]
    pairs = [(int(idx[t, j]), t, j) for t in range(T) for j in range(k)]
    pairs.sort()
    contrib = np.zeros((T, k + 1, D))
    active = []
    i = 0
    while i < len(pairs):
        e = pairs[i][0]
        j0 = i
        while i < len(pairs) and pairs[i][0] == e:
            i += 1
        rows = [(t, s) for (_, t, s) in pairs[j0:i]]
        wg, wu, wd = _expert_mats(moe, e)
        out = _ffn(x[[t for t, _ in rows]], wg, wu, wd)[3]
        for r, (t, s) in enumerate(rows):
            contrib[t, s] = float(w[t, s]) * out[r]
        active.append(e)
    if moe.has_shared:
        wg, wu, wd = _expert_mats(moe, moe.E)
        contrib[:, k] = _ffn(x, wg, wu, wd)[3]
        active.append(moe.E)
    return contrib.sum(axis=1), active


def moe_abs_bound(moe, idx, w, gemm_rel: float = 1e-3, combine_rel: float = 1e-6) -> np.ndarray:
    """First-order tolerance for the whole layer, per output element [T][D].

    Each GEMM may err by gemm_rel * sum|a*w| (the per-GEMM criterion); the gate
    and up errors reach h through GELU's derivative, h's error reaches y through
    |W_down|; the combine adds combine_rel of the summed |w_e * o_e|:

      dh_j  = gemm_rel * (|gelu'(g_j) u_j| G_j + |gelu(g_j)| U_j),
              G_j = sum_k |x_k Wg[j,k]|,  U_j = sum_k |x_k Wu[j,k]|
      bound = sum_e |w_e| (gemm_rel * sum_j |h_j Wd[n,j]| + sum_j |Wd[n,j]| dh_j)
              + combine_rel * sum_e |w_e o_e[n]|

    Each expert's weights are decoded once for all the tokens routed to it.
    """
    x = np.asarray(moe.x, np.float64)
    T, D = x.shape
    k = idx.shape[1]
    users = {}
    for t in range(T):
        for j in range(k):
            users.setdefault(int(idx[t, j]), []).append((t, float(w[t, j])))
    if moe.has_shared:
        users[moe.E] = [(t, 1.0) for t in range(T)]
    bound = np.zeros((T, D))
    for e in sorted(users):
        wg, wu, wd = _expert_mats(moe, e)
        rows = [t for t, _ in users[e]]
        we = np.array([v for _, v in users[e]])
        xr = x[rows]
        g, u, h, o = _ffn(xr, wg, wu, wd)
        G = np.abs(xr) @ np.abs(wg).T
        U = np.abs(xr) @ np.abs(wu).T
        dh = gemm_rel * (np.abs(gelu_tanh_deriv(g) * u) * G + np.abs(gelu_tanh(g)) * U)
        term = gemm_rel * (np.abs(h) @ np.abs(wd).T) + dh @ np.abs(wd).T
        contrib = np.abs(we)[:, None] * term + combine_rel * np.abs(we[:, None] * o)
        np.add.at(bound, rows, contrib)
    return bound
