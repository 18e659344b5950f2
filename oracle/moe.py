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


def a16(v):
    """The 16-bit activation of W4A16 [README, "Why it's NVIDIA-only": W4A16,
    4-bit weights times 16-bit activations]: v rounded to the nearest f16
    (ties to even; beyond the f16 range, infinite), returned in float64."""
    with np.errstate(over="ignore"):
        return np.asarray(v, np.float64).astype(np.float16).astype(np.float64)


def _ffn(x_rows, wg, wu, wd, a16_h=False):
    g = x_rows @ wg.T
    u = x_rows @ wu.T
    h = gelu_tanh(g) * u
    hd = a16(h) if a16_h else h
    return g, u, h, hd @ wd.T


def moe_ref(moe, idx, w, a16_h: bool = False) -> np.ndarray:
    """Per-token form: y[t] = sum_{j<k} w[t,j] * FFN_{idx[t,j]}(x[t]) + FFN_shared(x[t]).

    ``moe`` is a ``synth.MoeInputs``; idx/w are the routing (from ``route_topk``).
    a16_h: the down projection takes h as a 16-bit activation (a16), as the
    W4A16 GEMM it is; otherwise everything is exact float64.
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
            y[t] += float(w[t, j]) * _ffn(x[t:t + 1], wg, wu, wd, a16_h)[3][0]
        if moe.has_shared:
            wg, wu, wd = mats(moe.E)
            y[t] += _ffn(x[t:t + 1], wg, wu, wd, a16_h)[3][0]
    return y


def moe_ref_grouped(moe, idx, w, a16_h: bool = False):
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
        out = _ffn(x[[t for t, _ in rows]], wg, wu, wd, a16_h)[3]
        for r, (t, s) in enumerate(rows):
            contrib[t, s] = float(w[t, s]) * out[r]
        active.append(e)
    if moe.has_shared:
        wg, wu, wd = _expert_mats(moe, moe.E)
        contrib[:, k] = _ffn(x, wg, wu, wd, a16_h)[3]
        active.append(moe.E)
    return contrib.sum(axis=1), active


# sup |gelu_tanh''(u)| over all u: attained at u = 0, where it is sqrt(2/pi)
# (pinned by a test on a dense grid and the closed form at 0)
GELU_D2_MAX = _C
# f16 round-to-nearest of a finite value v: |f16(v) - v| <= 2^-11 |v| + 2^-25
# (relative half-ulp for normal results, half the subnormal spacing below)
F16_REL = 2.0 ** -11
F16_ABS = 2.0 ** -25
# one fp32 rounding: 2^-24 relative
F32_ULP = 2.0 ** -24


def _h_error(g, u, rg, ru, act_rel):
    """Bound on |h_gpu - h| for h = gelu_tanh(g) * u, when the device's gate and
    up outputs differ from the exact g, u by at most rg, ru (elementwise), it
    evaluates h in fp32 within act_rel of the exact h of its own inputs, and it
    stores h as f16.  By the mean value theorem,
      |gelu(g~) u~ - gelu(g) u| <= L rg (|u| + ru) + |gelu(g)| ru,
      L = max |gelu'| over [g - rg, g + rg] <= |gelu'(g)| + GELU_D2_MAX rg;
    then the fp32 evaluation and the f16 store of a value within that bound of h."""
    L = np.abs(gelu_tanh_deriv(g)) + GELU_D2_MAX * rg
    dh = L * rg * (np.abs(u) + ru) + np.abs(gelu_tanh(g)) * ru
    return dh + (act_rel + F16_REL * (1.0 + act_rel)) * (np.abs(gelu_tanh(g) * u) + dh) + F16_ABS


def moe_abs_bound(moe, idx, w, gemm_rel: float = 1e-3, in_rel: float = 0.0, in_abs: float = 0.0,
                  act_rel: float = 1e-4, w_rel: float = 0.0) -> np.ndarray:
    """Rigorous elementwise tolerance [T][D] for the device's MoE layer output.

    Assumptions, each the contract of one device step:
      * the device's GEMM inputs x~ satisfy |x~ - x| <= in_rel |x| + in_abs
        (0 for the layer, whose x is given in f16; the block's normalized rows
        are rounded to f16 on the device);
      * each GEMM output is within gemm_rel * sum_k |a_k w_k| of the exact
        product of the device's own inputs (the per-GEMM criterion);
      * h is evaluated in fp32 within act_rel of its exact value and stored as
        f16 (_h_error); the default 1e-4 covers a hardware exp2 whose fp32
        argument carries a few roundings, up to arguments of several hundred
        (beyond, exp2 overflows and h is exactly 0, within F16_ABS of h);
      * the routing weights the device uses are within w_rel |w| of w (0 when
        it is handed w itself), and its epilogue product w * o and the k + 1
        slot sums add at most (k + 3) 2^-24 of sum |w o|.
    With G = |Wg| |x| and A = |Wg| 1 (per row j), the gate error is at most
      rg = (in_rel + gemm_rel (1 + in_rel)) G + (1 + gemm_rel) in_abs A
    and likewise ru for up; h's error dh follows from _h_error; down gives
      do_n = sum_j |Wd[n,j]| dh_j + gemm_rel sum_j |Wd[n,j]| (|h_j| + dh_j)
    and the combine
      bound = sum_e |w_e| do_e + (w_rel + (k + 3) 2^-24 (1 + w_rel)) sum_e |w_e| (|o_e| + do_e).
    Every step is an upper bound, not a first-order estimate, so an error
    pattern that meets each assumption with equality stays within it.
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
    comb = w_rel + (k + 3) * F32_ULP * (1.0 + w_rel)
    g_rel = in_rel + gemm_rel * (1.0 + in_rel)
    g_abs = (1.0 + gemm_rel) * in_abs
    bound = np.zeros((T, D))
    for e in sorted(users):
        wg, wu, wd = _expert_mats(moe, e)
        rows = [t for t, _ in users[e]]
        we = np.abs(np.array([v for _, v in users[e]]))
        xr = x[rows]
        g, u, h, o = _ffn(xr, wg, wu, wd)
        ax = np.abs(xr)
        rg = g_rel * (ax @ np.abs(wg).T) + g_abs * np.abs(wg).sum(axis=1)
        ru = g_rel * (ax @ np.abs(wu).T) + g_abs * np.abs(wu).sum(axis=1)
        dh = _h_error(g, u, rg, ru, act_rel)
        awd = np.abs(wd).T
        do = dh @ awd + gemm_rel * ((np.abs(h) + dh) @ awd)
        contrib = we[:, None] * do + comb * we[:, None] * (np.abs(o) + do)
        np.add.at(bound, rows, contrib)
    return bound
