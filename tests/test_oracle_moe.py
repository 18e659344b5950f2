"""Pins of the oracle router / MoE: torch library routines (gelu tanh, softmax,
linear algebra) in float64 on weights decoded by an independent route,
closed-form special cases and brute force."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from conftest import read_golden
from perturb import perturbed_layer as _perturbed_layer

E2 = torch.tensor([float(v) for _, v in read_golden("e2m1_table.txt")], dtype=torch.float64)
E4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)


def _torch_dequant(codes, scales, g):
    c = torch.from_numpy(codes.astype(np.int64))
    q = torch.stack([c & 15, c >> 4], dim=-1).reshape(c.shape[0], -1)
    s = E4[torch.from_numpy(scales.astype(np.int64))].repeat_interleave(16, dim=1)
    return E2[q] * s * float(np.float32(g))


def test_gelu_matches_torch():
    u = torch.linspace(-12, 12, 20001, dtype=torch.float64)
    ref = F.gelu(u, approximate="tanh").numpy()
    got = oracle.gelu_tanh(u.numpy())
    assert np.max(np.abs(got - ref)) <= 1e-15 * (1 + np.abs(ref)).max()


def test_gelu_identities():
    u = np.linspace(-30, 30, 6001)
    assert oracle.gelu_tanh(0.0) == 0.0
    # tanh is odd: gelu(u) - gelu(-u) == u
    assert np.allclose(oracle.gelu_tanh(u) - oracle.gelu_tanh(-u), u, rtol=0, atol=1e-13)
    assert abs(oracle.gelu_tanh(30.0) - 30.0) < 1e-12 and abs(oracle.gelu_tanh(-30.0)) < 1e-12


def test_gelu_derivative_finite_difference():
    u = np.linspace(-6, 6, 241)
    h = 1e-6
    fd = (oracle.gelu_tanh(u + h) - oracle.gelu_tanh(u - h)) / (2 * h)
    assert np.max(np.abs(fd - oracle.gelu_tanh_deriv(u))) < 1e-8
    assert oracle.gelu_tanh_deriv(0.0) == 0.5


def test_softmax_matches_torch_and_sums_to_one():
    l = np.random.default_rng(0).normal(0, 3, (5, 128))
    ref = torch.softmax(torch.from_numpy(l), dim=1).numpy()
    got = oracle.softmax(l, axis=1)
    assert np.max(np.abs(got - ref)) < 1e-15
    assert np.allclose(got.sum(axis=1), 1.0, atol=1e-14)
    assert np.max(np.abs(oracle.softmax(l + 123.0, axis=1) - got)) < 1e-14   # shift invariance


def test_router_brute_force_and_ties():
    rng = np.random.default_rng(3)
    T, D, E, k = 6, 40, 16, 4
    x = rng.standard_normal((T, D)).astype(np.float16)
    wr = (rng.standard_normal((D, E)) * 0.02).astype(np.float32)
    wr[:, 9] = wr[:, 4]                    # planted exact tie between experts 4 and 9
    logits, idx, w = oracle.route_topk(x, wr, k)
    ref_l = torch.from_numpy(x.astype(np.float64)) @ torch.from_numpy(wr.astype(np.float64))
    assert np.max(np.abs(logits - ref_l.numpy())) < 1e-14
    p = torch.softmax(ref_l, dim=1).numpy()
    for t in range(T):
        l32 = logits[t].astype(np.float32)
        brute = sorted(range(E), key=lambda e: (-float(l32[e]), e))[:k]
        assert list(idx[t]) == brute
        assert np.allclose(w[t], p[t, brute], rtol=0, atol=1e-15)
        if 9 in idx[t]:
            assert 4 in idx[t] and list(idx[t]).index(4) < list(idx[t]).index(9)


def test_router_zero_matrix_is_uniform():
    x = np.random.default_rng(0).standard_normal((3, 32)).astype(np.float16)
    _, idx, w = oracle.route_topk(x, np.zeros((32, 128), np.float32), 8)
    assert np.array_equal(idx, np.tile(np.arange(8, dtype=np.int32), (3, 1)))
    assert np.all(w == 1.0 / 128)
    _, _, wn = oracle.route_topk(x, np.zeros((32, 128), np.float32), 8, renormalize=True)
    assert np.all(wn == 1.0 / 8)


def _tiny_moe(seed=5, T=3, D=32, E=4, F=16, k=2, shared=True):
    return synth.moe_layer(seed, T=T, D=D, E=E, F=F, k=k, has_shared=shared)


def _torch_moe(moe, idx, w):
    x = torch.from_numpy(moe.x.astype(np.float64))
    y = torch.zeros_like(x)
    for t in range(moe.T):
        sel = [(int(e), float(wt)) for e, wt in zip(idx[t], w[t])]
        if moe.has_shared:
            sel.append((moe.E, 1.0))
        for e, wt in sel:
            wg = _torch_dequant(*moe.gate[e])
            wu = _torch_dequant(*moe.up[e])
            wd = _torch_dequant(*moe.down[e])
            h = F.gelu(F.linear(x[t], wg), approximate="tanh") * F.linear(x[t], wu)
            y[t] += wt * F.linear(h, wd)
    return y.numpy()


def test_moe_matches_torch_composition():
    moe = _tiny_moe()
    _, idx, w = oracle.route_topk(moe.x, moe.w_router, moe.k)
    y = oracle.moe_ref(moe, idx, w)
    ref = _torch_moe(moe, idx, w)
    assert np.max(np.abs(y - ref)) <= 1e-13 * (1 + np.max(np.abs(ref)))


def test_moe_grouped_equals_per_token():
    moe = _tiny_moe(seed=8, T=5, D=64, E=6, F=32, k=3)
    _, idx, w = oracle.route_topk(moe.x, moe.w_router, moe.k)
    y = oracle.moe_ref(moe, idx, w)
    yg, active = oracle.moe_ref_grouped(moe, idx, w)
    assert np.max(np.abs(y - yg)) <= 1e-13 * (1 + np.max(np.abs(y)))
    assert active == sorted(set(idx.ravel().tolist())) + [moe.E]


def test_moe_all_experts_uniform_is_mean():
    # k == E with equal weights 1/E and no shared expert: the mean of all experts
    moe = _tiny_moe(seed=9, T=2, D=32, E=4, F=16, k=4, shared=False)
    idx = np.tile(np.arange(4, dtype=np.int32), (2, 1))
    w = np.full((2, 4), 0.25)
    y = oracle.moe_ref(moe, idx, w)
    singles = [oracle.moe_ref(moe, np.full((2, 1), e, np.int32), np.ones((2, 1))) for e in range(4)]
    assert np.max(np.abs(y - np.mean(singles, axis=0))) < 1e-13


def test_moe_single_expert_is_dense_gated_ffn():
    moe = _tiny_moe(seed=10, T=2, D=32, E=1, F=16, k=1, shared=False)
    y = oracle.moe_ref(moe, np.zeros((2, 1), np.int32), np.ones((2, 1)))
    x = moe.x.astype(np.float64)
    wg = _torch_dequant(*moe.gate[0]).numpy()
    wu = _torch_dequant(*moe.up[0]).numpy()
    wd = _torch_dequant(*moe.down[0]).numpy()
    g = x @ wg.T
    ref = (0.5 * g * (1 + np.tanh(math.sqrt(2 / math.pi) * (g + 0.044715 * g ** 3))) * (x @ wu.T)) @ wd.T
    assert np.max(np.abs(y - ref)) < 1e-13


# ---------------------------------------------------------------- composed bound

def test_gelu_second_derivative_is_bounded_by_its_value_at_zero():
    # the curvature constant of the bound: sup |gelu''| = sqrt(2/pi), at u = 0
    u = np.linspace(-40.0, 40.0, 800001)
    h = 1e-4
    d2 = (oracle.gelu_tanh_deriv(u + h) - oracle.gelu_tanh_deriv(u - h)) / (2 * h)
    assert np.max(np.abs(d2)) <= oracle.moe.GELU_D2_MAX * (1 + 1e-6)
    assert abs(d2[400000] - math.sqrt(2 / math.pi)) < 1e-6


def _check_layer_bound(moe, idx, w, rng):
    """every perturbation at the contract's limit stays within moe_abs_bound,
    and an aligned one reaches it; returns the worst deviation / bound"""
    y = oracle.moe_ref(moe, idx, w)
    bnd = oracle.moe_abs_bound(moe, idx, w)
    worst = 0.0
    for _ in range(3):
        dev = np.abs(_perturbed_layer(moe, idx, w, rng) - y)
        assert np.all(dev <= bnd), f"random signs: dev/bound {np.max(dev / bnd):.4f}"
        worst = max(worst, float(np.max(dev / bnd)))
    for t_n in range(3):
        n = int(rng.integers(moe.x.shape[1]))
        dev = np.abs(_perturbed_layer(moe, idx, w, rng, target=n) - y)
        assert np.all(dev <= bnd), f"aligned at {n}: dev/bound {np.max(dev / bnd):.4f}"
        # the aligned element of the token whose experts were aligned for it
        ratio = dev[:, n] / bnd[:, n]
        worst = max(worst, float(ratio.max()))
        assert ratio.min() >= 0.9, f"aligned error reaches only {ratio.min():.3f} of the bound"
    return worst


@pytest.mark.parametrize("T,D,E,F,k,shared", [(3, 64, 4, 32, 2, True), (2, 256, 6, 128, 3, False),
                                               (2, 704, 8, 64, 2, True)])
def test_moe_bound_dominates_contract_limit_errors_and_is_reached(T, D, E, F, k, shared):
    moe = _tiny_moe(seed=30 + D, T=T, D=D, E=E, F=F, k=k, shared=shared)
    _, idx, w = oracle.route_topk(moe.x, moe.w_router, moe.k)
    worst = _check_layer_bound(moe, idx, w, np.random.default_rng(D))
    assert worst >= 1 / 20  # not vacuous: a permitted error pattern comes close to it


def test_moe_bound_fails_without_the_h_error_term(monkeypatch):
    # a planted mistake: the bound without the gate/up errors propagated into
    # h (only h's own rounding kept) must be exceeded by the aligned pattern
    moe = _tiny_moe(seed=44, T=2, D=256, E=4, F=64, k=2, shared=True)
    _, idx, w = oracle.route_topk(moe.x, moe.w_router, moe.k)
    full = oracle.moe.moe_abs_bound(moe, idx, w)

    def h_error_rounding_only(g, u, rg, ru, act_rel):
        h = np.abs(oracle.gelu_tanh(g) * u)
        return (act_rel + oracle.moe.F16_REL) * h + oracle.moe.F16_ABS

    monkeypatch.setattr(oracle.moe, "_h_error", h_error_rounding_only)
    assert np.all(oracle.moe.moe_abs_bound(moe, idx, w) < full)
    with pytest.raises(AssertionError):
        _check_layer_bound(moe, idx, w, np.random.default_rng(1))


def test_moe_bound_grows_with_the_gemm_criterion():
    moe = _tiny_moe()
    _, idx, w = oracle.route_topk(moe.x, moe.w_router, moe.k)
    b1 = oracle.moe_abs_bound(moe, idx, w, 1e-3)
    b2 = oracle.moe_abs_bound(moe, idx, w, 2e-3)
    assert np.all(b1 > 0) and np.all(b2 > 1.9 * b1 - oracle.moe.F16_ABS * 1e3)


def test_a16_is_round_to_nearest_even_f16():
    # the 16-bit activation of W4A16: torch's fp16 conversion (RNE) on normal,
    # subnormal, tie and overflowing values
    v = np.concatenate([np.random.default_rng(4).standard_normal(10000) * 3,
                        [1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -24 * 1.5, 2.0 ** -25, 65504.0, 65520.0, -0.0]])
    got = oracle.a16(v)
    ref = torch.from_numpy(v).to(torch.float16).to(torch.float64).numpy()
    assert np.array_equal(got, ref, equal_nan=True)
    assert got[-7] == 1.0 and got[-6] == 1 + 2.0 ** -9 and np.isinf(got[-2])


def test_a16_h_moves_the_layer_within_its_rounding_bound():
    # the layer with h as an f16 activation differs from the exact one by at
    # most the bound's share for h's rounding (no GEMM error, no fp32 error)
    moe = _tiny_moe(seed=12, T=3, D=256, E=6, F=128, k=2)
    _, idx, w = oracle.route_topk(moe.x, moe.w_router, moe.k)
    d = np.abs(oracle.moe_ref(moe, idx, w, a16_h=True) - oracle.moe_ref(moe, idx, w))
    b = oracle.moe_abs_bound(moe, idx, w, gemm_rel=0.0, act_rel=0.0)
    assert np.all(d <= b) and np.max(d) > 0
    yg, _ = oracle.moe_ref_grouped(moe, idx, w, a16_h=True)
    assert np.max(np.abs(yg - oracle.moe_ref(moe, idx, w, a16_h=True))) < 1e-13
