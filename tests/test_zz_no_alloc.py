"""moe_grouped_qgemm_noalloc (no workspace, the library's per-device scratch
array) against moe_grouped_qgemm with a workspace, through the C ABI: two
calls in a row, the second on a smaller layer, each bitwise equal to the
workspace entry point and within the oracle's bound; a shape whose scratch
exceeds the array is refused."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def q4():
    import moe_w4a16_skinny_amd as m
    return m


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_both(moe, idx, w):
    m = q4()
    lib = m.raw()
    mw = m.moe_pack_experts(moe.gate, moe.up, moe.down, moe.E, moe.has_shared)
    d = mw.desc()
    x, ti, tw = dev(moe.x), dev(idx.astype(np.int32)), dev(w.astype(np.float32))
    T, k = idx.shape
    y_ws = torch.empty((T, moe.D), dtype=torch.float32, device="cuda")
    y_na = torch.full((T, moe.D), float("nan"), dtype=torch.float32, device="cuda")
    wsb = lib.moe_workspace_bytes(C.byref(d), T, k)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    s = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    vp = lambda t: C.c_void_p(t.data_ptr())
    rc = lib.moe_grouped_qgemm_noalloc(C.byref(d), vp(x), vp(ti), vp(tw), T, k, vp(y_na), m.Q4_F32, s)
    assert rc == 0, m.raw().q4_last_error()
    rc = lib.moe_grouped_qgemm(C.byref(d), vp(x), vp(ti), vp(tw), T, k, vp(y_ws), m.Q4_F32, vp(ws), wsb, s)
    assert rc == 0, m.raw().q4_last_error()
    torch.cuda.synchronize()
    return y_na.cpu().numpy(), y_ws.cpu().numpy()


def check(moe):
    _, idx, w = oracle.route_topk(moe.x, moe.w_router, moe.k)
    w32 = w.astype(np.float32).astype(np.float64)
    y_na, y_ws = run_both(moe, idx, w32)
    assert np.array_equal(y_na.view(np.uint32), y_ws.view(np.uint32)), "no-alloc output differs from the workspace one"
    ref, _ = oracle.moe_ref_grouped(moe, idx, w32)
    assert np.all(np.abs(y_na - ref) <= oracle.moe_abs_bound(moe, idx, w32))


def test_noalloc_equals_workspace_entry_two_calls():
    print("no-alloc MoE: the 129-expert layer, then a smaller one", flush=True)
    check(synth.moe_layer(104, T=16, D=2816, E=128, F=704, k=8, has_shared=True))
    check(synth.moe_layer(331, T=5, D=256, E=8, F=128, k=3, has_shared=True))


def test_noalloc_refuses_scratch_beyond_the_array():
    m = q4()
    lib = m.raw()
    p = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    a = C.c_void_p(p.data_ptr())
    big = m.q4_moe_desc(64, 1, 8192, 8192, a, a, a, a, a, a)   # (16 * 16 + 16) rows of 8192: > 8 MiB
    assert lib.moe_workspace_bytes(C.byref(big), 16, 16) > (8 << 20)
    rc = lib.moe_grouped_qgemm_noalloc(C.byref(big), a, a, a, 16, 16, a, m.Q4_F32,
                                       C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == m.Q4_ERR_UNSUPPORTED and b"8388608" in lib.q4_last_error()
