"""CPU tests of the C-ABI library: it loads, exports every declared symbol, its
offline repack is a bijection with the documented placement, and every
refusal returns its status before anything reaches a GPU."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import moe_w4a16_skinny_amd as q4
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "q4mi.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol():
    declared = _declared_functions()
    assert len(declared) >= 17
    lib = C.CDLL(q4.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(q4.EXPORTED)
    assert q4.abi_version() == 4


@pytest.mark.parametrize("N,K", [(16, 128), (32, 64), (16, 704), (48, 2816), (16, 80), (32, 176), (16, 16)])
def test_nvfp4_repack_round_trip(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (N, K // 16), dtype=np.uint8)
    packed = q4.q4_nvfp4_repack(codes, scales)
    Kp = (K + 63) // 64 * 64
    assert packed.size == q4.q4_nvfp4_packed_bytes(N, K) == (N // 16) * ((Kp // 128) * 1152 + (Kp % 128 // 64) * 576) + (Kp % 128 // 64) * 576
    if K % 64 == 0:  # no padding: exactly the algorithmic bytes, plus the zero guard after a half tile
        assert packed.size == N * K // 2 + N * K // 16 + (K % 128 // 64) * 576
        assert not packed[packed.size - (K % 128 // 64) * 576:].any()
    c2, s2 = q4.q4_nvfp4_unpack(packed, N, K)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    # every byte of the canonical input lands in a distinct packed byte
    assert np.count_nonzero(packed) <= codes.size + scales.size


@pytest.mark.parametrize("N,K", [(16, 128), (32, 64), (16, 5120), (48, 704)])
def test_affine_repack_round_trip(N, K):
    codes, s, b = synth.affine_weights(N + K, N, K)
    packed = q4.q4_affine4_repack(codes, s, b)
    assert packed.size == q4.q4_affine4_packed_bytes(N, K) == N * K // 2 + N * (K // 64) * 4 + (K % 128 // 64) * 576
    c2, s2, b2 = q4.q4_affine4_unpack(packed, N, K)
    assert np.array_equal(codes, c2) and np.array_equal(s, s2) and np.array_equal(b, b2)


def test_nvfp4_placement_matches_operand_layout():
    """A single code at (n, k) lands in lane (k%32)//8 * 16 + n%16 of its tile,
    code dword (k%128)//32, byte (k%8)//2, nibble k%2; its scale in word
    (n%16, (k%32)//16), byte (k%128)//32."""
    N, K = 32, 384
    for (n, k) in [(0, 0), (5, 37), (17, 200), (31, 383), (16, 129)]:
        q = np.zeros((N, K), np.uint8)
        q[n, k] = 0x7
        sc = np.zeros((N, K // 16), np.uint8)
        sc[n, k // 16] = 0x38
        packed = q4.q4_nvfp4_repack(synth.pack_nibbles(q), sc)
        pb = (K // 128) * 1152
        tile = (n // 16) * pb + (k // 128) * 1152
        lane = ((k % 32) // 8) * 16 + n % 16
        byte = tile + lane * 16 + ((k % 128) // 32) * 4 + (k % 8) // 2
        nz = np.flatnonzero(packed)
        assert len(nz) == 2
        assert nz[0] == byte and packed[byte] == (0x7 << (4 * (k % 2)))
        sbyte = tile + 1024 + ((n % 16) * 2 + (k % 32) // 16) * 4 + (k % 128) // 32
        assert nz[1] == sbyte and packed[sbyte] == 0x38


def test_affine_placement_matches_operand_layout():
    """Element k of column n: lane (k%32)//8*16 + n%16, dword (k%128)//32, element
    j = k%8 at nibble j//2 (+4 if j is odd); scale/bias of group k//64 at
    tile + 1024 + (n%16)*8 + ((k%128)//64)*4."""
    N, K = 16, 256
    for (n, k) in [(0, 0), (3, 9), (15, 255), (7, 130)]:
        q = np.zeros((N, K), np.uint8)
        q[n, k] = 0xB
        s = np.zeros((N, K // 64), np.uint16)
        b = np.zeros((N, K // 64), np.uint16)
        s[n, k // 64] = 0x3F80
        b[n, k // 64] = 0x4000
        packed = q4.q4_affine4_repack(synth.pack_nibbles(q), s, b)
        tile = (k // 128) * 1152
        lane = ((k % 32) // 8) * 16 + n
        j = k % 8
        word = tile + lane * 16 + ((k % 128) // 32) * 4
        shift = 4 * (j // 2) + (16 if j % 2 else 0)
        val = int.from_bytes(packed[word:word + 4].tobytes(), "little")
        assert val == 0xB << shift
        sb = tile + 1024 + n * 8 + ((k % 128) // 64) * 4
        assert packed[sb:sb + 4].tobytes() == bytes([0x80, 0x3F, 0x00, 0x40])
        assert np.count_nonzero(packed) == 1 + 3


def _err(status):
    return q4.raw().q4_last_error().decode()


def test_gemm_refusals_without_gpu():
    lib = q4.raw()
    buf = (C.c_uint8 * 4096)()
    base = C.addressof(buf)
    al = (base + 15) & ~15
    p = C.c_void_p(al)
    mis = C.c_void_p(al + 4)
    cases = [
        (lambda: lib.qgemm_nvfp4(None, 1.0, p, 1, 64, 16, p, q4.Q4_F32, None, None, 0, None), q4.Q4_ERR_INVALID_ARG, "w_packed"),
        (lambda: lib.qgemm_nvfp4(p, 1.0, p, 0, 64, 16, p, q4.Q4_F32, None, None, 0, None), q4.Q4_ERR_UNSUPPORTED, "M=0"),
        (lambda: lib.qgemm_nvfp4(p, 1.0, p, 17, 64, 16, p, q4.Q4_F32, p, p, 4096, None), q4.Q4_ERR_UNSUPPORTED, "M=17"),
        (lambda: lib.qgemm_nvfp4(p, 1.0, p, 65537, 64, 16, p, q4.Q4_F32, None, None, 0, None), q4.Q4_ERR_UNSUPPORTED,
         "M=65537"),
        (lambda: lib.qgemm_affine4(p, p, 17, 128, 16, p, q4.Q4_F32, None, 0, None), q4.Q4_ERR_UNSUPPORTED, "M=17"),
        (lambda: lib.qgemm_nvfp4(p, 1.0, p, 1, 64, 24, p, q4.Q4_F32, None, None, 0, None), q4.Q4_ERR_UNSUPPORTED, "N=24"),
        (lambda: lib.qgemm_nvfp4(p, 1.0, p, 1, 72, 16, p, q4.Q4_F32, None, None, 0, None), q4.Q4_ERR_UNSUPPORTED, "K=72"),
        (lambda: lib.qgemm_nvfp4(p, 1.0, p, 1, 64, 16, p, 9, None, None, 0, None), q4.Q4_ERR_INVALID_ARG, "out_dtype"),
        (lambda: lib.qgemm_nvfp4(mis, 1.0, p, 1, 64, 16, p, q4.Q4_F32, None, None, 0, None), q4.Q4_ERR_ALIGNMENT, "w_packed"),
        (lambda: lib.qgemm_nvfp4(p, 1.0, mis, 1, 64, 16, p, q4.Q4_F32, None, None, 0, None), q4.Q4_ERR_ALIGNMENT, "a is"),
        (lambda: lib.qgemm_nvfp4(p, 1.0, p, 1, 64, 16, p, q4.Q4_F32, p, None, 0, None), q4.Q4_ERR_WORKSPACE, "ws is NULL"),
        (lambda: lib.qgemm_nvfp4(p, 1.0, p, 1, 64, 16, p, q4.Q4_F32, p, p, 8, None), q4.Q4_ERR_WORKSPACE, "ws_bytes"),
        (lambda: lib.qgemm_affine4(p, p, 1, 96, 16, p, q4.Q4_F32, None, 0, None), q4.Q4_ERR_UNSUPPORTED, "K=96"),
        (lambda: lib.qgemm_affine4(p, p, 1, 128, 16, p, q4.Q4_F16, None, 0, None), q4.Q4_ERR_INVALID_ARG, "out_dtype"),
        (lambda: lib.qgemm_affine4(p, p, 16, 8192, 131072, p, q4.Q4_F32, None, 0, None), q4.Q4_ERR_WORKSPACE, "ws is NULL"),
        (lambda: lib.qgemm_nvfp4(p, 1.0, p, 16, 4096, 8192, p, q4.Q4_F16, p, p, 64, None), q4.Q4_ERR_WORKSPACE, "ws_bytes"),
        (lambda: lib.q4_dequant_nvfp4(p, 1.0, 15, 64, p, None), q4.Q4_ERR_UNSUPPORTED, "N=15"),
    ]
    # these shapes must need a workspace, or the refusal cases above would launch
    assert lib.qgemm_affine4_workspace_bytes(16, 8192, 131072) > 0
    assert lib.qgemm_nvfp4_workspace_bytes(16, 4096, 8192, 1) > 64
    for call, code, needle in cases:
        assert call() == code, needle
        assert needle in _err(code), (needle, _err(code))


def test_router_and_moe_refusals_without_gpu():
    lib = q4.raw()
    buf = (C.c_uint8 * 4096)()
    p = C.c_void_p((C.addressof(buf) + 15) & ~15)
    ws = lib.moe_route_workspace_bytes(16, 2816, 128)
    assert ws >= 256 + 16 * 128 * 4
    cases = [
        (lambda: lib.moe_route_topk(p, p, 65, 64, 128, 8, 0, None, p, p, p, 1 << 30, None), q4.Q4_ERR_UNSUPPORTED, "T=65"),
        (lambda: lib.moe_route_topk(p, p, 4, 64, 8, 9, 0, None, p, p, p, 1 << 30, None), q4.Q4_ERR_UNSUPPORTED, "k=9"),
        (lambda: lib.moe_route_topk(p, p, 4, 60, 8, 2, 0, None, p, p, p, 1 << 30, None), q4.Q4_ERR_UNSUPPORTED, "D=60"),
        (lambda: lib.moe_route_topk(p, p, 4, 64, 8, 2, 0, None, p, p, None, 0, None), q4.Q4_ERR_WORKSPACE, "ws"),
        (lambda: lib.moe_route_topk(p, p, 4, 64, 8, 2, 0, None, p, p, p, 16, None), q4.Q4_ERR_WORKSPACE, "ws_bytes"),
        (lambda: lib.moe_route_topk(None, p, 4, 64, 8, 2, 0, None, p, p, p, 1 << 30, None), q4.Q4_ERR_INVALID_ARG, "x"),
    ]
    for call, code, needle in cases:
        assert call() == code, needle
        assert needle in _err(code), (needle, _err(code))
    d = q4.q4_moe_desc(128, 1, 2816, 704, p.value, p.value, p.value, p.value, p.value, p.value)
    need = lib.moe_workspace_bytes(C.byref(d), 16, 8)
    assert need >= 144 * 704 * 2 + 144 * 2816 * 4
    mcases = [
        (lambda: lib.moe_grouped_qgemm(C.byref(d), p, p, p, 17, 8, p, q4.Q4_F32, p, need, None), q4.Q4_ERR_UNSUPPORTED, "T=17"),
        (lambda: lib.moe_grouped_qgemm(C.byref(d), p, p, p, 16, 129, p, q4.Q4_F32, p, need, None), q4.Q4_ERR_UNSUPPORTED, "k=129"),
        (lambda: lib.moe_grouped_qgemm(C.byref(d), p, p, p, 16, 65, p, q4.Q4_F32, p, need, None), q4.Q4_ERR_UNSUPPORTED, "k=65"),
        (lambda: lib.moe_grouped_qgemm(C.byref(d), p, p, p, 16, 8, p, q4.Q4_BF16, p, need, None), q4.Q4_ERR_INVALID_ARG, "out_dtype"),
        (lambda: lib.moe_grouped_qgemm(C.byref(d), p, p, p, 16, 8, p, q4.Q4_F32, p, need - 1, None), q4.Q4_ERR_WORKSPACE, "ws_bytes"),
        (lambda: lib.moe_grouped_qgemm(None, p, p, p, 16, 8, p, q4.Q4_F32, p, need, None), q4.Q4_ERR_INVALID_ARG, "w is NULL"),
    ]
    for call, code, needle in mcases:
        assert call() == code, needle
        assert needle in _err(code), (needle, _err(code))
    bad = q4.q4_moe_desc(128, 1, 2800, 704, p.value, p.value, p.value, p.value, p.value, p.value)
    assert lib.moe_grouped_qgemm(C.byref(bad), p, p, p, 16, 8, p, q4.Q4_F32, p, 1 << 30, None) == q4.Q4_ERR_UNSUPPORTED


def test_repack_refusals():
    with pytest.raises(q4.Q4Error) as ei:
        q4.q4_nvfp4_repack(np.zeros((24, 32), np.uint8), np.zeros((24, 4), np.uint8))
    assert ei.value.status == q4.Q4_ERR_UNSUPPORTED and "N=24" in str(ei.value)
    with pytest.raises(q4.Q4Error) as ei:
        q4.q4_affine4_repack(np.zeros((16, 48), np.uint8), np.zeros((16, 1), np.uint16), np.zeros((16, 1), np.uint16))
    assert ei.value.status == q4.Q4_ERR_UNSUPPORTED and "K=96" in str(ei.value)
    assert q4.q4_nvfp4_packed_bytes(16, 24) == 0 and q4.q4_affine4_packed_bytes(16, 96) == 0


def test_quantize_refusals_without_gpu():
    lib = q4.raw()
    buf = (C.c_uint8 * 4096)()
    al = (C.addressof(buf) + 15) & ~15
    p = C.c_void_p(al)
    mis = C.c_void_p(al + 4)
    nb = lib.q4_nvfp4_packed_bytes(16, 64)
    wsb = lib.q4_nvfp4_quantize_workspace_bytes()
    assert wsb > 0
    cases = [
        (lambda: lib.q4_nvfp4_quantize(None, 16, 64, 0.0, p, nb, None, p, wsb, None), q4.Q4_ERR_INVALID_ARG, "w"),
        (lambda: lib.q4_nvfp4_quantize(p, 16, 64, 0.0, None, nb, None, p, wsb, None), q4.Q4_ERR_INVALID_ARG, "packed"),
        (lambda: lib.q4_nvfp4_quantize(p, 15, 64, 0.0, p, nb, None, p, wsb, None), q4.Q4_ERR_UNSUPPORTED, "N=15"),
        (lambda: lib.q4_nvfp4_quantize(p, 16, 72, 0.0, p, nb, None, p, wsb, None), q4.Q4_ERR_UNSUPPORTED, "K=72"),
        (lambda: lib.q4_nvfp4_quantize(p, 16, 64, 0.0, p, nb - 1, None, p, wsb, None), q4.Q4_ERR_INVALID_ARG,
         "packed_bytes"),
        (lambda: lib.q4_nvfp4_quantize(p, 16, 64, float("nan"), p, nb, None, p, wsb, None), q4.Q4_ERR_INVALID_ARG,
         "not finite"),
        (lambda: lib.q4_nvfp4_quantize(p, 16, 64, float("-inf"), p, nb, None, p, wsb, None), q4.Q4_ERR_INVALID_ARG,
         "not finite"),
        (lambda: lib.q4_nvfp4_quantize(mis, 16, 64, 0.0, p, nb, None, p, wsb, None), q4.Q4_ERR_ALIGNMENT, "w is"),
        (lambda: lib.q4_nvfp4_quantize(p, 16, 64, 0.0, mis, nb, None, p, wsb, None), q4.Q4_ERR_ALIGNMENT, "packed is"),
        (lambda: lib.q4_nvfp4_quantize(p, 16, 64, 0.0, p, nb, None, None, 0, None), q4.Q4_ERR_WORKSPACE, "ws is NULL"),
        (lambda: lib.q4_nvfp4_quantize(p, 16, 64, 0.0, p, nb, None, p, wsb - 1, None), q4.Q4_ERR_WORKSPACE,
         "ws_bytes"),
        (lambda: lib.q4_nvfp4_quantize(p, 16, 64, 0.0, p, nb, None, mis, wsb, None), q4.Q4_ERR_ALIGNMENT, "ws is"),
    ]
    for call, code, needle in cases:
        assert call() == code, needle
        assert needle in _err(code), (needle, _err(code))


@pytest.mark.parametrize("bits", [2, 3, 5, 6, 8])
@pytest.mark.parametrize("N,K", [(16, 64), (32, 192), (48, 640)])
def test_affine_bits_repack_round_trip_and_placement(bits, N, K):
    import synth
    q, s, b = synth.affine_weights_bits(11 + bits, N, K, bits)
    packed = q4.q4_affine_bits_repack(q, s, b, bits)
    nt = -(-K // 128)
    assert packed.size == N // 16 * nt * (256 * bits + 128) == q4.raw().q4_affine_bits_packed_bytes(N, K, bits)
    q2, s2, b2 = q4.q4_affine_bits_unpack(packed, N, K, bits)
    assert np.array_equal(q2, q) and np.array_equal(s2, s) and np.array_equal(b2, b)
    # placement as documented: lane (c, o) of tile t holds 4 * bits bytes, code (i, j)
    # (k = 128 t + 32 i + 8 o + j) at bit 8 bits i + bits j, byte x of that stream in
    # piece x // P at 64 P (x // P) + P lane + x % P; then (scale | bias << 16) words
    rng = np.random.default_rng(bits)
    tb = 256 * bits + 128
    P = 16 if bits % 4 == 0 else (8 if bits % 2 == 0 else 4)
    for _ in range(200):
        n, k = int(rng.integers(N)), int(rng.integers(K))
        p, c, t = n // 16, n % 16, k // 128
        i, o, j = (k % 128) // 32, (k % 32) // 8, k % 8
        lane = 16 * o + c
        tile = (p * nt + t) * tb
        at = lambda x: tile + 64 * P * (x // P) + P * lane + x % P
        bit = 8 * bits * i + bits * j
        val = sum(((int(packed[at((bit + x) // 8)]) >> ((bit + x) % 8)) & 1) << x for x in range(bits))
        assert val == q[n, k]
        g = k // 64
        off = (p * nt + t) * tb + 256 * bits + (c * 2 + g % 2) * 4
        assert int(packed[off]) | int(packed[off + 1]) << 8 == s[n, g]
        assert int(packed[off + 2]) | int(packed[off + 3]) << 8 == b[n, g]


def test_affine_bits_refusals_without_gpu():
    lib = q4.raw()
    buf = (C.c_uint8 * 4096)()
    p = C.c_void_p((C.addressof(buf) + 15) & ~15)
    assert lib.q4_affine_bits_packed_bytes(16, 64, 4) == 0
    assert lib.qgemm_affine_bits(p, p, 1, 64, 16, 4, p, q4.Q4_F32, None) == q4.Q4_ERR_UNSUPPORTED
    assert lib.qgemm_affine_bits(p, p, 17, 64, 16, 2, p, q4.Q4_F32, None) == q4.Q4_ERR_UNSUPPORTED
    assert lib.qgemm_affine_bits(p, p, 1, 96, 16, 2, p, q4.Q4_F32, None) == q4.Q4_ERR_UNSUPPORTED
    assert lib.qgemm_affine_bits(p, p, 1, 64, 16, 2, p, q4.Q4_F16, None) == q4.Q4_ERR_INVALID_ARG
    codes = np.full((16, 64), 4, np.uint8)
    with pytest.raises(q4.Q4Error):
        q4.q4_affine_bits_repack(codes, np.zeros((16, 1), np.uint16), np.zeros((16, 1), np.uint16), 2)


def test_moe_block_refusals_without_gpu():
    lib = q4.raw()
    buf = (C.c_uint8 * 8192)()
    al = (C.addressof(buf) + 255) & ~255
    p = C.c_void_p(al)
    exp = q4.q4_moe_desc(8, 0, 256, 64, p, p, p, p, p, p)
    dense = q4.q4_moe_desc(1, 0, 256, 128, p, p, p, p, p, p)
    d = q4.q4_moe_block_desc(exp, dense, p, p, None, p, p, p, p, p, 1e-6)
    wsb = lib.moe_block_workspace_bytes(C.byref(d), 4, 2)
    assert wsb > 32768

    def call(desc, T=4, k=2, ws=p, nb=wsb, idx=None, w=None):
        return lib.moe_block_forward(C.byref(desc), p, T, k, idx, w, ws, nb, None)

    bad_eps = q4.q4_moe_block_desc(exp, dense, p, p, None, p, p, p, p, p, 0.0)
    assert call(bad_eps) == q4.Q4_ERR_INVALID_ARG and "eps" in _err(0)
    shared = q4.q4_moe_desc(8, 1, 256, 64, p, p, p, p, p, p)
    assert call(q4.q4_moe_block_desc(shared, dense, p, p, None, p, p, p, p, p, 1e-6)) == q4.Q4_ERR_INVALID_ARG
    two = q4.q4_moe_desc(2, 0, 256, 128, p, p, p, p, p, p)
    assert call(q4.q4_moe_block_desc(exp, two, p, p, None, p, p, p, p, p, 1e-6)) == q4.Q4_ERR_INVALID_ARG
    other_d = q4.q4_moe_desc(1, 0, 512, 128, p, p, p, p, p, p)
    assert call(q4.q4_moe_block_desc(exp, other_d, p, p, None, p, p, p, p, p, 1e-6)) == q4.Q4_ERR_INVALID_ARG
    assert call(q4.q4_moe_block_desc(exp, dense, p, None, None, p, p, p, p, p, 1e-6)) == q4.Q4_ERR_INVALID_ARG
    assert call(d, T=17) == q4.Q4_ERR_UNSUPPORTED
    assert call(d, ws=None) == q4.Q4_ERR_WORKSPACE
    assert call(d, nb=wsb - 1) == q4.Q4_ERR_WORKSPACE
    big = q4.q4_moe_desc(8, 0, 8192, 64, p, p, p, p, p, p)
    bigd = q4.q4_moe_desc(1, 0, 8192, 128, p, p, p, p, p, p)
    assert call(q4.q4_moe_block_desc(big, bigd, p, p, None, p, p, p, p, p, 1e-6)) == q4.Q4_ERR_UNSUPPORTED


def test_moe_block_refuses_downstream_shapes_before_any_launch():
    # conditions that only the router or the grouped MoE check: the block must
    # refuse them before its first launch (without a GPU, a launch would
    # surface as Q4_ERR_HIP instead)
    lib = q4.raw()
    buf = (C.c_uint8 * 8192)()
    p = C.c_void_p((C.addressof(buf) + 255) & ~255)
    odd = C.c_void_p(p.value + 4)

    def blk(E=8, D=256, F=64, Fd=128):
        return q4.q4_moe_block_desc(q4.q4_moe_desc(E, 0, D, F, p, p, p, p, p, p),
                                    q4.q4_moe_desc(1, 0, D, Fd, p, p, p, p, p, p), p, p, None, p, p, p, p, p, 1e-6)

    def call(desc, T=4, k=2, idx=None, w=None):
        return lib.moe_block_forward(C.byref(desc), p, T, k, idx, w, p, 1 << 30, None)

    cases = [
        (lambda: call(blk(E=32), k=17), q4.Q4_ERR_UNSUPPORTED, "k=17"),
        (lambda: call(blk(E=8), k=9), q4.Q4_ERR_UNSUPPORTED, "k=9"),
        (lambda: call(blk(), k=0), q4.Q4_ERR_INVALID_ARG, "k=0"),
        (lambda: call(blk(), k=-3), q4.Q4_ERR_INVALID_ARG, "k=-3"),
        (lambda: call(blk(), T=0), q4.Q4_ERR_INVALID_ARG, "T=0"),
        (lambda: call(blk(D=2824)), q4.Q4_ERR_UNSUPPORTED, "D=2824"),
        (lambda: call(blk(D=260)), q4.Q4_ERR_UNSUPPORTED, "D=260"),
        (lambda: call(blk(F=700)), q4.Q4_ERR_UNSUPPORTED, "F=700"),
        (lambda: call(blk(Fd=100)), q4.Q4_ERR_UNSUPPORTED, "F=100"),
        (lambda: call(blk(E=300)), q4.Q4_ERR_UNSUPPORTED, "E=300"),
        (lambda: call(blk(), idx=odd), q4.Q4_ERR_ALIGNMENT, "topk_idx_out"),
    ]
    for fn, code, needle in cases:
        assert fn() == code, needle
        assert needle in _err(code), (needle, _err(code))
    assert lib.moe_block_workspace_bytes(C.byref(blk()), 4, -3) == 0
    nulls = q4.q4_moe_block_desc(q4.q4_moe_desc(8, 0, 256, 64, None, p, p, p, p, p),
                                 q4.q4_moe_desc(1, 0, 256, 128, p, p, p, p, p, p), p, p, None, p, p, p, p, p, 1e-6)
    assert call(nulls) == q4.Q4_ERR_INVALID_ARG


def test_dynamic_lds_limit_setup_is_thread_safe():
    # launchers on many host threads at once: every call must either be
    # refused on the host or fail at its launch for lack of a GPU, never
    # with another thread's error (this host has no device, so each launch
    # reports Q4_ERR_HIP; what is checked is that the calls run concurrently
    # without corrupting the library's state)
    import threading
    lib = q4.raw()
    buf = (C.c_uint8 * 65536)()
    p = C.c_void_p((C.addressof(buf) + 255) & ~255)
    out = []

    def worker(M):
        for _ in range(50):
            out.append(lib.qgemm_affine4(p, p, M, 5120, 15360, p, q4.Q4_F32, p, 1 << 30, None))

    th = [threading.Thread(target=worker, args=(m,)) for m in (1, 4, 16, 8)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert len(out) == 200 and set(out) <= {q4.Q4_ERR_HIP, q4.Q4_OK}
