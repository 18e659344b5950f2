"""Python binding of libq4mi (W4A16 skinny GEMM and top-k MoE for MI355X).

Argument marshalling only: every function below forwards to the C entry point
of the same name in ``libq4mi.so`` (declared in ``include/q4mi.h``), passing
tensor data pointers, sizes and ``torch.cuda.current_stream()``.  Device
memory comes from torch; all arithmetic happens in the library's HIP kernels
(GPU entry points) or its C++ host code (repack).  If the shared library is
missing, importing this package raises: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq4mi.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python moe_w4a16_skinny_amd/build.py` "
                      "from the repository root (or __graft_entry__.build()) before using the library")
_lib = C.CDLL(LIB_PATH)

Q4_OK, Q4_ERR_INVALID_ARG, Q4_ERR_UNSUPPORTED, Q4_ERR_ALIGNMENT, Q4_ERR_WORKSPACE, Q4_ERR_HIP = 0, -1, -2, -3, -4, -5
Q4_F16, Q4_BF16, Q4_F32 = 1, 2, 3

_vp, _i64, _i32, _sz, _f32 = C.c_void_p, C.c_int64, C.c_int, C.c_size_t, C.c_float


class q4_moe_desc(C.Structure):
    _fields_ = [("E", C.c_int), ("has_shared", C.c_int), ("D", C.c_int), ("F", C.c_int),
                ("gate_packed", _vp), ("up_packed", _vp), ("down_packed", _vp),
                ("g_gate", _vp), ("g_up", _vp), ("g_down", _vp)]


class q4_moe_block_desc(C.Structure):
    _fields_ = [("experts", q4_moe_desc), ("dense", q4_moe_desc), ("w_router", _vp), ("router_scale", _vp),
                ("down_scale", _vp), ("ffn_norm", _vp), ("post_ffw_norm_1", _vp), ("pre_ffw_norm_2", _vp),
                ("post_ffw_norm_2", _vp), ("post_ffw_norm", _vp), ("eps", _f32)]


_SIGS = {
    "q4_abi_version": (_i32, []),
    "q4_last_error": (C.c_char_p, []),
    "q4_nvfp4_packed_bytes": (_sz, [_i64, _i64]),
    "q4_nvfp4_repack": (_i32, [_vp, _vp, _i64, _i64, _vp, _sz]),
    "q4_nvfp4_unpack": (_i32, [_vp, _i64, _i64, _vp, _vp]),
    "q4_affine4_packed_bytes": (_sz, [_i64, _i64]),
    "q4_affine4_repack": (_i32, [_vp, _vp, _vp, _i64, _i64, _vp, _sz]),
    "q4_affine4_unpack": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "qgemm_nvfp4_workspace_bytes": (_sz, [_i32, _i64, _i64, _i32]),
    "qgemm_nvfp4": (_i32, [_vp, _f32, _vp, _i32, _i64, _i64, _vp, _i32, _vp, _vp, _sz, _vp]),
    "qgemm_nvfp4_sample": (_i32, [_vp, _f32, _vp, _i32, _i64, _i64, _f32, _f32, C.c_uint64, C.c_uint32, _vp, _i32,
                                  _vp, _vp, _sz, _vp]),
    "q4_sample_uniforms": (_i32, [C.c_uint64, C.c_uint32, _i32, _i64, _vp, _vp]),
    "q4_nvfp4_quantize_workspace_bytes": (_sz, []),
    "q4_nvfp4_quantize": (_i32, [_vp, _i64, _i64, _f32, _vp, _sz, _vp, _vp, _sz, _vp]),
    "qgemm_affine4_workspace_bytes": (_sz, [_i32, _i64, _i64]),
    "qgemm_affine4": (_i32, [_vp, _vp, _i32, _i64, _i64, _vp, _i32, _vp, _sz, _vp]),
    "moe_route_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_route_topk": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_workspace_bytes": (_sz, [C.POINTER(q4_moe_desc), _i32, _i32]),
    "moe_grouped_qgemm": (_i32, [C.POINTER(q4_moe_desc), _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _sz, _vp]),
    "moe_grouped_qgemm_noalloc": (_i32, [C.POINTER(q4_moe_desc), _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp]),
    "moe_route_grouped_workspace_bytes": (_sz, [C.POINTER(q4_moe_desc), _i32, _i32]),
    "moe_route_grouped_qgemm": (_i32, [C.POINTER(q4_moe_desc), _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32,
                                       _vp, _sz, _vp]),
    "q4_affine_bits_packed_bytes": (_sz, [_i64, _i64, _i32]),
    "q4_affine_bits_repack": (_i32, [_vp, _vp, _vp, _i64, _i64, _i32, _vp, _sz]),
    "q4_affine_bits_unpack": (_i32, [_vp, _i64, _i64, _i32, _vp, _vp, _vp]),
    "qgemm_affine_bits": (_i32, [_vp, _vp, _i32, _i64, _i64, _i32, _vp, _i32, _vp]),
    "moe_block_workspace_bytes": (_sz, [C.POINTER(q4_moe_block_desc), _i32, _i32]),
    "moe_block_forward": (_i32, [C.POINTER(q4_moe_block_desc), _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "q4_dequant_nvfp4": (_i32, [_vp, _f32, _i64, _i64, _vp, _vp]),
    "q4_dequant_affine4": (_i32, [_vp, _i64, _i64, _vp, _vp]),
    "q4_stream_read": (_i32, [_vp, _sz, _i32, _i32, _i32, _vp, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class Q4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def _check(status: int):
    if status != Q4_OK:
        raise Q4Error(status, _lib.q4_last_error().decode())


def abi_version() -> int:
    return _lib.q4_abi_version()


def raw():
    """The ctypes handle of libq4mi.so (for tests that call the C ABI directly)."""
    return _lib


# ---------------------------------------------------------------- host repack

def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(_vp)


def q4_nvfp4_packed_bytes(N: int, K: int) -> int:
    return _lib.q4_nvfp4_packed_bytes(N, K)


def q4_nvfp4_repack(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    N, K = codes.shape[0], codes.shape[1] * 2
    if scales.shape != (N, K // 16):
        raise ValueError("scales must be [N][K/16]")
    nb = _lib.q4_nvfp4_packed_bytes(N, K)
    out = np.empty(max(nb, 1), np.uint8)
    _check(_lib.q4_nvfp4_repack(_np_ptr(codes), _np_ptr(scales), N, K, _np_ptr(out), nb))
    return out[:nb]


def q4_nvfp4_unpack(packed: np.ndarray, N: int, K: int):
    packed = np.ascontiguousarray(packed, np.uint8)
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.zeros((N, K // 16), np.uint8)
    _check(_lib.q4_nvfp4_unpack(_np_ptr(packed), N, K, _np_ptr(codes), _np_ptr(scales)))
    return codes, scales


def q4_affine4_packed_bytes(N: int, K: int) -> int:
    return _lib.q4_affine4_packed_bytes(N, K)


def q4_affine4_repack(codes: np.ndarray, scale_bf16: np.ndarray, bias_bf16: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    s = np.ascontiguousarray(scale_bf16, np.uint16)
    b = np.ascontiguousarray(bias_bf16, np.uint16)
    N, K = codes.shape[0], codes.shape[1] * 2
    if s.shape != (N, K // 64) or b.shape != (N, K // 64):
        raise ValueError("scale/bias must be [N][K/64]")
    nb = _lib.q4_affine4_packed_bytes(N, K)
    out = np.empty(max(nb, 1), np.uint8)
    _check(_lib.q4_affine4_repack(_np_ptr(codes), _np_ptr(s), _np_ptr(b), N, K, _np_ptr(out), nb))
    return out[:nb]


def q4_affine4_unpack(packed: np.ndarray, N: int, K: int):
    packed = np.ascontiguousarray(packed, np.uint8)
    codes = np.zeros((N, K // 2), np.uint8)
    s = np.zeros((N, K // 64), np.uint16)
    b = np.zeros((N, K // 64), np.uint16)
    _check(_lib.q4_affine4_unpack(_np_ptr(packed), N, K, _np_ptr(codes), _np_ptr(s), _np_ptr(b)))
    return codes, s, b


# ---------------------------------------------------------------- device calls

def _torch():
    import torch
    return torch


def _stream():
    return _vp(_torch().cuda.current_stream().cuda_stream)


def _tptr(t):
    return None if t is None else _vp(t.data_ptr())


_DT = {}


def _dtype_code(dt) -> int:
    torch = _torch()
    if not _DT:
        _DT.update({torch.float16: Q4_F16, torch.bfloat16: Q4_BF16, torch.float32: Q4_F32})
    return _DT[dt]


def to_device(arr: np.ndarray, device="cuda"):
    """Copy a host array (any dtype) into a new device tensor with the same bytes."""
    torch = _torch()
    arr = np.ascontiguousarray(arr)
    t = torch.from_numpy(arr.view(np.uint8).reshape(-1).copy())
    return t.to(device)


_WS = {}


def workspace(nbytes: int, device=None):
    """A zero-filled device workspace shared by calls on this device (grown on demand).

    The library leaves every workspace zero-filled when a call completes, so
    one buffer serves all calls issued in stream order."""
    torch = _torch()
    dev = torch.device(device if device is not None else "cuda")
    if dev.index is None:
        dev = torch.device(dev.type, torch.cuda.current_device())
    key = (dev.type, dev.index)
    cur = _WS.get(key)
    if cur is None or cur.numel() < nbytes:
        cur = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _WS[key] = cur
    return cur


def qgemm_nvfp4(w_packed, global_scale: float, a, N: int, out=None, out_dtype=None, want_argmax=False):
    """y = a . W^T for NVFP4 W [N][K] packed on the device; a f16 [M][K].

    Returns ``out`` (and the int32 argmax per row if ``want_argmax``)."""
    torch = _torch()
    M, K = a.shape
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a.device)
    amax = torch.empty((16,), dtype=torch.int32, device=a.device) if want_argmax else None
    wsb = _lib.qgemm_nvfp4_workspace_bytes(M, K, N, 1 if want_argmax else 0)
    ws = workspace(wsb, a.device) if wsb else None
    _check(_lib.qgemm_nvfp4(_tptr(w_packed), float(global_scale), _tptr(a), M, K, N, _tptr(out),
                            _dtype_code(out.dtype), _tptr(amax), _tptr(ws), wsb, _stream()))
    return (out, amax[:M]) if want_argmax else out


def qgemm_nvfp4_sample(w_packed, global_scale: float, a, N: int, softcap: float = 0.0, temperature: float = 0.0,
                       seed: int = 0, offset: int = 0, want_logits: bool = True, out_dtype=None):
    """lm_head with fused sampling: (logits z [M][N] or None, token int32 [M]).

    z = softcap * tanh(y / softcap) (softcap > 0); token = argmax(z / T + Gumbel
    noise) for T > 0, argmax z for T = 0."""
    torch = _torch()
    M, K = a.shape
    out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a.device) if want_logits else None
    tok = torch.empty((16,), dtype=torch.int32, device=a.device)
    wsb = _lib.qgemm_nvfp4_workspace_bytes(M, K, N, 1)
    ws = workspace(wsb, a.device)
    _check(_lib.qgemm_nvfp4_sample(_tptr(w_packed), float(global_scale), _tptr(a), M, K, N, float(softcap),
                                   float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFF,
                                   _tptr(out), _dtype_code(out.dtype if out is not None else torch.float32),
                                   _tptr(tok), _tptr(ws), wsb, _stream()))
    return out, tok[:M]


def q4_sample_uniforms(seed: int, offset: int, M: int, N: int, device=None):
    """The uniforms U[M][N] (fp32) that qgemm_nvfp4_sample draws (test export)."""
    torch = _torch()
    out = torch.empty((M, N), dtype=torch.float32, device=device or "cuda")
    _check(_lib.q4_sample_uniforms(int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFF, M, N, _tptr(out),
                                   _stream()))
    return out


def q4_nvfp4_quantize(w, global_scale: float = 0.0, packed=None):
    """NVFP4-quantize fp32 weights w [N][K] on the device into the packed layout.

    global_scale <= 0 takes g = amax|w| / (448 * 6).  Returns (packed uint8
    tensor of q4_nvfp4_packed_bytes(N, K), g as a float32 tensor [1])."""
    torch = _torch()
    if w.dtype != torch.float32 or not w.is_contiguous() or w.dim() != 2:
        raise ValueError("w must be a contiguous fp32 [N][K] tensor")
    N, K = w.shape
    nb = _lib.q4_nvfp4_packed_bytes(N, K)
    if packed is None:
        packed = torch.empty((max(nb, 1),), dtype=torch.uint8, device=w.device)
    g = torch.empty((1,), dtype=torch.float32, device=w.device)
    use_ws = not (float(global_scale) > 0.0)
    wsb = _lib.q4_nvfp4_quantize_workspace_bytes() if use_ws else 0
    ws = workspace(wsb, w.device) if use_ws else None
    _check(_lib.q4_nvfp4_quantize(_tptr(w), N, K, float(global_scale), _tptr(packed), packed.numel(), _tptr(g),
                                  _tptr(ws), wsb, _stream()))
    return packed[:nb], g


def qgemm_affine4(w_packed, a, N: int, out=None, out_dtype=None):
    """y = a . W^T for affine 4-bit W [N][K] packed on the device; a bf16 [M][K]."""
    torch = _torch()
    M, K = a.shape
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a.device)
    wsb = _lib.qgemm_affine4_workspace_bytes(M, K, N)
    ws = workspace(wsb, a.device) if wsb else None
    _check(_lib.qgemm_affine4(_tptr(w_packed), _tptr(a), M, K, N, _tptr(out), _dtype_code(out.dtype), _tptr(ws),
                              wsb, _stream()))
    return out


def moe_route_topk(x, w_router, k: int, renormalize: bool = False, want_logits: bool = True):
    """Router: (logits fp32 [T][E] or None, idx int32 [T][k], weights fp32 [T][k])."""
    torch = _torch()
    T, D = x.shape
    E = w_router.shape[1]
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if want_logits else None
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    wsb = _lib.moe_route_workspace_bytes(T, D, E)
    ws = workspace(wsb, x.device)
    _check(_lib.moe_route_topk(_tptr(x), _tptr(w_router), T, D, E, k, int(bool(renormalize)), _tptr(logits),
                               _tptr(idx), _tptr(w), _tptr(ws), wsb, _stream()))
    return logits, idx, w


@dataclass
class MoeWeights:
    """Device-resident expert weights of one MoE layer (see q4_moe_desc)."""
    E: int
    has_shared: bool
    D: int
    F: int
    gate: object   # uint8 device tensors: packed matrices, expert after expert
    up: object
    down: object
    g_gate: object  # fp32 device tensors [E + has_shared]
    g_up: object
    g_down: object

    def desc(self) -> q4_moe_desc:
        return q4_moe_desc(self.E, int(self.has_shared), self.D, self.F, self.gate.data_ptr(), self.up.data_ptr(),
                           self.down.data_ptr(), self.g_gate.data_ptr(), self.g_up.data_ptr(),
                           self.g_down.data_ptr())


def moe_pack_experts(gate, up, down, E: int, has_shared: bool, device="cuda") -> MoeWeights:
    """Repack per-expert canonical NVFP4 (codes, scales, g) triples with q4_nvfp4_repack
    and upload them expert after expert."""
    torch = _torch()
    F, D = gate[0][0].shape[0], gate[0][0].shape[1] * 2
    blobs = []
    for mats in (gate, up, down):
        blobs.append(np.concatenate([q4_nvfp4_repack(c, s) for (c, s, _) in mats]))
    gs = [np.array([float(g) for (_, _, g) in mats], np.float32) for mats in (gate, up, down)]
    return MoeWeights(E, has_shared, D, F, *(to_device(b, device) for b in blobs),
                      *(torch.from_numpy(g).to(device) for g in gs))


def moe_grouped_qgemm(weights: MoeWeights, x, topk_idx, topk_w, out=None, out_dtype=None):
    """Grouped MoE layer: y [T][D] = sum_j w * FFN_idx(x) + FFN_shared(x)."""
    torch = _torch()
    T, D = x.shape
    k = topk_idx.shape[1]
    if out is None:
        out = torch.empty((T, D), dtype=out_dtype or torch.float32, device=x.device)
    d = weights.desc()
    wsb = _lib.moe_workspace_bytes(C.byref(d), T, k)
    ws = workspace(wsb, x.device)
    _check(_lib.moe_grouped_qgemm(C.byref(d), _tptr(x), _tptr(topk_idx), _tptr(topk_w), T, k, _tptr(out),
                                  _dtype_code(out.dtype), _tptr(ws), wsb, _stream()))
    return out


def moe_grouped_qgemm_noalloc(weights: MoeWeights, x, topk_idx, topk_w, out):
    """moe_grouped_qgemm with the library's per-device scratch array instead of
    a workspace (no allocation in the call; `out` must be given)."""
    T, D = x.shape
    k = topk_idx.shape[1]
    d = weights.desc()
    _check(_lib.moe_grouped_qgemm_noalloc(C.byref(d), _tptr(x), _tptr(topk_idx), _tptr(topk_w), T, k, _tptr(out),
                                          _dtype_code(out.dtype), _stream()))
    return out


def moe_route_grouped_qgemm(weights: MoeWeights, x, w_router, k: int, renormalize: bool = False,
                            want_logits: bool = False, out=None, out_dtype=None, ws=None):
    """Router and grouped MoE layer in one call: (y [T][D], logits or None, idx [T][k], weights [T][k]).
    ws: an optional zero-filled workspace of at least moe_route_grouped_workspace_bytes."""
    torch = _torch()
    T, D = x.shape
    E = w_router.shape[1]
    if out is None:
        out = torch.empty((T, D), dtype=out_dtype or torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if want_logits else None
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    d = weights.desc()
    wsb = _lib.moe_route_grouped_workspace_bytes(C.byref(d), T, k)
    if ws is None:
        ws = workspace(wsb, x.device)
    _check(_lib.moe_route_grouped_qgemm(C.byref(d), _tptr(x), _tptr(w_router), T, k, int(bool(renormalize)),
                                        _tptr(logits), _tptr(idx), _tptr(w), _tptr(out), _dtype_code(out.dtype),
                                        _tptr(ws), ws.numel() if ws is not None else 0, _stream()))
    return out, logits, idx, w


def q4_dequant_nvfp4(w_packed, global_scale: float, N: int, K: int):
    torch = _torch()
    out = torch.empty((N, K), dtype=torch.float32, device=w_packed.device)
    _check(_lib.q4_dequant_nvfp4(_tptr(w_packed), float(global_scale), N, K, _tptr(out), _stream()))
    return out


def q4_dequant_affine4(w_packed, N: int, K: int):
    torch = _torch()
    out = torch.empty((N, K), dtype=torch.float32, device=w_packed.device)
    _check(_lib.q4_dequant_affine4(_tptr(w_packed), N, K, _tptr(out), _stream()))
    return out


@dataclass
class MoeBlockWeights:
    """Device-resident Gemma-4 MoE block (see q4_moe_block_desc)."""
    experts: MoeWeights
    dense: MoeWeights
    w_router: object      # fp32 device tensors
    router_scale: object
    down_scale: object
    norms: tuple          # ffn_norm, post_ffw_norm_1, pre_ffw_norm_2, post_ffw_norm_2, post_ffw_norm
    eps: float = 1e-6

    def desc(self) -> q4_moe_block_desc:
        n = [t.data_ptr() for t in self.norms]
        return q4_moe_block_desc(self.experts.desc(), self.dense.desc(), self.w_router.data_ptr(),
                                 self.router_scale.data_ptr(),
                                 self.down_scale.data_ptr() if self.down_scale is not None else None,
                                 *n, float(self.eps))


def moe_block_pack(blk, eps: float = 1e-6, device="cuda") -> MoeBlockWeights:
    """Upload a block given as canonical NVFP4 triples and fp32 vectors (the
    fields of a MoeBlockInputs-like object)."""
    torch = _torch()
    experts = moe_pack_experts(blk.gate, blk.up, blk.down, blk.E, False, device)
    dense = moe_pack_experts([blk.dense_gate], [blk.dense_up], [blk.dense_down], 1, False, device)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    norms = tuple(f(v) for v in (blk.ffn_norm, blk.post_ffw_norm_1, blk.pre_ffw_norm_2, blk.post_ffw_norm_2,
                                 blk.post_ffw_norm))
    return MoeBlockWeights(experts, dense, f(blk.w_router), f(blk.router_scale),
                           f(blk.down_scale) if blk.down_scale is not None else None, norms, eps)


def moe_block_forward(block: MoeBlockWeights, residual, k: int, want_routing: bool = False):
    """One MoE block on the residual stream (fp32 [T][D] device tensor), in place; returns it,
    or (residual, topk_idx int32 [T][k], topk_w fp32 [T][k]) with want_routing."""
    torch = _torch()
    if residual.dtype != torch.float32 or not residual.is_contiguous():
        raise ValueError("residual must be a contiguous fp32 [T][D] tensor")
    T = residual.shape[0]
    d = block.desc()
    wsb = _lib.moe_block_workspace_bytes(C.byref(d), T, k)
    ws = workspace(wsb, residual.device)
    idx = w = None
    if want_routing:
        idx = torch.empty((T, max(k, 1)), dtype=torch.int32, device=residual.device)
        w = torch.empty((T, max(k, 1)), dtype=torch.float32, device=residual.device)
    _check(_lib.moe_block_forward(C.byref(d), _tptr(residual), T, k, _tptr(idx), _tptr(w), _tptr(ws), wsb,
                                  _stream()))
    return (residual, idx, w) if want_routing else residual


def q4_affine_bits_repack(codes: np.ndarray, scale_bf16: np.ndarray, bias_bf16: np.ndarray, bits: int) -> np.ndarray:
    """codes u8 [N][K] (one per byte), scale/bias bf16 bits [N][K/64] -> packed b-bit layout."""
    codes = np.ascontiguousarray(codes, np.uint8)
    s = np.ascontiguousarray(scale_bf16, np.uint16)
    b = np.ascontiguousarray(bias_bf16, np.uint16)
    N, K = codes.shape
    nb = _lib.q4_affine_bits_packed_bytes(N, K, bits)
    out = np.empty(max(nb, 1), np.uint8)
    _check(_lib.q4_affine_bits_repack(_np_ptr(codes), _np_ptr(s), _np_ptr(b), N, K, bits, _np_ptr(out), nb))
    return out[:nb]


def q4_affine_bits_unpack(packed: np.ndarray, N: int, K: int, bits: int):
    packed = np.ascontiguousarray(packed, np.uint8)
    codes = np.zeros((N, K), np.uint8)
    s = np.zeros((N, K // 64), np.uint16)
    b = np.zeros((N, K // 64), np.uint16)
    _check(_lib.q4_affine_bits_unpack(_np_ptr(packed), N, K, bits, _np_ptr(codes), _np_ptr(s), _np_ptr(b)))
    return codes, s, b


def qgemm_affine_bits(w_packed, a, N: int, bits: int, out=None, out_dtype=None):
    """y = a . W^T for affine b-bit W [N][K] (bits 2, 3, 5, 6, 8) packed on the device; a bf16 [M][K]."""
    torch = _torch()
    M, K = a.shape
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a.device)
    _check(_lib.qgemm_affine_bits(_tptr(w_packed), _tptr(a), M, K, N, int(bits), _tptr(out), _dtype_code(out.dtype),
                                  _stream()))
    return out
