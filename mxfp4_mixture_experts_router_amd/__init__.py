"""GPT-OSS MXFP4 mixture-of-experts layer for MI355X (gfx950).

Thin ctypes binding over the C-ABI library ``libmoe_mxfp4.so`` (declared in
``include/moe_mxfp4.h``). This module only marshals arguments: it checks dtypes,
shapes, devices and contiguity of torch tensors, allocates outputs and the
workspace with the torch caching allocator, and passes raw device pointers and
the current HIP stream to the library. Every step of the layer runs in the
library's HIP kernels; there is no Python or CPU fallback. If the library is not
built, every call raises ``MoeLibraryMissing``.

Tensor conventions (all device tensors, row-major, contiguous):
  x [T, H] bf16; router_w [E, H] bf16; router_b [E] bf16;
  gu_blocks [E, 2I, H/2] uint8; gu_scales [E, 2I, H/32] uint8; gu_bias [E, 2I] bf16;
  dn_blocks [E, H, I/2] uint8;  dn_scales [E, H, I/32] uint8;  dn_bias [E, H] bf16.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "MoeError", "MoeLibraryMissing", "library_path", "load_library", "abi_version",
    "workspace_bytes", "moe_forward", "route", "permute", "expert_up", "expert_down",
    "combine", "dequant", "permute_workspace_bytes", "DECODE_MAX_T", "DECODE_MAX_K", "uses_decode_path", "mx8_bytes",
    "quantize_act", "quantize_h", "rmsnorm", "moe_forward_dequantized", "dequantize_bank", "workspace_bytes_dequantized",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmoe_mxfp4.so")
_lib = None

DECODE_MAX_T = 64
DECODE_MAX_K = 4096


def uses_decode_path(T, H, I):
    """Whether moe_forward takes the few-token path (3 launches below 4 tokens, 4 from 4 to 64
    tokens; no permutation)."""
    return T <= DECODE_MAX_T and H <= DECODE_MAX_K and I <= DECODE_MAX_K

MAX_LAUNCHES = 6

STATUS = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_ESHAPE", 3: "MOE_EALIGN", 4: "MOE_EWORKSPACE",
          5: "MOE_EHIP"}


class MoeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


class MoeLibraryMissing(RuntimeError):
    pass


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("swiglu_alpha", ctypes.c_float), ("swiglu_limit", ctypes.c_float)]


_vp = ctypes.c_void_p
_SIGS = {
    "moe_mxfp4_abi_version": (ctypes.c_int, []),
    "moe_mxfp4_clock_probe": (ctypes.c_int, [_vp, ctypes.c_int, ctypes.c_int, _vp]),
    "moe_mxfp4_last_error": (ctypes.c_char_p, []),
    "moe_mxfp4_check_shape": (ctypes.c_int, [ctypes.POINTER(Shape)]),
    "moe_mxfp4_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_size_t)]),
    "moe_mxfp4_forward": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 13 + [ctypes.c_size_t, _vp]),
    "moe_mxfp4_forward_timed": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 13
                                + [ctypes.c_size_t, _vp, _vp, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]),
    "moe_mxfp4_forward_prenorm": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, _vp, ctypes.c_double]
                                  + [_vp] * 12 + [ctypes.c_size_t, _vp]),
    "moe_mxfp4_forward_prenorm_timed": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, _vp, ctypes.c_double]
                                        + [_vp] * 12 + [ctypes.c_size_t, _vp, _vp, ctypes.c_int,
                                                        ctypes.POINTER(ctypes.c_int)]),
    "moe_mxfp4_forward_dequantized": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 11
                                      + [ctypes.c_size_t, _vp]),
    "moe_mxfp4_forward_dequantized_timed": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 11
                                            + [ctypes.c_size_t, _vp, _vp, ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_int)]),
    "moe_mxfp4_workspace_bytes_dequantized": (ctypes.c_int, [ctypes.POINTER(Shape),
                                                             ctypes.POINTER(ctypes.c_size_t)]),
    "moe_mxfp4_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 12 + [_vp]),
    "moe_mxfp4_noalloc_max_bytes": (ctypes.c_size_t, []),
    "moe_mxfp4_rmsnorm": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, _vp, _vp]),
    "moe_mxfp4_route": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 7),
    "moe_mxfp4_permute": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 7),
    "moe_mxfp4_permute_ws": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 7 + [ctypes.c_size_t, _vp]),
    "moe_mxfp4_permute_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(Shape),
                                                         ctypes.POINTER(ctypes.c_size_t)]),
    "moe_mxfp4_expert_up": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 8),
    "moe_mxfp4_expert_down": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 8),
    "moe_mxfp4_combine": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 4),
    "moe_mxfp4_dequant": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp]),
    "moe_mxfp4_mx8_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32]),
    "moe_mxfp4_quantize_act": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp]),
    "moe_mxfp4_quantize_h": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp]),
}


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmoe_mxfp4.so (raises MoeLibraryMissing if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise MoeLibraryMissing(
            f"{_LIB_PATH} is not built; run `python -m mxfp4_mixture_experts_router_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def abi_version() -> int:
    return load_library().moe_mxfp4_abi_version()


def _check(status: int):
    if status != 0:
        msg = load_library().moe_mxfp4_last_error().decode(errors="replace")
        raise MoeError(status, msg)


def _shape(T, H, I, E, k, alpha=1.702, limit=7.0) -> Shape:
    return Shape(int(T), int(H), int(I), int(E), int(k), float(alpha), float(limit))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtypes, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)


def workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    out = ctypes.c_size_t(0)
    s = _shape(T, H, I, E, k)
    _check(load_library().moe_mxfp4_workspace_bytes(ctypes.byref(s), ctypes.byref(out)))
    return int(out.value)


def _dims(x, router_w, gu_blocks):
    T, H = x.shape
    E = router_w.shape[0]
    I = gu_blocks.shape[1] // 2
    return T, H, I, E


def moe_forward(x, router_w, router_b, gu_blocks, gu_scales, gu_bias, dn_blocks, dn_scales,
                dn_bias, k: int, alpha: float = 1.702, limit: float = 7.0, *,
                workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                return_topk: bool = False, norm_weight: Optional[torch.Tensor] = None,
                norm_eps: float = 1e-5, stream=None):
    """The whole layer. Returns y [T, H] bf16 (and (topk_idx, topk_w) if return_topk).

    With ``norm_weight`` ([H] bf16), the pre-norm block ``y = x + layer(rmsnorm(x))``
    (moe_mxfp4_forward_prenorm); the routing returned is that of the normalized rows."""
    T, H, I, E = _dims(x, router_w, gu_blocks)
    dev = x.device
    _need(x, "x", _BF16, (T, H), dev)
    if norm_weight is not None:
        _need(norm_weight, "norm_weight", _BF16, (H,), dev)
    _need(router_w, "router_w", _BF16, (E, H), dev)
    _need(router_b, "router_b", _BF16, (E,), dev)
    _need(gu_blocks, "gu_blocks", _U8, (E, 2 * I, H // 2), dev)
    _need(gu_scales, "gu_scales", _U8, (E, 2 * I, H // 32), dev)
    _need(gu_bias, "gu_bias", _BF16, (E, 2 * I), dev)
    _need(dn_blocks, "dn_blocks", _U8, (E, H, I // 2), dev)
    _need(dn_scales, "dn_scales", _U8, (E, H, I // 32), dev)
    _need(dn_bias, "dn_bias", _BF16, (E, H), dev)
    shape = _shape(T, H, I, E, k, alpha, limit)
    lib = load_library()
    nbytes = ctypes.c_size_t(0)
    _check(lib.moe_mxfp4_workspace_bytes(ctypes.byref(shape), ctypes.byref(nbytes)))
    if workspace is None:
        workspace = torch.empty(max(int(nbytes.value), 256), dtype=torch.uint8, device=dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if out is None else out
    _need(y, "out", _BF16, (T, H), dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev) if return_topk else None
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if return_topk else None
    tail = (_ptr(router_w), _ptr(router_b), _ptr(gu_blocks), _ptr(gu_scales), _ptr(gu_bias),
            _ptr(dn_blocks), _ptr(dn_scales), _ptr(dn_bias), _ptr(y), _ptr(idx), _ptr(w),
            _ptr(workspace), workspace.numel(), _stream(stream))
    if norm_weight is None:
        _check(lib.moe_mxfp4_forward(ctypes.byref(shape), _ptr(x), *tail))
    else:
        _check(lib.moe_mxfp4_forward_prenorm(ctypes.byref(shape), _ptr(x), _ptr(norm_weight),
                                             float(norm_eps), *tail))
    return (y, idx, w) if return_topk else y


def workspace_bytes_dequantized(T: int, H: int, I: int, E: int, k: int) -> int:
    out = ctypes.c_size_t(0)
    s = _shape(T, H, I, E, k)
    _check(load_library().moe_mxfp4_workspace_bytes_dequantized(ctypes.byref(s), ctypes.byref(out)))
    return int(out.value)


def dequantize_bank(gu_blocks, gu_scales, dn_blocks, dn_scales, stream=None, out=None):
    """The packed bank expanded once to bf16 (moe_mxfp4_dequant): (gu_w [E, 2I, H], dn_w [E, H, I]),
    written into the pair ``out`` when given."""
    gu_out, dn_out = out if out is not None else (None, None)
    return dequant(gu_blocks, gu_scales, stream, gu_out), dequant(dn_blocks, dn_scales, stream, dn_out)


def moe_forward_dequantized(x, router_w, router_b, gu_w, gu_bias, dn_w, dn_bias, k: int,
                            alpha: float = 1.702, limit: float = 7.0, *,
                            workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                            return_topk: bool = False, stream=None):
    """The layer on a bf16 bank from dequantize_bank (moe_mxfp4_forward_dequantized). Returns
    y [T, H] bf16 (and (topk_idx, topk_w) if return_topk)."""
    T, H = x.shape
    E, I2, _ = gu_w.shape
    I = I2 // 2
    dev = x.device
    _need(x, "x", _BF16, (T, H), dev)
    _need(router_w, "router_w", _BF16, (E, H), dev)
    _need(router_b, "router_b", _BF16, (E,), dev)
    _need(gu_w, "gu_w", _BF16, (E, 2 * I, H), dev)
    _need(gu_bias, "gu_bias", _BF16, (E, 2 * I), dev)
    _need(dn_w, "dn_w", _BF16, (E, H, I), dev)
    _need(dn_bias, "dn_bias", _BF16, (E, H), dev)
    shape = _shape(T, H, I, E, k, alpha, limit)
    lib = load_library()
    nbytes = ctypes.c_size_t(0)
    _check(lib.moe_mxfp4_workspace_bytes_dequantized(ctypes.byref(shape), ctypes.byref(nbytes)))
    if workspace is None:
        workspace = torch.empty(max(int(nbytes.value), 256), dtype=torch.uint8, device=dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if out is None else out
    _need(y, "out", _BF16, (T, H), dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev) if return_topk else None
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if return_topk else None
    _check(lib.moe_mxfp4_forward_dequantized(
        ctypes.byref(shape), _ptr(x), _ptr(router_w), _ptr(router_b), _ptr(gu_w), _ptr(gu_bias),
        _ptr(dn_w), _ptr(dn_bias), _ptr(y), _ptr(idx), _ptr(w), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return (y, idx, w) if return_topk else y


def route(x, router_w, router_b, k: int, return_logits: bool = False, stream=None):
    """Router + top-k + softmax. Returns (topk_idx int32 [T,k], topk_w fp32 [T,k][, logits fp32 [T,E]])."""
    T, H = x.shape
    E = router_w.shape[0]
    dev = x.device
    _need(x, "x", _BF16, (T, H), dev)
    _need(router_w, "router_w", _BF16, (E, H), dev)
    _need(router_b, "router_b", _BF16, (E,), dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if return_logits else None
    shape = _shape(T, H, 32, E, k)
    _check(load_library().moe_mxfp4_route(ctypes.byref(shape), _ptr(x), _ptr(router_w),
                                          _ptr(router_b), _ptr(idx), _ptr(w), _ptr(logits),
                                          _stream(stream)))
    return (idx, w, logits) if return_logits else (idx, w)


def permute_workspace_bytes(T: int, E: int, k: int) -> int:
    """Workspace bytes of the many-workgroup permutation (0: it runs on one workgroup)."""
    out = ctypes.c_size_t(0)
    s = _shape(T, 32, 32, E, k)
    _check(load_library().moe_mxfp4_permute_workspace_bytes(ctypes.byref(s), ctypes.byref(out)))
    return int(out.value)


def permute(topk_idx, topk_w, E: int, stream=None, multi_block: bool = False):
    """Expert-sorted permutation. Returns (offsets [E+1], sorted_token, sorted_weight, slot_row).

    ``multi_block``: the histogram (+ scan) + scatter passes the forward calls run
    (moe_mxfp4_permute_ws), instead of the one-workgroup kernel (moe_mxfp4_permute)."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    _need(topk_idx, "topk_idx", (torch.int32,), (T, k), dev)
    _need(topk_w, "topk_w", (torch.float32,), (T, k), dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_token = torch.empty(T * k, dtype=torch.int32, device=dev)
    sorted_w = torch.empty(T * k, dtype=torch.float32, device=dev)
    slot_row = torch.empty(T * k, dtype=torch.int32, device=dev)
    shape = _shape(T, 32, 32, E, k)
    if multi_block:
        nbytes = permute_workspace_bytes(T, E, k)
        ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=dev)
        _check(load_library().moe_mxfp4_permute_ws(ctypes.byref(shape), _ptr(topk_idx), _ptr(topk_w),
                                                   _ptr(offsets), _ptr(sorted_token), _ptr(sorted_w),
                                                   _ptr(slot_row), _ptr(ws), ws.numel(), _stream(stream)))
    else:
        _check(load_library().moe_mxfp4_permute(ctypes.byref(shape), _ptr(topk_idx), _ptr(topk_w),
                                                _ptr(offsets), _ptr(sorted_token), _ptr(sorted_w),
                                                _ptr(slot_row), _stream(stream)))
    return offsets, sorted_token, sorted_w, slot_row


def rmsnorm(x, norm_weight, eps: float = 1e-5, stream=None):
    """Pre-LN RMSNorm of the rows of x [R, C] bf16 with scale norm_weight [C] bf16: returns
    bf16(x * norm_weight / sqrt(mean(x^2) + eps)) [R, C] (moe_mxfp4_rmsnorm)."""
    R, C = x.shape
    dev = x.device
    _need(x, "x", _BF16, (R, C), dev)
    _need(norm_weight, "norm_weight", _BF16, (C,), dev)
    xn = torch.empty((R, C), dtype=torch.bfloat16, device=dev)
    _check(load_library().moe_mxfp4_rmsnorm(_ptr(x), _ptr(norm_weight), R, C, float(eps), _ptr(xn),
                                            _stream(stream)))
    return xn


def mx8_bytes(rows: int, cols: int) -> int:
    """Bytes of an mx8 activation matrix of rows x cols values (see moe_mxfp4.h)."""
    return int(load_library().moe_mxfp4_mx8_bytes(rows, cols))


def quantize_act(x, stream=None):
    """bf16 [R, K] -> mx8 matrix (flat uint8 tensor of mx8_bytes(R, K) bytes)."""
    R, K = x.shape
    dev = x.device
    _need(x, "x", _BF16, (R, K), dev)
    q8 = torch.empty(mx8_bytes(R, K), dtype=torch.uint8, device=dev)
    _check(load_library().moe_mxfp4_quantize_act(_ptr(x), R, K, _ptr(q8), _stream(stream)))
    return q8


def quantize_h(h, stream=None):
    """bf16 [R, K] -> h8 matrix (group-major scales; what expert_down takes), a flat uint8
    tensor of mx8_bytes(R, K) bytes."""
    R, K = h.shape
    dev = h.device
    _need(h, "h", _BF16, (R, K), dev)
    h8 = torch.empty(mx8_bytes(R, K), dtype=torch.uint8, device=dev)
    _check(load_library().moe_mxfp4_quantize_h(_ptr(h), R, K, _ptr(h8), _stream(stream)))
    return h8


def expert_up(x8, T: int, gu_blocks, gu_scales, gu_bias, offsets, sorted_token, k: int,
              alpha: float = 1.702, limit: float = 7.0, stream=None):
    """Grouped gate_up GEMM + SwiGLU over sorted rows, from x8 (mx8, T rows of H). Returns
    h8: the h8 matrix (group-major scales) of T*k rows of I (flat uint8)."""
    E, I2, Hh = gu_blocks.shape
    I, H = I2 // 2, 2 * Hh
    dev = gu_blocks.device
    _need(x8, "x8", _U8, (mx8_bytes(T, H),), dev)
    _need(gu_blocks, "gu_blocks", _U8, (E, 2 * I, H // 2), dev)
    _need(gu_scales, "gu_scales", _U8, (E, 2 * I, H // 32), dev)
    _need(gu_bias, "gu_bias", _BF16, (E, 2 * I), dev)
    _need(offsets, "offsets", (torch.int32,), (E + 1,), dev)
    _need(sorted_token, "sorted_token", (torch.int32,), (T * k,), dev)
    h8 = torch.empty(mx8_bytes(T * k, I), dtype=torch.uint8, device=dev)
    shape = _shape(T, H, I, E, k, alpha, limit)
    _check(load_library().moe_mxfp4_expert_up(ctypes.byref(shape), _ptr(x8), _ptr(gu_blocks),
                                               _ptr(gu_scales), _ptr(gu_bias), _ptr(offsets),
                                               _ptr(sorted_token), _ptr(h8), _stream(stream)))
    return h8


def expert_down(h8, T: int, dn_blocks, dn_scales, dn_bias, offsets, sorted_weight, k: int, stream=None):
    """Grouped down GEMM + bias, times the row's routing weight, from h8 (T*k rows of I, as
    expert_up or quantize_h write it).
    Returns o [T*k, H] fp32."""
    E, H, Ih = dn_blocks.shape
    I, N = 2 * Ih, T * k
    dev = dn_blocks.device
    _need(h8, "h8", _U8, (mx8_bytes(N, I),), dev)
    _need(dn_blocks, "dn_blocks", _U8, (E, H, I // 2), dev)
    _need(dn_scales, "dn_scales", _U8, (E, H, I // 32), dev)
    _need(dn_bias, "dn_bias", _BF16, (E, H), dev)
    _need(offsets, "offsets", (torch.int32,), (E + 1,), dev)
    _need(sorted_weight, "sorted_weight", (torch.float32,), (N,), dev)
    o = torch.empty((N, H), dtype=torch.float32, device=dev)
    shape = _shape(T, H, I, E, k)
    _check(load_library().moe_mxfp4_expert_down(ctypes.byref(shape), _ptr(h8), _ptr(dn_blocks),
                                                 _ptr(dn_scales), _ptr(dn_bias), _ptr(offsets),
                                                 _ptr(sorted_weight), _ptr(o), _stream(stream)))
    return o


def combine(o, slot_row, k: int, stream=None):
    """Un-permute + sum over the k slots. Returns y [T, H] bf16."""
    N, H = o.shape
    T = N // k
    dev = o.device
    _need(o, "o", (torch.float32,), (N, H), dev)
    _need(slot_row, "slot_row", (torch.int32,), (N,), dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    shape = _shape(T, H, 32, max(k, 1), k)
    _check(load_library().moe_mxfp4_combine(ctypes.byref(shape), _ptr(o), _ptr(slot_row), _ptr(y),
                                            _stream(stream)))
    return y


def dequant(blocks, scales, stream=None, out: Optional[torch.Tensor] = None):
    """MXFP4 -> bf16 for a packed [..., rows, cols/2] tensor. Returns [..., rows, cols] bf16
    (written into ``out`` when given)."""
    cols = blocks.shape[-1] * 2
    rows = blocks.numel() // (cols // 2) if blocks.numel() else 0
    dev = blocks.device
    _need(blocks, "blocks", _U8, None, dev)
    _need(scales, "scales", _U8, tuple(blocks.shape[:-1]) + (cols // 32,), dev)
    oshape = tuple(blocks.shape[:-1]) + (cols,)
    if out is None:
        out = torch.empty(oshape, dtype=torch.bfloat16, device=dev)
    _need(out, "out", _BF16, oshape, dev)
    _check(load_library().moe_mxfp4_dequant(_ptr(blocks), _ptr(scales), rows, cols, _ptr(out),
                                            _stream(stream)))
    return out
