"""CPU oracle for the GPT-OSS MXFP4 mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the benchmark's CPU-baseline leg, never by the product package. It is a
thin ctypes wrapper around ``oracle.c`` (plain C, IEEE double, built with gcc
without fast-math or FMA contraction). It shares no code with the HIP library.

Every function takes the host numpy arrays produced by ``workloads.make_inputs``
(bf16 as uint16 bit patterns, packed MXFP4 as uint8) and returns float64
results. See ``oracle.c`` for the page passages each step follows.

Two modes compute the whole layer:
* ``forward`` (brute mode): per token and per selected expert, every weight decoded inside
  the dot product that uses it, sums in index order (``oracle_forward_tokens``).
* ``forward_expert_major``: the ZeroModels GPT-OSS page's "dequantize the whole bank once"
  strategy ("MXFP4 experts"): the same routing, then each selected expert's weights are
  decoded once to double and applied to all of its routed tokens as float64 matrix products
  (a library matmul as the GEMM step), SwiGLU element by element, the weighted sum over the
  k slots in slot order. Only the summation order inside the dot products differs from the
  brute mode, so the two agree to double rounding; it is the mode that finishes the
  4096-token and 120B-shaped workloads in seconds.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = np.ctypeslib.ndpointer
_u8 = _P(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16 = _P(dtype=np.uint16, flags="C_CONTIGUOUS")
_i32 = _P(dtype=np.int32, flags="C_CONTIGUOUS")
_i64 = _P(dtype=np.int64, flags="C_CONTIGUOUS")
_f64 = _P(dtype=np.float64, flags="C_CONTIGUOUS")
_f64_or_null = ctypes.c_void_p


def build(force: bool = True, sanitize: bool = False, out: Optional[str] = None) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it (gcc, OpenMP). With ``sanitize``
    the build carries AddressSanitizer and UndefinedBehaviorSanitizer checks (every
    undefined-behaviour report is fatal) and goes to ``out``; a process loading it needs
    gcc's libasan and libubsan preloaded, and names the file in ORACLE_LIB."""
    lib = out or _LIB
    if force or not os.path.exists(lib):
        opt = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"])
        cmd = ["gcc", *opt, "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-fvisibility=hidden",
               _SRC, "-o", lib + ".tmp", "-lm"]
        subprocess.check_call(cmd)
        os.replace(lib + ".tmp", lib)
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("ORACLE_LIB")
    if path is None:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
    lib = ctypes.CDLL(path)
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_e2m1.restype = ctypes.c_double
    lib.oracle_e2m1.argtypes = [ctypes.c_int]
    lib.oracle_e8m0.restype = ctypes.c_double
    lib.oracle_e8m0.argtypes = [ctypes.c_int]
    lib.oracle_swiglu.restype = ctypes.c_double
    lib.oracle_swiglu.argtypes = [ctypes.c_double] * 4
    lib.oracle_dequant.restype = None
    lib.oracle_dequant.argtypes = [_u8, _u8, ctypes.c_int64, ctypes.c_int64, _f64]
    lib.oracle_router.restype = None
    lib.oracle_router.argtypes = [_u16, _u16, _u16, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                  _f64, _f64_or_null]
    lib.oracle_topk_softmax.restype = None
    lib.oracle_topk_softmax.argtypes = [_f64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _i32, _f64]
    lib.oracle_expert.restype = None
    lib.oracle_expert.argtypes = [_u16, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  _u8, _u8, _u16, _u8, _u8, _u16,
                                  ctypes.c_double, ctypes.c_double, _f64_or_null, _f64]
    lib.oracle_swiglu_n.restype = None
    lib.oracle_swiglu_n.argtypes = [_f64, _f64, ctypes.c_int64, ctypes.c_double, ctypes.c_double, _f64]
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    lib.oracle_bf16_round.argtypes = [ctypes.c_double]
    lib.oracle_rmsnorm.restype = None
    lib.oracle_rmsnorm.argtypes = [_u16, _u16, ctypes.c_int64, ctypes.c_int, ctypes.c_double, _u16,
                                   _f64_or_null]
    lib.oracle_forward_tokens.restype = None
    lib.oracle_forward_tokens.argtypes = [
        _i64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _u16, _u16, _u16, _u8, _u8, _u16, _u8, _u8, _u16,
        ctypes.c_double, ctypes.c_double,
        _f64, _f64_or_null, _i32, _f64, _f64_or_null, _f64_or_null, _f64]
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    """Threads the oracle's token-parallel loops use."""
    return _load().oracle_max_threads()


def e2m1(code: int) -> float:
    return _load().oracle_e2m1(int(code))


def e8m0(byte: int) -> float:
    return _load().oracle_e8m0(int(byte))


def swiglu(gate: float, up: float, alpha: float = 1.702, limit: float = 7.0) -> float:
    return _load().oracle_swiglu(float(gate), float(up), float(alpha), float(limit))


def dequant(blocks: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed ``[..., rows, cols/2]`` blocks + ``[..., rows, cols/32]`` scales -> float64 ``[..., rows, cols]``."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    cols = blocks.shape[-1] * 2
    rows = int(np.prod(blocks.shape[:-1]))
    if scales.shape[:-1] != blocks.shape[:-1] or scales.shape[-1] * 32 != cols:
        raise ValueError("blocks/scales shape mismatch")
    out = np.empty(blocks.shape[:-1] + (cols,), dtype=np.float64)
    _load().oracle_dequant(blocks.reshape(-1), scales.reshape(-1), rows, cols, out.reshape(-1))
    return out


def bf16_round(v: float) -> int:
    """The bf16 bit pattern nearest to ``v`` (ties to even)."""
    return int(_load().oracle_bf16_round(float(v)))


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float = 1e-5, with_exact: bool = False):
    """Pre-LN RMSNorm of bf16 rows ``x [T, H]`` with bf16 weights ``gamma [H]``: bf16 bit
    patterns ``[T, H]`` (and the values before rounding, when ``with_exact``)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    T, H = x.shape
    xn = np.empty((T, H), dtype=np.uint16)
    exact = np.empty((T, H), dtype=np.float64) if with_exact else None
    _load().oracle_rmsnorm(x, gamma, T, H, float(eps), xn, _ptr(exact))
    return (xn, exact) if with_exact else xn


def router(x, router_w, router_b, with_abs_sum: bool = False):
    T, H = x.shape
    E = router_w.shape[0]
    logits = np.empty((T, E), dtype=np.float64)
    abs_sum = np.empty((T, E), dtype=np.float64) if with_abs_sum else None
    _load().oracle_router(np.ascontiguousarray(x), np.ascontiguousarray(router_w),
                          np.ascontiguousarray(router_b), T, H, E, logits, _ptr(abs_sum))
    return (logits, abs_sum) if with_abs_sum else logits


def topk_softmax(logits: np.ndarray, k: int):
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    _load().oracle_topk_softmax(logits, T, E, k, idx, w)
    return idx, w


def expert(x_row, e: int, inp: Dict[str, np.ndarray], alpha=1.702, limit=7.0):
    """One expert on one bf16 token row; returns (h [I], o [H]) in float64."""
    H = inp["router_w"].shape[1]
    I = inp["dn_blocks"].shape[2] * 2
    h = np.empty(I, dtype=np.float64)
    o = np.empty(H, dtype=np.float64)
    _load().oracle_expert(np.ascontiguousarray(x_row), int(e), H, I, inp["gu_blocks"],
                          inp["gu_scales"], inp["gu_bias"], inp["dn_blocks"], inp["dn_scales"],
                          inp["dn_bias"], float(alpha), float(limit), _ptr(h), o)
    return h, o


def forward_prenorm(inp: Dict[str, np.ndarray], k: int, tokens: Optional[Sequence[int]] = None,
                    alpha: float = 1.702, limit: float = 7.0, eps: float = 1e-5,
                    intermediates: bool = False):
    """The Pre-LN block around the layer: ``y = x + layer(rmsnorm(x))`` (MLX README,
    "Architecture Details"; ZM "API" norm_eps). Same outputs as ``forward``, plus ``xn``
    (the normalized rows, bf16 bits, of the listed tokens); ``y`` includes the residual."""
    xn = rmsnorm(inp["x"], inp["norm_w"], eps)
    out = forward(dict(inp, x=xn), k, tokens=tokens, alpha=alpha, limit=limit,
                  intermediates=intermediates)
    x_tok = np.ascontiguousarray(inp["x"][out["tokens"]], dtype=np.uint16)
    out["y"] = out["y"] + (x_tok.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out["xn"] = xn[out["tokens"]]
    return out


def forward(inp: Dict[str, np.ndarray], k: int, tokens: Optional[Sequence[int]] = None,
            alpha: float = 1.702, limit: float = 7.0, intermediates: bool = False):
    """The whole layer for ``tokens`` (default: all rows of ``inp['x']``).

    Returns a dict with ``y [n, H]``, ``idx [n, k]``, ``w [n, k]``, ``logits [n, E]``,
    ``abs_sum [n, E]`` and, when ``intermediates``, ``h [n, k, I]`` and ``o [n, k, H]``.
    """
    x = inp["x"]
    T, H = x.shape
    E = inp["router_w"].shape[0]
    I = inp["dn_blocks"].shape[2] * 2
    tok = np.arange(T, dtype=np.int64) if tokens is None else np.asarray(tokens, dtype=np.int64)
    n = tok.shape[0]
    out = {
        "tokens": tok,
        "logits": np.empty((n, E), dtype=np.float64),
        "abs_sum": np.empty((n, E), dtype=np.float64),
        "idx": np.empty((n, k), dtype=np.int32),
        "w": np.empty((n, k), dtype=np.float64),
        "y": np.empty((n, H), dtype=np.float64),
    }
    h = np.empty((n, k, I), dtype=np.float64) if intermediates else None
    o = np.empty((n, k, H), dtype=np.float64) if intermediates else None
    _load().oracle_forward_tokens(
        np.ascontiguousarray(tok), n, H, I, E, k, np.ascontiguousarray(x),
        inp["router_w"], inp["router_b"], inp["gu_blocks"], inp["gu_scales"], inp["gu_bias"],
        inp["dn_blocks"], inp["dn_scales"], inp["dn_bias"], float(alpha), float(limit),
        out["logits"], _ptr(out["abs_sum"]), out["idx"], out["w"], _ptr(h), _ptr(o), out["y"])
    if intermediates:
        out["h"], out["o"] = h, o
    return out


def _bf16_rows_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def swiglu_n(gate: np.ndarray, up: np.ndarray, alpha: float = 1.702, limit: float = 7.0) -> np.ndarray:
    """``swiglu`` element by element over two arrays of equal shape."""
    g = np.ascontiguousarray(gate, dtype=np.float64)
    u = np.ascontiguousarray(up, dtype=np.float64)
    if g.shape != u.shape:
        raise ValueError("gate/up shape mismatch")
    h = np.empty_like(g)
    _load().oracle_swiglu_n(g.reshape(-1), u.reshape(-1), g.size, float(alpha), float(limit), h.reshape(-1))
    return h


def forward_expert_major(inp: Dict[str, np.ndarray], k: int, tokens: Optional[Sequence[int]] = None,
                         alpha: float = 1.702, limit: float = 7.0, intermediates: bool = False):
    """The whole layer for ``tokens`` (default: all rows of ``inp['x']``), expert by expert
    (ZeroModels GPT-OSS page, "MXFP4 experts": the bank dequantized once, then evaluated).

    Steps, in the order of the "Mixture-of-experts feed-forward" item:
      1. routing of every listed token: ``router`` (with |x w| sums) and ``topk_softmax``;
      2. for each expert e selected by some listed token, in index order:
         Wgu = dequant(gu_blocks[e], gu_scales[e])  [2I, H]   (MB orientation)
         Wdn = dequant(dn_blocks[e], dn_scales[e])  [H, I]
         X   = the bf16 rows of the tokens that selected e   [n_e, H]
         G   = X Wgu^T + bgu[e]                       (float64 matrix product)
         h   = swiglu(G[:, 0::2], G[:, 1::2])          (MT: gate even, up odd)
         O   = h Wdn^T + bdn[e]                       (float64 matrix product)
      3. y[t] = sum_{j = 0..k-1} w[t, j] O[t, j], added in slot order.
    Returns the dict of ``forward`` (``y``, ``idx``, ``w``, ``logits``, ``abs_sum``, ``tokens``
    and, when ``intermediates``, ``h [n, k, I]`` and ``o [n, k, H]``).
    """
    x = inp["x"]
    T, H = x.shape
    I = inp["dn_blocks"].shape[2] * 2
    tok = np.arange(T, dtype=np.int64) if tokens is None else np.asarray(tokens, dtype=np.int64)
    n = tok.shape[0]
    x_tok = np.ascontiguousarray(x[tok], dtype=np.uint16)
    logits, abs_sum = router(x_tok, inp["router_w"], inp["router_b"], with_abs_sum=True)
    idx, w = topk_softmax(logits, k)
    o = np.zeros((n, k, H), dtype=np.float64)
    h_all = np.zeros((n, k, I), dtype=np.float64) if intermediates else None
    xf = _bf16_rows_f64(x_tok)
    gu_bias = _bf16_rows_f64(inp["gu_bias"])
    dn_bias = _bf16_rows_f64(inp["dn_bias"])
    for e in np.unique(idx):
        rows, slots = np.nonzero(idx == e)          # (listed token, slot) pairs routed to e
        w_gu = dequant(inp["gu_blocks"][e], inp["gu_scales"][e])
        w_dn = dequant(inp["dn_blocks"][e], inp["dn_scales"][e])
        g = np.matmul(xf[rows], w_gu.T) + gu_bias[e]
        h = swiglu_n(g[:, 0::2], g[:, 1::2], alpha, limit)
        o[rows, slots] = np.matmul(h, w_dn.T) + dn_bias[e]
        if intermediates:
            h_all[rows, slots] = h
    y = np.zeros((n, H), dtype=np.float64)
    for j in range(k):
        y += w[:, j:j + 1] * o[:, j]
    out = {"tokens": tok, "logits": logits, "abs_sum": abs_sum, "idx": idx, "w": w, "y": y}
    if intermediates:
        out["h"], out["o"] = h_all, o
    return out


def forward_prenorm_expert_major(inp: Dict[str, np.ndarray], k: int, tokens: Optional[Sequence[int]] = None,
                                 alpha: float = 1.702, limit: float = 7.0, eps: float = 1e-5):
    """``forward_prenorm`` with the layer in expert-major mode."""
    xn = rmsnorm(inp["x"], inp["norm_w"], eps)
    out = forward_expert_major(dict(inp, x=xn), k, tokens=tokens, alpha=alpha, limit=limit)
    out["y"] = out["y"] + _bf16_rows_f64(inp["x"][out["tokens"]])
    out["xn"] = xn[out["tokens"]]
    return out
