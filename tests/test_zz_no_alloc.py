"""The allocation-free forward (moe_mxfp4_forward_noalloc) through the C ABI: bit-identical
to moe_mxfp4_forward with a caller workspace (the same kernels), on consecutive calls that
share the library's per-GPU scratch array, each later call smaller than the one before, and
within the oracle's bar; shapes beyond the array are rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import mxfp4_mixture_experts_router_amd as moe
import oracle
from workloads import CONFIGS, make_inputs

from gpu_util import assert_close_rows, bf16_to_f64, check_selection, upload

pytestmark = pytest.mark.gpu

EWORKSPACE = 4


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return moe.load_library()


def _noalloc(lib, d, cfg, T):
    """y, topk_idx, topk_w from moe_mxfp4_forward_noalloc on the current stream."""
    dev = d["x"].device
    y = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
    w = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
    shape = moe._shape(T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.alpha, cfg.limit)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = lib.moe_mxfp4_forward_noalloc(
        ctypes.byref(shape), P(d["x"]), P(d["router_w"]), P(d["router_b"]), P(d["gu_blocks"]),
        P(d["gu_scales"]), P(d["gu_bias"]), P(d["dn_blocks"]), P(d["dn_scales"]), P(d["dn_bias"]),
        P(y), P(idx), P(w), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.moe_mxfp4_last_error().decode()
    return y, idx, w


def _with_workspace(d, cfg):
    return moe.moe_forward(d["x"], d["router_w"], d["router_b"], d["gu_blocks"], d["gu_scales"],
                           d["gu_bias"], d["dn_blocks"], d["dn_scales"], d["dn_bias"], cfg.k, cfg.alpha,
                           cfg.limit, return_topk=True)


@pytest.mark.parametrize("name,Ts", [
    ("tiny", (300, 65, 17, 3)),          # grouped sequence, then both decode sequences
    ("batched_decode_20b", (700, 64, 1)),  # 700 tokens: near the scratch limit at the 20B shape
])
def test_noalloc_matches_forward_on_consecutive_calls(lib, name, Ts):
    cfg = CONFIGS[name]
    weights = make_inputs(cfg, seed=4, parts=tuple(p for p in ("router_w", "router_b", "gu_blocks", "gu_scales",
                                                                   "gu_bias", "dn_blocks", "dn_scales", "dn_bias")))
    dw = upload(weights)
    for T in Ts:          # each call smaller than the last: the scratch keeps the previous contents
        x = make_inputs(cfg, seed=40 + T, T=T, parts=("x",))
        d = dict(dw, **upload(x))
        assert moe.workspace_bytes(T, cfg.H, cfg.I, cfg.E, cfg.k) <= lib.moe_mxfp4_noalloc_max_bytes()
        y, idx, w = _noalloc(lib, d, cfg, T)
        y_ref, idx_ref, w_ref = _with_workspace(d, cfg)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (name, T)
        assert torch.equal(idx, idx_ref) and torch.equal(w, w_ref), (name, T)
        # and the oracle's bar, on a few tokens
        tokens = np.unique(np.linspace(0, T - 1, min(T, 8)).astype(np.int64))
        ref = oracle.forward(dict(weights, **x), cfg.k, tokens=tokens, alpha=cfg.alpha, limit=cfg.limit)
        ok = check_selection(idx.cpu().numpy()[tokens], ref, cfg.H, cfg.k)
        assert_close_rows(bf16_to_f64(y)[tokens][ok], ref["y"][ok], f"noalloc y ({name}, T={T})")


def test_noalloc_rejects_shapes_beyond_the_scratch(lib):
    cfg = CONFIGS["prefill_20b"]
    assert moe.workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k) > lib.moe_mxfp4_noalloc_max_bytes()
    shape = moe._shape(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
    A = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails before any launch
    st = lib.moe_mxfp4_forward_noalloc(ctypes.byref(shape), *([A] * 10), None, None, None)
    assert st == EWORKSPACE
    assert "workspace" in lib.moe_mxfp4_last_error().decode()
