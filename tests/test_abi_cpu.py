"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch.

Every call here fails validation (or is a pure host query), so the HIP runtime is
never asked to launch anything; pointer arguments are fake addresses that are never
dereferenced.
"""
import ctypes
import os
import re

import pytest

import mxfp4_mixture_experts_router_amd as moe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "moe_mxfp4.h")
EINVAL, ESHAPE, EALIGN, EWORKSPACE = 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.library_path()):
        from mxfp4_mixture_experts_router_amd import build
        build.build()
    return moe.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_mxfp4_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(moe._SIGS), "binding signatures and header disagree"


def test_abi_version(lib):
    assert moe.abi_version() == 6
    assert "#define MOE_MXFP4_ABI_VERSION 6" in open(HEADER).read()


def shape(T=1, H=2880, I=2880, E=32, k=4, alpha=1.702, limit=7.0):
    return moe._shape(T, H, I, E, k, alpha, limit)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), EINVAL), (dict(H=2881), ESHAPE), (dict(H=0), ESHAPE), (dict(I=48), ESHAPE),
    (dict(E=0), ESHAPE), (dict(E=257), ESHAPE), (dict(k=0), ESHAPE), (dict(k=9, E=16), ESHAPE),
    (dict(k=5, E=4), ESHAPE), (dict(T=(1 << 24) + 1), ESHAPE),
    (dict(alpha=float("nan")), EINVAL), (dict(limit=float("inf")), EINVAL),
])
def test_check_shape_rejects(lib, kw, code):
    s = shape(**kw)
    assert lib.moe_mxfp4_check_shape(ctypes.byref(s)) == code
    assert lib.moe_mxfp4_last_error().decode()
    n = ctypes.c_size_t(12345)
    assert lib.moe_mxfp4_workspace_bytes(ctypes.byref(s), ctypes.byref(n)) == code
    assert n.value == 12345  # nothing written on error


def test_check_shape_null(lib):
    assert lib.moe_mxfp4_check_shape(None) == EINVAL


@pytest.mark.parametrize("T,H,I,E,k", [(1, 2880, 2880, 32, 4), (64, 2880, 2880, 32, 4),
                                       (4096, 2880, 2880, 32, 4), (2048, 2880, 2880, 128, 4),
                                       (8, 64, 64, 4, 2), (0, 64, 64, 4, 2)])
def test_workspace_sizes(lib, T, H, I, E, k):
    s = shape(T, H, I, E, k)
    assert lib.moe_mxfp4_check_shape(ctypes.byref(s)) == 0
    assert lib.moe_mxfp4_last_error() == b""
    n = moe.workspace_bytes(T, H, I, E, k)
    N = T * k
    if moe.uses_decode_path(T, H, I):
        assert n >= 4 * N * I + 2 * T * H + 2 * N * 4        # mx8 h (half-block rows) and x
    else:
        assert n >= N * (2 * I + H * 4) + 2 * T * H + 3 * N * 4   # mx8 h and x, fp32 o
    assert n % 256 == 0


A = 0x10000  # fake, 16-byte aligned device addresses; never dereferenced


def fwd(lib, s, **over):
    args = dict(x=A, rw=A, rb=A, gb=A, gs=A, gbias=A, db=A, ds=A, dbias=A, y=A, idx=None, w=None,
                ws=0x100000, wsb=1 << 40, stream=None)
    args.update(over)
    return lib.moe_mxfp4_forward(ctypes.byref(s), *[args[k] for k in
                                 ("x", "rw", "rb", "gb", "gs", "gbias", "db", "ds", "dbias", "y",
                                  "idx", "w", "ws")], args["wsb"], args["stream"])


@pytest.mark.parametrize("field", ["x", "rw", "rb", "gb", "gs", "gbias", "db", "ds", "dbias", "y"])
def test_forward_null_pointer(lib, field):
    s = shape()
    assert fwd(lib, s, **{field: None}) == EINVAL
    assert "NULL" in lib.moe_mxfp4_last_error().decode()


@pytest.mark.parametrize("field", ["x", "rw", "gb", "db", "y"])
def test_forward_misaligned(lib, field):
    s = shape()
    assert fwd(lib, s, **{field: A + 2}) == EALIGN


def test_forward_workspace_checks(lib):
    s = shape()
    need = moe.workspace_bytes(1, 2880, 2880, 32, 4)
    assert fwd(lib, s, ws=None) == EWORKSPACE
    assert fwd(lib, s, wsb=need - 1) == EWORKSPACE
    assert fwd(lib, s, ws=0x100010) == EALIGN


def test_forward_timed_validates_events(lib):
    s = shape()
    base = [ctypes.byref(s)] + [A] * 10 + [None, None, 0x100000, 1 << 40, None]
    n = ctypes.c_int(-1)
    evs = (ctypes.c_void_p * (2 * moe.MAX_LAUNCHES))(*([A] * (2 * moe.MAX_LAUNCHES)))
    assert lib.moe_mxfp4_forward_timed(*base, None, 2 * moe.MAX_LAUNCHES, ctypes.byref(n)) == EINVAL
    assert lib.moe_mxfp4_forward_timed(*base, evs, 2 * moe.MAX_LAUNCHES - 1, ctypes.byref(n)) == EINVAL
    assert "n_events" in lib.moe_mxfp4_last_error().decode()
    evs[3] = None
    assert lib.moe_mxfp4_forward_timed(*base, evs, 2 * moe.MAX_LAUNCHES, ctypes.byref(n)) == EINVAL
    assert "events[3]" in lib.moe_mxfp4_last_error().decode()


def test_forward_bad_shape_before_pointers(lib):
    s = shape(k=0)
    assert fwd(lib, s, x=None) == ESHAPE


def test_zero_tokens_is_a_no_op(lib):
    # T = 0 validates, then returns without touching the device
    s = shape(T=0)
    assert fwd(lib, s) == 0
    assert lib.moe_mxfp4_route(ctypes.byref(s), A, A, A, A, A, None, None) == 0


def test_stage_entry_points_validate(lib):
    s = shape()
    assert lib.moe_mxfp4_route(ctypes.byref(s), A, A, A, None, A, None, None) == EINVAL
    assert lib.moe_mxfp4_route(ctypes.byref(s), A + 8, A, A, A, A, None, None) == EALIGN
    assert lib.moe_mxfp4_permute(ctypes.byref(s), A, A, A, A, A, None, None) == EINVAL
    assert lib.moe_mxfp4_expert_up(ctypes.byref(s), A, A, A, A, A, A, A + 4, None) == EALIGN
    assert lib.moe_mxfp4_expert_down(ctypes.byref(s), A, A, A, A, A, None, A, None) == EINVAL
    assert lib.moe_mxfp4_combine(ctypes.byref(s), A, A, None, None) == EINVAL
    bad = shape(E=300)
    assert lib.moe_mxfp4_permute(ctypes.byref(bad), A, A, A, A, A, A, None) == ESHAPE


def fwd_prenorm(lib, s, timed=False, **over):
    args = dict(x=A, nw=A, eps=1e-5, rw=A, rb=A, gb=A, gs=A, gbias=A, db=A, ds=A, dbias=A, y=A,
                idx=None, w=None, ws=0x100000, wsb=1 << 40, stream=None)
    args.update(over)
    call = [ctypes.byref(s)] + [args[k] for k in ("x", "nw", "eps", "rw", "rb", "gb", "gs", "gbias", "db",
                                                  "ds", "dbias", "y", "idx", "w", "ws", "wsb", "stream")]
    if timed:
        n = ctypes.c_int(-1)
        return lib.moe_mxfp4_forward_prenorm_timed(*call, None, 0, ctypes.byref(n))
    return lib.moe_mxfp4_forward_prenorm(*call)


@pytest.mark.parametrize("over,code,msg", [
    (dict(nw=None), EINVAL, "norm_w"), (dict(nw=A + 2), EALIGN, "norm_w"),
    (dict(eps=float("nan")), EINVAL, "norm_eps"), (dict(eps=-1e-6), EINVAL, "norm_eps"),
    (dict(eps=float("inf")), EINVAL, "norm_eps"), (dict(x=None), EINVAL, "x"),
    (dict(ws=None), EWORKSPACE, "workspace"),
])
def test_forward_prenorm_validates(lib, over, code, msg):
    s = shape()
    assert fwd_prenorm(lib, s, **over) == code
    assert msg in lib.moe_mxfp4_last_error().decode()


def test_forward_prenorm_edges(lib):
    assert fwd_prenorm(lib, shape(k=0), nw=None) == ESHAPE          # shape first
    assert fwd_prenorm(lib, shape(T=0), nw=None) == 0               # no tokens: no pointer read
    assert fwd_prenorm(lib, shape(), timed=True) == EINVAL          # events required
    assert "events" in lib.moe_mxfp4_last_error().decode()
    # the pre-norm block needs no more workspace than the plain layer
    s = shape()
    need = moe.workspace_bytes(1, 2880, 2880, 32, 4)
    assert fwd_prenorm(lib, s, wsb=need - 1) == EWORKSPACE


def test_forward_dequantized_validates(lib):
    s = shape()
    base = dict(x=A, rw=A, rb=A, gw=A, gb=A, dw=A, db=A, y=A, idx=None, w=None, ws=0x100000, wsb=1 << 40)
    order = ("x", "rw", "rb", "gw", "gb", "dw", "db", "y", "idx", "w", "ws", "wsb")

    def call(**over):
        args = dict(base, **over)
        return lib.moe_mxfp4_forward_dequantized(ctypes.byref(s), *[args[k] for k in order], None)
    for field in ("x", "rw", "rb", "gw", "gb", "dw", "db", "y"):
        assert call(**{field: None}) == EINVAL, field
    for field in ("x", "rw", "gw", "dw", "y"):
        assert call(**{field: A + 2}) == EALIGN, field
    assert call(ws=None) == EWORKSPACE
    need = moe.workspace_bytes_dequantized(1, 2880, 2880, 32, 4)
    assert call(wsb=need - 1) == EWORKSPACE
    assert need >= 4 * (2880 * 2 + 2880 * 4)       # h bf16 and o fp32 rows of the 4 pairs
    n = ctypes.c_int(-1)
    assert lib.moe_mxfp4_forward_dequantized_timed(ctypes.byref(s), *[base[k] for k in order], None,
                                                   None, 0, ctypes.byref(n)) == EINVAL
    bad = shape(k=9, E=16)
    assert lib.moe_mxfp4_forward_dequantized(ctypes.byref(bad), *[base[k] for k in order], None) == ESHAPE


def test_rmsnorm_validates(lib):
    assert lib.moe_mxfp4_rmsnorm(A, A, 4, 60, 1e-5, A, None) == ESHAPE
    assert lib.moe_mxfp4_rmsnorm(A, A, 4, 0, 1e-5, A, None) == ESHAPE
    assert lib.moe_mxfp4_rmsnorm(A, A, -1, 64, 1e-5, A, None) == EINVAL
    assert lib.moe_mxfp4_rmsnorm(A, A, (1 << 24) + 1, 64, 1e-5, A, None) == ESHAPE
    assert lib.moe_mxfp4_rmsnorm(A, A, 4, 64, float("nan"), A, None) == EINVAL
    assert lib.moe_mxfp4_rmsnorm(A, A, 4, 64, -1.0, A, None) == EINVAL
    assert lib.moe_mxfp4_rmsnorm(A, None, 4, 64, 1e-5, A, None) == EINVAL
    assert lib.moe_mxfp4_rmsnorm(A, A + 8, 4, 64, 1e-5, A, None) == EALIGN
    assert lib.moe_mxfp4_rmsnorm(A, A, 4, 64, 1e-5, A + 2, None) == EALIGN
    assert lib.moe_mxfp4_rmsnorm(None, None, 0, 64, 1e-5, None, None) == 0   # empty: no launch


def test_mx8_format_entry_points(lib):
    # 2R (K + roundup16(K/32)) bytes; validation only (no device work)
    assert lib.moe_mxfp4_mx8_bytes(3, 2880) == 2 * 3 * (2880 + 96)
    assert lib.moe_mxfp4_mx8_bytes(1, 32) == 2 * (32 + 16)
    assert lib.moe_mxfp4_mx8_bytes(0, 64) == 0
    assert lib.moe_mxfp4_quantize_act(A, 4, 48, A, None) == ESHAPE
    assert lib.moe_mxfp4_quantize_act(A, -1, 64, A, None) == EINVAL
    assert lib.moe_mxfp4_quantize_act(A, 4, 64, None, None) == EINVAL
    assert lib.moe_mxfp4_quantize_act(A + 2, 4, 64, A, None) == EALIGN
    assert lib.moe_mxfp4_quantize_act(None, 0, 64, None, None) == 0
    # the h8 layout (group-major scales) fits the same allocation for every K
    for K in range(32, 4097, 32):
        assert 2 * K + 16 * ((K + 511) // 512) <= lib.moe_mxfp4_mx8_bytes(1, K)
    assert lib.moe_mxfp4_quantize_h(A, 4, 48, A, None) == ESHAPE
    assert lib.moe_mxfp4_quantize_h(A, -1, 64, A, None) == EINVAL
    assert lib.moe_mxfp4_quantize_h(A, 4, 64, None, None) == EINVAL
    assert lib.moe_mxfp4_quantize_h(A, 4, 64, A + 8, None) == EALIGN
    assert lib.moe_mxfp4_quantize_h(None, 0, 64, None, None) == 0


def test_dequant_validates(lib):
    assert lib.moe_mxfp4_dequant(A, A, 4, 48, A, None) == ESHAPE
    assert lib.moe_mxfp4_dequant(A, A, -1, 64, A, None) == EINVAL
    assert lib.moe_mxfp4_dequant(None, A, 4, 64, A, None) == EINVAL
    assert lib.moe_mxfp4_dequant(A + 1, A, 4, 64, A, None) == EALIGN
    assert lib.moe_mxfp4_dequant(A, A, 0, 64, A, None) == 0       # empty: no launch


def test_clock_probe_validates(lib):
    assert lib.moe_mxfp4_clock_probe(None, 256, 100, None) == EINVAL
    assert lib.moe_mxfp4_clock_probe(A, 0, 100, None) == EINVAL
    assert lib.moe_mxfp4_clock_probe(A, 65537, 100, None) == EINVAL
    assert lib.moe_mxfp4_clock_probe(A, 256, 0, None) == EINVAL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(moe.MoeLibraryMissing):
        moe.load_library()


@pytest.mark.parametrize("T,E,k,blocks", [(64, 32, 4, 1), (65, 32, 4, 2), (4096, 32, 4, 64), (2048, 128, 4, 32),
                                          (65536, 32, 4, 1024), (65537, 32, 4, 1025), (1, 256, 8, 1),
                                          (1 << 24, 128, 4, 1 << 18), (0, 32, 4, -1)])
def test_permute_workspace_bytes(lib, T, E, k, blocks):
    """One histogram row of E ints per 256 pairs plus one row of per-expert totals, at any
    size; nothing for no pairs."""
    s = shape(T=T, E=E, k=k)
    n = ctypes.c_size_t(12345)
    assert lib.moe_mxfp4_permute_workspace_bytes(ctypes.byref(s), ctypes.byref(n)) == 0
    assert n.value == (blocks + 1) * E * 4


def test_permute_ws_validation(lib):
    s = shape(T=100, E=32, k=4)       # 400 pairs: 2 histogram rows of 32 ints and the totals
    need = 3 * 32 * 4
    args = [A, A, A, A, A, A]
    assert lib.moe_mxfp4_permute_ws(ctypes.byref(s), *args, None, need, None) == EWORKSPACE
    assert lib.moe_mxfp4_permute_ws(ctypes.byref(s), *args, A, need - 1, None) == EWORKSPACE
    assert lib.moe_mxfp4_permute_ws(ctypes.byref(s), *args, A + 2, need, None) == EALIGN
    for i in range(6):
        bad = list(args)
        bad[i] = None
        assert lib.moe_mxfp4_permute_ws(ctypes.byref(s), *bad, A, need, None) == EINVAL
    bad_shape = shape(T=100, E=32, k=33)
    assert lib.moe_mxfp4_permute_ws(ctypes.byref(bad_shape), *args, A, need, None) == ESHAPE
    zero = shape(T=0, E=32, k=4)
    assert lib.moe_mxfp4_permute_ws(ctypes.byref(zero), None, None, None, None, None, None, None, 0, None) == 0


def test_noalloc_limit_and_rejection(lib):
    """The allocation-free forward states its scratch size and rejects larger workspaces on the
    host, before touching the GPU."""
    limit = lib.moe_mxfp4_noalloc_max_bytes()
    assert limit == 64 << 20
    assert moe.workspace_bytes(64, 2880, 2880, 32, 4) <= limit          # every decode batch fits
    s = shape(T=4096)
    assert moe.workspace_bytes(4096, 2880, 2880, 32, 4) > limit
    st = lib.moe_mxfp4_forward_noalloc(ctypes.byref(s), *([A] * 10), None, None, None)
    assert st == EWORKSPACE
    assert "workspace" in lib.moe_mxfp4_last_error().decode()
    bad = shape(H=2881)
    assert lib.moe_mxfp4_forward_noalloc(ctypes.byref(bad), *([A] * 10), None, None, None) == ESHAPE
