"""Host sanitizer runs (CPU only, no GPU needed).

* The oracle (``oracle/oracle.c``) built with AddressSanitizer and UndefinedBehaviorSanitizer
  runs its entry points, brute and expert-major, on small and edge shapes.
* The C-ABI library with AddressSanitizer in its host code runs the host-side validation and
  the size queries of every entry point (fake device pointers, never dereferenced; no launch).

Each run happens in a child process with the sanitizer runtime preloaded; any report fails
the test.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gcc_runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _run(script, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", textwrap.dedent(script)], capture_output=True, text=True,
                       env=env, timeout=900, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "sanitized run done" in r.stdout
    return r.stdout


ORACLE_SCRIPT = """
import numpy as np
import oracle
from workloads import CONFIGS, make_inputs
cfg = CONFIGS["tiny"]
for (T, H, I, E, k) in [(8, 64, 64, 4, 2), (3, 96, 32, 5, 5), (1, 32, 64, 1, 1), (17, 64, 96, 8, 3)]:
    c = cfg.with_(H=H, I=I, E=E, k=k)
    inp = make_inputs(c, seed=1, T=T)
    a = oracle.forward(inp, k, alpha=c.alpha, limit=c.limit, intermediates=True)
    b = oracle.forward_expert_major(inp, k, alpha=c.alpha, limit=c.limit, intermediates=True)
    assert np.allclose(a["y"], b["y"], rtol=1e-9, atol=1e-9)
    oracle.forward_prenorm(inp, k, alpha=c.alpha, limit=c.limit, eps=1e-5)
    oracle.forward_prenorm_expert_major(inp, k, alpha=c.alpha, limit=c.limit, eps=1e-5)
    oracle.dequant(inp["gu_blocks"], inp["gu_scales"])
    oracle.rmsnorm(inp["x"], inp["norm_w"], 1e-5)
lg = np.array([[1.0, 1.0, 0.5, 1.0]])
oracle.topk_softmax(lg, 4)
oracle.swiglu_n(np.linspace(-9, 9, 37), np.linspace(9, -9, 37))
print([oracle.e2m1(c) for c in range(16)], [oracle.e8m0(b) for b in (0, 1, 127, 254, 255)])
print("sanitized run done")
"""


def test_oracle_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    import oracle
    lib = oracle.build(force=True, sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    _run(ORACLE_SCRIPT, {"LD_PRELOAD": f"{asan}:{ubsan}", "ORACLE_LIB": lib,
                         "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                         "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})


ABI_SCRIPT = """
import ctypes, os
lib = ctypes.CDLL(os.environ["MOE_LIB"])
vp, i64 = ctypes.c_void_p, ctypes.c_int64


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("swiglu_alpha", ctypes.c_float), ("swiglu_limit", ctypes.c_float)]


def sh(T=1, H=2880, I=2880, E=32, k=4):
    return Shape(T, H, I, E, k, 1.702, 7.0)


lib.moe_mxfp4_last_error.restype = ctypes.c_char_p
lib.moe_mxfp4_abi_version.restype = ctypes.c_int
assert lib.moe_mxfp4_abi_version() >= 4
A = 0x100000
size = ctypes.c_size_t(0)
codes = []
for s in [sh(), sh(T=64), sh(T=4096), sh(T=2048, E=128), sh(T=0), sh(k=0), sh(k=9), sh(E=300), sh(H=100),
          sh(I=48), sh(T=-1), sh(k=33, E=32)]:
    codes.append(lib.moe_mxfp4_check_shape(ctypes.byref(s)))
    codes.append(lib.moe_mxfp4_workspace_bytes(ctypes.byref(s), ctypes.byref(size)))
    codes.append(lib.moe_mxfp4_workspace_bytes_dequantized(ctypes.byref(s), ctypes.byref(size)))
    codes.append(lib.moe_mxfp4_permute_workspace_bytes(ctypes.byref(s), ctypes.byref(size)))
    lib.moe_mxfp4_last_error()
assert codes[0] == 0 and any(c != 0 for c in codes)
s = sh()
fwd_args = [ctypes.byref(s)] + [vp(A)] * 10 + [None, None, vp(A), ctypes.c_size_t(1 << 40), None]
for i in range(1, 11):   # every pointer NULL in turn (rejected before any launch)
    a = list(fwd_args)
    a[i] = None
    assert lib.moe_mxfp4_forward(*a) == 1, lib.moe_mxfp4_last_error()
for i in (1, 2, 4, 7, 10):   # x, router_w, gu_blocks, dn_blocks, y misaligned
    a = list(fwd_args)
    a[i] = vp(A + 2)
    assert lib.moe_mxfp4_forward(*a) == 3, lib.moe_mxfp4_last_error()
a = list(fwd_args)
a[14] = ctypes.c_size_t(10)   # workspace smaller than needed
assert lib.moe_mxfp4_forward(*a) == 4
n = ctypes.c_int(-1)
evs = (vp * 32)(*([A] * 32))
assert lib.moe_mxfp4_forward_timed(*fwd_args, None, 32, ctypes.byref(n)) == 1
assert lib.moe_mxfp4_forward_timed(*fwd_args, evs, 3, ctypes.byref(n)) == 1
bad = sh(k=0)
assert lib.moe_mxfp4_forward(ctypes.byref(bad), *fwd_args[1:]) == 2
assert lib.moe_mxfp4_forward_noalloc(ctypes.byref(sh(T=100000)), *([vp(A)] * 10), None, None, None) == 4
lib.moe_mxfp4_noalloc_max_bytes.restype = ctypes.c_size_t
assert lib.moe_mxfp4_noalloc_max_bytes() > 0
lib.moe_mxfp4_mx8_bytes.restype = ctypes.c_size_t
assert lib.moe_mxfp4_mx8_bytes(i64(3), ctypes.c_int32(64)) > 0
assert lib.moe_mxfp4_route(ctypes.byref(s), vp(A), vp(A), vp(A), None, vp(A), None, None) == 1
assert lib.moe_mxfp4_permute(ctypes.byref(s), vp(A), vp(A), vp(A), vp(A), vp(A), None, None) == 1
assert lib.moe_mxfp4_dequant(None, vp(A), i64(4), ctypes.c_int32(64), vp(A), None) == 1
assert lib.moe_mxfp4_quantize_h(vp(A), i64(4), ctypes.c_int32(48), vp(A), None) == 2
assert lib.moe_mxfp4_quantize_h(vp(A), i64(4), ctypes.c_int32(64), None, None) == 1
assert lib.moe_mxfp4_last_error()
print("sanitized run done")
"""


def test_abi_validation_under_host_asan(tmp_path):
    from mxfp4_mixture_experts_router_amd import build
    try:
        rt = build.asan_runtime()
    except RuntimeError:
        pytest.skip("clang's ASan runtime is not installed")
    lib = build.build(host_asan=True, out=str(tmp_path / "libmoe_mxfp4_host_asan.so"))
    _run(ABI_SCRIPT, {"LD_PRELOAD": rt, "MOE_LIB": lib, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1"})
