"""Build libmoe_mxfp4.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Every source under csrc/ is compiled to an object in ``_build/`` (in parallel) and
linked into ``libmoe_mxfp4.so`` next to this file. The build fails if the compiled kernels
break the counted-wait invariants their correctness rests on (``isa_check``). Run ``python -m
mxfp4_mixture_experts_router_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

if __package__:
    from . import isa_check
else:   # run as a file
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from mxfp4_mixture_experts_router_amd import isa_check

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_mxfp4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # packed-fp32 VALU forms are left to the compiler's scalar code generation off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# Host-side AddressSanitizer (the ABI layer's validation and host logic; the device code is
# built as usual): each flag applies to the host compilation only.
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, host_asan: bool = False, out: str | None = None) -> str:
    """Build the library (in-tree by default). With ``host_asan`` the host code carries
    AddressSanitizer checks and the library goes to ``out``; a process loading it needs
    clang's ASan runtime (``asan_runtime()``) preloaded."""
    lib = out or LIB
    build_dir = BUILD + ("_host_asan" if host_asan else "")
    extra = HOST_ASAN if host_asan else []
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        # the counted-wait invariants of the compiled kernels are checked alongside (isa_check)
        checked = ex.submit(isa_check.check, build_dir)
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), srcs))
        checked.result()
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if not host_asan:
        write_build_info()
    if verbose:
        print(f"built {lib}")
    return lib


BUILD_INFO = os.path.join(PKG, "build_info.json")


def sources_sha16() -> str:
    """Hash of the library's sources (the public header and csrc/), as bench.py also computes."""
    import hashlib
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "include"), CSRC):
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def write_build_info() -> None:
    """Record next to the library which sources it was built from: the git commit (when the
    tree is a checkout) and a hash of the sources, so that a run on a copy of the tree without
    its history can still name the commit and tell whether the library matches the sources."""
    import json
    sha, dirty = None, None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        if r.returncode == 0:
            sha = r.stdout.strip() or None
            d = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--", "include",
                                os.path.relpath(CSRC, ROOT)], capture_output=True, text=True, timeout=10)
            dirty = bool(d.stdout.strip()) if d.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        pass
    with open(BUILD_INFO, "w") as f:
        json.dump({"git_sha": sha, "sources_dirty": dirty, "sources_sha16": sources_sha16()}, f)


def asan_runtime() -> str:
    """clang's shared AddressSanitizer runtime (the one hipcc's host compiler links against)."""
    r = subprocess.run([os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path):
        raise RuntimeError("clang's ASan runtime not found")
    return path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
