"""Properties of the compiled gfx950 code that the kernels' correctness rests on (CPU only:
hipcc cross-compiles the device code to assembly here).

The weight-streaming kernels copy the activation rows into LDS with global_load_lds and
then wait for those copies with s_waitcnt vmcnt(9 + 2 * kUB (+ the next item's copies, issued
first)): the copies are older than exactly that many vector-memory loads (8 weight-scale
dwords, the bias, 2 kUB weight loads). If the
compiler merged, dropped or moved one of those loads, the wait would end before the copies
had landed. This test reads the generated assembly and counts.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp4_mixture_experts_router_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _device_asm(src: str, tmp_path) -> str:
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    out = tmp_path / "dev.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(asm: str, name: str):
    """(symbol, body lines) of every kernel whose mangled name contains `name`."""
    res = []
    for m in re.finditer(r"^(_Z\S*" + name + r"\S*):", asm, re.M):
        body = asm[m.end():]
        end = body.find("s_endpgm")
        res.append((m.group(1), body[:end].split("\n")))
    return res


def test_stream_copies_wait_counts_the_younger_loads(tmp_path):
    src = open(os.path.join(CSRC, "gemm_stream.hip")).read()
    ub = int(re.search(r"constexpr int kUB = (\d+);", src).group(1))
    younger_expected = 9 + 2 * ub
    asm = _device_asm("gemm_stream.hip", tmp_path)
    kernels = _kernels(asm, "k_stream")
    assert len(kernels) == 2   # up and down
    load = re.compile(r"^\s*(global_load|buffer_load|flat_load)\w*\s")
    for sym, lines in kernels:
        # the wait may also allow for the next item's copies (issued before the loads): any
        # vmcnt(n) with n in [younger, younger + 9] must follow the copies by exactly
        # `younger` loads
        pat = re.compile(r"s_waitcnt\s+vmcnt\((\d+)\)")
        waits = [i for i, l in enumerate(lines)
                 if pat.search(l) and younger_expected <= int(pat.search(l).group(1)) <= younger_expected + 9]
        assert waits, sym
        for w in waits:
            copies = [i for i in range(w) if "global_load_lds" in lines[i]]
            assert copies, sym
            younger = [lines[i] for i in range(copies[-1] + 1, w)
                       if load.match(lines[i]) and "global_load_lds" not in lines[i]]
            assert len(younger) == younger_expected, (sym, w, len(younger))


def _blocks_with_depth(lines):
    """(loop depth, line) for every line of a kernel body, from the compiler's block comments
    ('; in Loop: Header=... Depth=n' on each basic-block label inside a loop)."""
    depth = 0
    for line in lines:
        if re.match(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)", line):
            m = re.search(r"Depth=(\d+)", line)
            depth = int(m.group(1)) if m else 0
        yield depth, line


def test_grouped_gemm_waits_are_its_own(tmp_path):
    """The prefill GEMMs issue their operand loads from inline assembly (global_load_lds, which
    the compiler does not track) and wait for a stage with s_waitcnt vmcnt(n), n = the loads of
    the next stage (3 to 10). That is only right if, inside the contraction loop, no load the
    compiler issued itself (a scratch spill reload, a global load hoisted into the loop) adds
    to the count or brings a compiler-inserted wait: every vector-memory load there must be a
    global_load_lds, every vmcnt one of the kernel's own counts, and no kernel may use scratch."""
    asm = _device_asm("gemm_grouped.hip", tmp_path)
    kernels = _kernels(asm, "k_gemm_mx")
    assert len(kernels) == 4   # up / down x full / small-group tiles
    vload = re.compile(r"^\s*(global_load|buffer_load|flat_load|scratch_load)\w*\s")
    vmcnt = re.compile(r"s_waitcnt\s+vmcnt\((\d+)\)")
    for sym, lines in kernels:
        assert not any("scratch_" in l for l in lines), sym
        inner = [l for d, l in _blocks_with_depth(lines) if d >= 2]
        assert any("global_load_lds" in l for l in inner), sym
        assert any("v_mfma_scale_f32_16x16x128_f8f6f4" in l for l in inner), sym
        stray = [l.strip() for l in inner if vload.match(l) and "global_load_lds" not in l]
        assert not stray, (sym, stray[:4])
        counts = {int(m.group(1)) for l in inner for m in [vmcnt.search(l)] if m}
        assert counts <= {0, 3, 4, 6, 7, 8, 9, 10}, (sym, sorted(counts))
