"""Properties of the compiled gfx950 code that the kernels' correctness rests on.

Two families of kernels issue loads the compiler does not track and then wait for them with a
counted ``s_waitcnt vmcnt(n)``. The count is only right if the compiler emitted exactly the loads
the source asks for, in the order it asks for them. A different compiler version could merge,
drop, move or add a load (a spill reload, a hoisted load) and the wait would then end early,
with no error and wrong results. ``build()`` therefore reads the device assembly of those two
sources after every build and refuses a library whose code breaks either property; the CPU
tests run the same checks.

* Weight-streaming kernels (``k_stream``): the activation rows are copied into LDS with
  global_load_lds, then exactly 9 + 2 kUB ordinary loads are issued (8 weight-scale dwords, the
  bias, 2 kUB weight loads), then ``s_waitcnt vmcnt(9 + 2 kUB)`` waits for the copies alone.
* Grouped GEMMs (``k_gemm_mx``): inside the contraction loop every vector-memory load is a
  global_load_lds issued from inline assembly, every vmcnt is one of the kernel's own counts,
  and no kernel uses scratch memory.
"""
from __future__ import annotations

import os
import re
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

STREAM_SRC = "gemm_stream.hip"
GROUPED_SRC = "gemm_grouped.hip"
GROUPED_WAIT_COUNTS = {0, 3, 4, 6, 7, 8, 9, 10}


def device_asm(src: str, out: str) -> str:
    """gfx950 assembly of csrc/<src> (device code only), written to `out` and returned."""
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr[-2000:]}")
    with open(out) as f:
        return f.read()


def kernels(asm: str, name: str):
    """(symbol, body lines) of every kernel whose mangled name contains `name`."""
    res = []
    for m in re.finditer(r"^(_Z\S*" + name + r"\S*):", asm, re.M):
        body = asm[m.end():]
        end = body.find("s_endpgm")
        res.append((m.group(1), body[:end].split("\n")))
    return res


def stream_unroll() -> int:
    with open(os.path.join(CSRC, STREAM_SRC)) as f:
        return int(re.search(r"constexpr int kUB = (\d+);", f.read()).group(1))


def stream_problems(asm: str) -> list[str]:
    """Every k_stream wait of 9 + 2 kUB (up to 9 more, for copies issued ahead) must follow
    the last global_load_lds before it by exactly 9 + 2 kUB ordinary loads."""
    younger_expected = 9 + 2 * stream_unroll()
    found = kernels(asm, "k_stream")
    if len(found) != 2:
        return [f"expected the up and down k_stream kernels, found {len(found)}"]
    load = re.compile(r"^\s*(global_load|buffer_load|flat_load)\w*\s")
    pat = re.compile(r"s_waitcnt\s+vmcnt\((\d+)\)")
    problems = []
    for sym, lines in found:
        waits = [i for i, l in enumerate(lines)
                 if pat.search(l) and younger_expected <= int(pat.search(l).group(1)) <= younger_expected + 9]
        if not waits:
            problems.append(f"{sym}: no wait for the activation copies")
        for w in waits:
            copies = [i for i in range(w) if "global_load_lds" in lines[i]]
            if not copies:
                problems.append(f"{sym}: the wait at line {w} follows no global_load_lds")
                continue
            younger = [lines[i] for i in range(copies[-1] + 1, w)
                       if load.match(lines[i]) and "global_load_lds" not in lines[i]]
            if len(younger) != younger_expected:
                problems.append(f"{sym}: {len(younger)} loads between the copies and the wait at line {w}, "
                                f"expected {younger_expected}")
    return problems


def _blocks_with_depth(lines):
    """(loop depth, line) for every line of a kernel body, from the compiler's block comments
    ('; in Loop: Header=... Depth=n' on each basic-block label inside a loop)."""
    depth = 0
    for line in lines:
        if re.match(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)", line):
            m = re.search(r"Depth=(\d+)", line)
            depth = int(m.group(1)) if m else 0
        yield depth, line


def grouped_problems(asm: str) -> list[str]:
    """Inside the grouped GEMMs' contraction loops: only global_load_lds loads, only the
    kernel's own vmcnt counts, and no scratch anywhere."""
    found = kernels(asm, "k_gemm_mx")
    if len(found) != 4:
        return [f"expected 4 k_gemm_mx kernels (up / down x full / small-group tiles), found {len(found)}"]
    vload = re.compile(r"^\s*(global_load|buffer_load|flat_load|scratch_load)\w*\s")
    vmcnt = re.compile(r"s_waitcnt\s+vmcnt\((\d+)\)")
    problems = []
    for sym, lines in found:
        if any("scratch_" in l for l in lines):
            problems.append(f"{sym}: uses scratch memory")
        inner = [l for d, l in _blocks_with_depth(lines) if d >= 2]
        if not any("global_load_lds" in l for l in inner):
            problems.append(f"{sym}: no global_load_lds inside the contraction loop")
        if not any("v_mfma_scale_f32_16x16x128_f8f6f4" in l for l in inner):
            problems.append(f"{sym}: no block-scaled MFMA inside the contraction loop")
        stray = [l.strip() for l in inner if vload.match(l) and "global_load_lds" not in l]
        if stray:
            problems.append(f"{sym}: compiler-issued loads inside the contraction loop: {stray[:4]}")
        counts = {int(m.group(1)) for l in inner for m in [vmcnt.search(l)] if m}
        if not counts <= GROUPED_WAIT_COUNTS:
            problems.append(f"{sym}: vmcnt counts {sorted(counts - GROUPED_WAIT_COUNTS)} are not the kernel's own")
    return problems


def check(build_dir: str, pool=None) -> None:
    """Assemble both sources into build_dir and raise RuntimeError on any broken property.
    With `pool` (a concurrent.futures executor) the two compilations run in it."""
    jobs = [(STREAM_SRC, stream_problems), (GROUPED_SRC, grouped_problems)]
    outs = [os.path.join(build_dir, src + ".s") for src, _ in jobs]
    if pool is not None:
        texts = list(pool.map(device_asm, [src for src, _ in jobs], outs))
    else:
        texts = [device_asm(src, out) for (src, _), out in zip(jobs, outs)]
    problems = [p for (_, fn), text in zip(jobs, texts) for p in fn(text)]
    if problems:
        raise RuntimeError("the compiled kernels break the counted-wait invariants their correctness "
                           "rests on:\n  " + "\n  ".join(problems))
