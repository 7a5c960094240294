"""Properties of the compiled gfx950 code that the kernels' correctness rests on (CPU only:
hipcc cross-compiles the device code to assembly here). The checks themselves live in the
package (isa_check), where build() also runs them, so that a library whose code breaks them is
never built; these tests run them on their own and show that each check can fail.

The weight-streaming kernels copy the activation rows into LDS with global_load_lds and then
wait for those copies with s_waitcnt vmcnt(9 + 2 * kUB): the copies are older than exactly
that many vector-memory loads (8 weight-scale dwords, the bias, 2 kUB weight loads). The
grouped GEMMs issue all their contraction-loop loads from inline assembly and wait with their
own counts.
"""
import os
import shutil

import pytest

from mxfp4_mixture_experts_router_amd import isa_check


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not (os.path.exists(isa_check.HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("isa")
    return {src: isa_check.device_asm(src, str(d / (src + ".s")))
            for src in (isa_check.STREAM_SRC, isa_check.GROUPED_SRC)}


def test_stream_copies_wait_counts_the_younger_loads(asm):
    assert isa_check.stream_problems(asm[isa_check.STREAM_SRC]) == []


def test_grouped_gemm_waits_are_its_own(asm):
    assert isa_check.grouped_problems(asm[isa_check.GROUPED_SRC]) == []


def test_checks_catch_a_changed_load_sequence(asm):
    """An extra ordinary load between the copies and the stream wait, a compiler-issued load
    or a foreign count inside a GEMM loop, and scratch use are each reported."""
    s = asm[isa_check.STREAM_SRC]
    wait = "s_waitcnt vmcnt(%d)" % (9 + 2 * isa_check.stream_unroll())
    i = s.index(wait)
    broken = s[:i] + "global_load_dword v0, v[0:1], off\n\t" + s[i:]
    assert any("loads between the copies" in p for p in isa_check.stream_problems(broken))

    g = asm[isa_check.GROUPED_SRC]
    j = g.index("v_mfma_scale_f32_16x16x128_f8f6f4")
    broken = g[:j] + "global_load_dword v0, v[0:1], off\n\ts_waitcnt vmcnt(5)\n\t" + g[j:]
    problems = isa_check.grouped_problems(broken)
    assert any("compiler-issued loads" in p for p in problems)
    assert any("not the kernel's own" in p for p in problems)
    broken = g[:j] + "scratch_load_dword v0, off, s0\n\t" + g[j:]
    assert any("scratch" in p for p in isa_check.grouped_problems(broken))
