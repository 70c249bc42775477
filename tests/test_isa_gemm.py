"""The GEMM's LDS-DMA loads set m0 from inline assembly, which the compiler is
not told about.  That is sound only while no compiler-generated instruction in
the kernel reads or writes m0; this test compiles the kernel source to gfx950
assembly with the library's own flags and checks exactly that: every m0
reference is one of the asm sequences `s_mov_b32 m0, sN; s_nop 0;
global_load_lds_*`."""
import os
import re
import subprocess
import tempfile

import pytest

from precision_quantization_block_amd import _build

SRC = os.path.join(_build.CSRC, "k_gemm.hip")


@pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="hipcc not available")
def test_only_the_dma_asm_touches_m0():
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k_gemm.s")
        flags = [f for f in _build.FLAGS if f != "-fPIC"]
        subprocess.run([_build.HIPCC, *flags, "-S", "--offload-device-only", SRC, "-o", out],
                       check=True, capture_output=True)
        lines = [ln.strip() for ln in open(out) if not ln.strip().startswith(";")]
    uses = [i for i, ln in enumerate(lines) if re.search(r"\bm0\b", ln)]
    assert uses, "expected the DMA sequences to set m0"
    for i in uses:
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", lines[i]), lines[i]
        assert lines[i + 1] == "s_nop 0", lines[i + 1]
        assert lines[i + 2].startswith("global_load_lds_dword"), lines[i + 2]
