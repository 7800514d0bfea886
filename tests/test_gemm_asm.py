"""The grouped GEMM's LDS DMAs are inline assembly that sets M0 and issues
global_load_lds_dwordx4 in one statement.  The compiler treats M0 as a
reserved register and ignores it in an asm clobber list, so the DMAs are
only safe while no compiler-generated code uses M0 in these kernels.  This
test compiles the GEMM source to gfx950 assembly (CPU only) and checks that
every use of M0 is one of those pairs, each M0 write directly followed by
its DMA."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "sparse_moe_ffn_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_m0_is_only_used_by_the_lds_dmas():
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not found")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gg.s")
        subprocess.run([cc, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                        "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only",
                        "-S", os.path.join(CSRC, "grouped_gemm.hip"), "-o", out],
                       check=True, capture_output=True, timeout=600)
        lines = [l.strip() for l in open(out) if l.strip() and not l.strip().startswith(("//", ";", "."))]
    n_dma = 0
    for i, l in enumerate(lines):
        if "m0" not in l.replace(",", " ").split():
            continue
        if l.startswith("s_mov_b32 m0,"):
            assert lines[i + 1].startswith("global_load_lds_dwordx4"), f"M0 write not followed by its DMA: {l}"
            n_dma += 1
        else:
            raise AssertionError(f"compiler-generated use of M0: {l}")
    dmas = sum(1 for l in lines if l.startswith("global_load_lds_dwordx4"))
    assert n_dma > 0 and n_dma == dmas
