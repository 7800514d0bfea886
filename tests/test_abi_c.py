"""The C ABI from C: tests/c/abi_host.c includes the public header as C99,
links the library and calls its host-side entry points (no GPU).  Its
figures must equal the Python binding's, and bad arguments must come back
as the documented codes."""
import os
import shutil
import subprocess

import pytest

import sparse_moe_ffn_amd as moe
from sparse_moe_ffn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def c_output(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib = moe.load_library()
    libdir = os.path.dirname(lib._name)
    exe = str(tmp_path_factory.mktemp("abi") / "abi_host")
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", libdir, "-lmoe_mi355x",
                    f"-Wl,-rpath,{libdir}", "-o", exe], check=True)
    run = subprocess.run([exe], check=True, capture_output=True, text=True)
    rows = {}
    for line in run.stdout.splitlines():
        key, *vals = line.split()
        rows.setdefault(key, []).append([int(v) for v in vals])
    return rows


def test_layout_from_c_matches_binding(c_output):
    for N, nbytes, block_m, max_tiles, ids_products, act, y in c_output["layout"]:
        p = moe.problem(N, 2048, 128, 8, 768, weight_layout=moe.MOE_LAYOUT_BLOCKED)
        lay = moe.moe_get_workspace_layout(p)
        assert moe.moe_workspace_size(p) == nbytes
        assert (lay["block_m"], lay["max_tiles"], lay["ids_products"], lay["act"], lay["y"]) == \
            (block_m, max_tiles, ids_products, act, y)
    [[rows, tiles]] = c_output["capacity"]
    assert (rows, tiles) == moe.moe_align_capacity(32768, 128, 320)


def test_error_codes_from_c(c_output):
    assert c_output["top_k_above_E"] == [[B.MOE_EINVAL]]
    assert c_output["top_k_above_limit"] == [[B.MOE_EUNSUPPORTED]]
    assert c_output["null_problem"] == [[B.MOE_EINVAL]]
    assert c_output["forward_null_tensors"] == [[B.MOE_EINVAL]]
    assert c_output["last_error_set"] == [[1]]
