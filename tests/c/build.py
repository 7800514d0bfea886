"""Build the C caller of the whole block (tests/c/forward_gpu) against the
in-tree library: ``python tests/c/build.py``.  The binary finds the library
through a path relative to itself, so the tree can move."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "forward_gpu")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def c_compiler():
    return shutil.which("gcc") or shutil.which("cc")


def build() -> str:
    cc = c_compiler()
    if cc is None:
        raise RuntimeError("no C compiler")
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "forward_gpu.c"), "-o", EXE + ".tmp",
           "-L", os.path.join(ROOT, "sparse_moe_ffn_amd"), "-lmoe_mi355x", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../sparse_moe_ffn_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
