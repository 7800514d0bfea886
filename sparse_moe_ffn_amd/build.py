"""Build the HIP library in-tree: ``python -m sparse_moe_ffn_amd.build``.

Compiles every source under ``csrc/`` for gfx950 into
``sparse_moe_ffn_amd/libmoe_mi355x.so`` (one hipcc call per source, then one
link).  Packed-FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
SOURCES = ["route.hip", "align.hip", "grouped_gemm.hip", "combine.hip", "norm.hip", "peak_probe.hip", "moe_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False, jobs: int = 4) -> str:
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="moe_build_")
    try:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmd = [cc] + flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len([p for _, p in procs if p.poll() is None]) >= jobs:
                procs[-jobs][1].wait()
        errors = []
        for src, p in procs:
            out = p.communicate()[0].decode(errors="replace")
            noise = [l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip()]
            if p.returncode != 0:
                errors.append(f"--- {src}\n" + "\n".join(noise))
            elif noise and verbose:
                print("\n".join(noise))
        if errors:
            raise RuntimeError("HIP build failed:\n" + "\n".join(errors))
        tmp_lib = LIB + ".tmp"
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, capture_output=not verbose)
        os.replace(tmp_lib, LIB)
        return LIB
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
