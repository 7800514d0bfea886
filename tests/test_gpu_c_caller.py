"""The whole block called from C (tests/c/forward_gpu.c): the program
allocates device memory with hipMalloc, sizes the workspace with
moe_workspace_size and calls moe_forward on the default stream.  Its output
must equal the Python binding's bit for bit (same library, same inputs) and
the oracle's within the tolerance."""
import importlib.util
import os
import subprocess

import numpy as np
import pytest
import torch

import sparse_moe_ffn_amd as moe
from oracle import moe_oracle as O
from sparse_moe_ffn_amd.inputs import CONFIGS, make_inputs, random_case

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c", "forward_gpu")
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    if not os.path.exists(EXE):                      # normally built beside the library (tests/c/build.py)
        spec = importlib.util.spec_from_file_location("c_caller_build", os.path.join(HERE, "c", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


def raw(t):
    """Raw element bytes of a CPU tensor (bfloat16 as its 16-bit pattern)."""
    t = t.detach().cpu().contiguous()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).numpy().tobytes()


CASES = [CONFIGS["tiny"],
         random_case(600, 128, 16, 2, 64, I_shared=64, dtype="bf16", seed=3),     # grouped tiles, shared expert
         random_case(64, 256, 16, 4, 128, dtype="bf16", seed=4)]                  # the ids products


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_forward_from_c(cfg, tmp_path):
    t = make_inputs(cfg, DEV)
    shared = cfg.I_shared > 0
    names = ["x", "router_w", "w_gate_up", "w_down"] + (["shared_w_gate_up", "shared_w_down", "shared_gate"]
                                                        if shared else [])
    for n in names:
        (tmp_path / f"{n}.bin").write_bytes(raw(t[n]))
    dtype = 1 if cfg.dtype == "bf16" else 0
    (tmp_path / "meta.txt").write_text(f"{cfg.N} {cfg.H} {cfg.E} {cfg.top_k} {cfg.I} {cfg.I_shared} "
                                       f"{int(cfg.norm_topk_prob)} {dtype}\n")
    print(f"running {EXE} on {cfg.name}", flush=True)
    run = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    out_c = np.frombuffer((tmp_path / "out.bin").read_bytes(), dtype=np.int16 if dtype else np.float32)
    out_c = torch.from_numpy(out_c.copy()).view(t["x"].dtype).reshape(cfg.N, cfg.H)

    out_py = moe.moe_forward(t["x"], t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob,
                             t["shared_w_gate_up"], t["shared_w_down"], t["shared_gate"])
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_py.cpu())

    h = {k: (v.float().cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    sh = {"w_gate_up": h["shared_w_gate_up"], "w_down": h["shared_w_down"], "gate": h["shared_gate"]} if shared else None
    ref, (_, _, _, margin) = O.moe_forward(h["x"], h["router_w"], h["w_gate_up"], h["w_down"], cfg.top_k,
                                           cfg.norm_topk_prob, shared=sh)
    keep = margin >= 1e-6
    err = float(np.abs(out_c.float().numpy()[keep] - ref[keep]).max())
    tol = O.tolerance(ref[keep], cfg.dtype)
    assert err <= tol, (err, tol)
