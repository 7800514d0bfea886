"""Seeded synthetic inputs for the sparse MoE FFN block.

This module draws tensors and nothing else: it holds none of the block's
arithmetic (no router product, softmax, top-k, grouping or SwiGLU).  Both the
GPU path and the CPU oracle read the tensors it returns, so it is the only code
they share.

Workloads (Qwen3-30B-A3B-shaped layers, plus the tiny-thinker shape of the
"M08 tiny thinker KV-cache greedy decode" page, section "真实数字": 6 experts,
top-2, hidden 64):

    tiny     N=8     H=64   E=6   k=2 I=128  fp32  std 0.05  renorm on
    decode   N=64    H=2048 E=128 k=8 I=768  bf16  std 0.02  renorm on
    prefill  N=4096  (same layer)                            renorm on
    skew     N=16384 (same layer), Zipf(1.2) expert load     renorm off
    talker   N=8192  (same layer) + shared SwiGLU I_s=2048   renorm on

Recipe: ``torch.Generator(device).manual_seed(seed)``; draws in the fixed order
x, router_w, w_gate_up, w_down, [shared_w_gate_up, shared_w_down,
shared_gate], each ``randn(fp32) * std`` (x: std 1) rounded once to the
workload dtype.  Tensors are drawn on the device that will use them (torch's
CPU and GPU generators give different streams for one seed, so a GPU run and a
CPU run of the same workload see different, equally valid, inputs; the oracle
always receives host copies of exactly the tensors the GPU read).

Skewed load: every token gets ``x[:, 0] = 1`` and router row e gets
``router_w[e, 0] = b_e``, so expert e's logit is b_e plus a zero-mean
Gaussian term of standard deviation std * sqrt(H - 1).  Eight experts get
b = -64 and are never chosen.  The other biases are fitted so that the
expected per-expert load follows Zipf(s = 1.2) over a seeded random ranking,
capped at N (an expert holds a token at most once); the fit uses only a
Gaussian model of the logits (see ``skew_biases``), never the block itself.
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass, replace

import numpy as np
import torch

__all__ = ["MoEConfig", "CONFIGS", "DENSE_LAYERS", "make_inputs", "make_dense_inputs", "make_norm_inputs",
           "skew_biases", "zipf_targets"]


@dataclass(frozen=True)
class MoEConfig:
    name: str
    N: int
    H: int
    E: int
    top_k: int
    I: int
    I_shared: int = 0
    dtype: str = "bf16"          # "bf16" or "f32": dtype of x, every weight and out
    norm_topk_prob: bool = True
    std: float = 0.02            # std of router / expert / shared weights
    x_std: float = 1.0
    seed: int = 0
    skew: bool = False           # Zipf(1.2) expert load with dead experts
    skew_dead: int = 8
    skew_s: float = 1.2

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def pairs(self) -> int:
        return self.N * self.top_k

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)

    def flops(self) -> float:
        """Algorithmic FLOPs of one block pass (padding not counted)."""
        f = 2.0 * self.N * self.H * self.E                      # router product
        f += 6.0 * self.N * self.top_k * self.H * self.I        # gate, up, down per pair
        if self.I_shared:
            f += 6.0 * self.N * self.H * self.I_shared + 2.0 * self.N * self.H
        return f


_LAYER = dict(H=2048, E=128, top_k=8, I=768, dtype="bf16", std=0.02)

CONFIGS = {
    "tiny": MoEConfig("tiny", N=8, H=64, E=6, top_k=2, I=128, dtype="f32", std=0.05),
    "decode": MoEConfig("decode", N=64, **_LAYER),
    "prefill": MoEConfig("prefill", N=4096, **_LAYER),
    "skew": MoEConfig("skew", N=16384, norm_topk_prob=False, skew=True, **_LAYER),
    "talker": MoEConfig("talker", N=8192, I_shared=2048, **_LAYER),
}


def _randn(shape, g, device, std, dtype):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def zipf_targets(n_live: int, total: int, cap: int, s: float) -> np.ndarray:
    """Water-filled Zipf loads: t_r = min(cap, C * r^-s), r = 1..n_live, sum = total."""
    r = np.arange(1, n_live + 1, dtype=np.float64)
    shape = r ** (-s)
    lo, hi = 0.0, float(total) * 4.0
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(cap, c * shape).sum() > total:
            hi = c
        else:
            lo = c
    return np.minimum(cap, 0.5 * (lo + hi) * shape)


def _inclusion_prob(b: np.ndarray, k: int, sigma: float, z: np.ndarray, wz: np.ndarray) -> np.ndarray:
    """P(expert e is among the k largest of b_j + sigma*Z_j), Z_j iid N(0,1).

    For each e and each quadrature node z of its own noise, the number of other
    experts above b_e + sigma*z is Poisson-binomial; a short recursion over the
    others gives P(count <= k-1).  Plain probability, not the block's routing.
    """
    from scipy.special import ndtr

    E = b.shape[0]
    thr = b[:, None] + sigma * z[None, :]                        # [E, Z]: e's own level
    dp = np.zeros((E, k, z.shape[0]))
    dp[:, 0, :] = 1.0
    for j in range(E):
        q = ndtr((b[j] - thr) / sigma)                           # P(j above e's level)
        q[j, :] = 0.0                                            # e does not race itself
        shifted = np.concatenate([np.zeros((E, 1, z.shape[0])), dp[:, :-1, :]], axis=1)
        dp = dp * (1.0 - q)[:, None, :] + shifted * q[:, None, :]
    return (dp.sum(axis=1) * wz[None, :]).sum(axis=1)


@functools.lru_cache(maxsize=8)
def _fit_live_biases(n_live: int, N: int, k: int, sigma: float, s: float) -> tuple:
    """Damped fixed point b += 0.35*log(target/load) on the Gaussian load model."""
    targets = zipf_targets(n_live, N * k, N, s)
    z = np.linspace(-7.0, 7.0, 141)
    wz = np.exp(-0.5 * z * z)
    wz /= wz.sum()
    b = np.log(targets / targets.max()) * 0.5
    for _ in range(60):
        load = N * _inclusion_prob(b, k, sigma, z, wz)
        b = b + 0.35 * np.log(targets / np.maximum(load, 0.5))
        b = b - b.max()
    return tuple(float(v) for v in b), tuple(float(v) for v in targets)


def skew_biases(cfg: MoEConfig, perm: torch.Tensor) -> torch.Tensor:
    """Per-expert logit offsets b_e for the skewed-load workload.

    ``perm`` (a seeded permutation of the experts) assigns Zipf ranks: the
    first ``E - skew_dead`` entries are ranks 1.., the rest are dead (b=-64).
    """
    n_live = cfg.E - cfg.skew_dead
    sigma = cfg.std * math.sqrt(cfg.H - 1) * cfg.x_std
    live, _ = _fit_live_biases(n_live, cfg.N, cfg.top_k, round(sigma, 6), cfg.skew_s)
    b = torch.full((cfg.E,), -64.0, dtype=torch.float64)
    b[perm[:n_live].cpu()] = torch.tensor(live, dtype=torch.float64)
    return b


def make_inputs(cfg: MoEConfig, device="cpu") -> dict:
    """All tensors of one workload, drawn with the recipe in the module doc."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)
    dt = cfg.torch_dtype
    N, H, E, I = cfg.N, cfg.H, cfg.E, cfg.I
    out = {}
    out["x"] = _randn((N, H), g, device, cfg.x_std, dt)
    out["router_w"] = _randn((E, H), g, device, cfg.std, dt)
    out["w_gate_up"] = _randn((E, 2 * I, H), g, device, cfg.std, dt)
    out["w_down"] = _randn((E, H, I), g, device, cfg.std, dt)
    if cfg.I_shared:
        Is = cfg.I_shared
        out["shared_w_gate_up"] = _randn((2 * Is, H), g, device, cfg.std, dt)
        out["shared_w_down"] = _randn((H, Is), g, device, cfg.std, dt)
        out["shared_gate"] = _randn((H,), g, device, cfg.std, dt)
    else:
        out["shared_w_gate_up"] = out["shared_w_down"] = out["shared_gate"] = None
    if cfg.skew:
        perm = torch.randperm(E, generator=g, device=device)
        b = skew_biases(cfg, perm)
        out["x"][:, 0] = 1.0
        out["router_w"][:, 0] = b.to(device=device, dtype=dt)
        out["skew_perm"] = perm
    return out


# Dense SwiGLU layers of hidden 2048 with I = 6144 = 8 * 768: the same work
# per token as the 8 routed experts of the MoE layer above.
DENSE_LAYERS = {
    "dense_decode": dict(N=64, H=2048, I=6144),
    "dense_prefill": dict(N=4096, H=2048, I=6144),
}


def make_dense_inputs(N, H, I, dtype="bf16", seed=0, std=0.02, device="cpu") -> dict:
    """x [N, H] (std 1), w_gate_up [2I, H] and w_down [H, I] (std `std`), drawn
    in that order, each randn * std rounded once to the dtype."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    return {"x": _randn((N, H), g, device, 1.0, dt), "w_gate_up": _randn((2 * I, H), g, device, std, dt),
            "w_down": _randn((H, I), g, device, std, dt)}


def make_norm_inputs(N, H, dtype="bf16", seed=0, device="cpu") -> dict:
    """Inputs of the residual add + RMSNorm: x [N, H] (the sub-layer output,
    std 1), residual [N, H] (std 1) and the norm weight [H] = 1 + 0.1 * randn,
    drawn in that order and rounded once to the dtype."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    x = _randn((N, H), g, device, 1.0, dt)
    residual = _randn((N, H), g, device, 1.0, dt)
    w = torch.randn((H,), generator=g, device=device, dtype=torch.float32).mul_(0.1).add_(1.0).to(dt)
    return {"x": x, "residual": residual, "weight": w}


def random_case(N, H, E, top_k, I, I_shared=0, dtype="bf16", norm_topk_prob=True,
                seed=0, std=None) -> MoEConfig:
    """A small ad-hoc workload (ragged sizes, edge cases) with the same recipe."""
    if std is None:
        std = 0.05 if dtype == "f32" else 0.02
    return MoEConfig(f"case_N{N}_H{H}_E{E}_k{top_k}_I{I}_s{I_shared}_{dtype}", N=N, H=H, E=E,
                     top_k=top_k, I=I, I_shared=I_shared, dtype=dtype,
                     norm_topk_prob=norm_topk_prob, std=std, seed=seed)
