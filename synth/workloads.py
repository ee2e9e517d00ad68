"""Layer shapes and seeded input draws.

Layer shapes that stand in for the serving workloads the pages discuss
(Qwen3-30B-A3B and Qwen3-235B-A22B MoE layers with PTPC-FP8, the
DeepSeek-R1 MoE layer with blockwise FP8, hidden 7168 and top-8 routing, and
a 512-expert top-10 layer with a shared expert), plus a tiny bf16 layer.  No dataset or trained weight is used: every tensor is
a seeded draw from ``torch.Generator`` on the device the caller names, so the
HIP path and the oracle see the same values (the GPU-side tests copy what the
oracle needs back to the host).

Recipes (sigma is a standard deviation):
  x ~ N(0, 1) rounded to bf16;
  tiny layer: router weight ~ N(0, 0.02) fp32 and the logits come from the
    router projection; expert weights ~ N(0, 1/sqrt(D)) for W13 and W2;
  other layers: logits are drawn directly, fp32 [T, E]:
    "normal"       N(0, 1) (near-uniform routing),
    "normal_bias"  N(0, 1) + b_e with b_e ~ N(0, 0.5) (mild load imbalance),
    "zipf"         N(0, 1) - s * ln(rank_e), rank a seeded permutation of
                   1..E, so expert popularity falls off as rank^-s (s = 1.2);
    master expert weights ~ N(0, 1/sqrt(fan_in)) (W13: D, W2: I) rounded to
    bf16; the FP8 layers quantize these masters.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "get", "seed_of", "gen_x", "gen_logits",
           "gen_router_w", "gen_expert_master", "gen_masters", "bf16_to_f32_np",
           "gen_uniform_bf16", "gen_normal_f32"]


@dataclass(frozen=True)
class Workload:
    name: str
    cid: int
    T: int
    D: int
    E: int
    k: int
    I: int
    quant: str                     # "bf16" | "ptpc_fp8" | "block128_fp8" | "mxfp4"
    scoring: str = "softmax"       # or "sigmoid_grouped"
    n_groups: int = 1
    topk_groups: int = 1
    route_scale: float = 1.0
    n_shared: int = 0
    router: str = "logits"         # "gemm": logits = x Wr^T ; "logits": drawn
    logit_recipe: str = "normal"   # "normal" | "normal_bias" | "zipf"
    zipf_s: float = 1.2
    bias_std: float = 0.5
    w_std_rule: str = "fan_in"     # "fan_in" | "sqrt_D"

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def E_total(self) -> int:
        return self.E + self.n_shared

    def w13_std(self) -> float:
        return 1.0 / np.sqrt(self.D)

    def w2_std(self) -> float:
        return 1.0 / np.sqrt(self.D if self.w_std_rule == "sqrt_D" else self.I)

    def flops(self) -> float:
        """Algorithmic FLOPs of the expert GEMMs over unpadded routed rows."""
        rows = self.T * (self.k + self.n_shared)
        f = 2.0 * rows * (2 * self.I * self.D + self.D * self.I)
        if self.router == "gemm":
            f += 2.0 * self.T * self.E * self.D
        return f


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_bf16", 1, T=64, D=256, E=8, k=2, I=128, quant="bf16",
                 router="gemm", w_std_rule="sqrt_D"),
        Workload("qwen3_30b_a3b_ptpc", 2, T=256, D=2048, E=128, k=8, I=768,
                 quant="ptpc_fp8", logit_recipe="normal"),
        Workload("qwen3_235b_prefill_ptpc", 3, T=8192, D=4096, E=128, k=8, I=1536,
                 quant="ptpc_fp8", logit_recipe="normal_bias"),
        Workload("qwen3_235b_decode_ptpc", 4, T=32, D=4096, E=128, k=8, I=1536,
                 quant="ptpc_fp8", logit_recipe="zipf"),
        Workload("deepseek_r1_block_fp8", 5, T=4096, D=7168, E=256, k=8, I=2048,
                 quant="block128_fp8", scoring="sigmoid_grouped", n_groups=8,
                 topk_groups=4, route_scale=2.5, n_shared=1),
        # 512 small experts, top-10 (a k that is not a power of two) plus one
        # always-on shared expert: the expert layout of the Qwen 3.5 TPU
        # page, at an 8192-token prefill (81,920 routed rows)
        Workload("e512_top10_shared_ptpc", 6, T=8192, D=4096, E=512, k=10, I=1024,
                 quant="ptpc_fp8", n_shared=1, logit_recipe="normal"),
        # the Qwen3-235B-shaped prefill layer routed by its own router gate
        # (router weight ~ N(0, 0.02), logits = x . Wr^T) instead of given logits
        Workload("qwen3_235b_prefill_router", 7, T=8192, D=4096, E=128, k=8, I=1536,
                 quant="ptpc_fp8", router="gemm"),
        # MXFP4 (A4W4) expert arithmetic on the Qwen3-235B-shaped prefill and
        # the DeepSeek-R1-shaped layer: 4-bit activations and weights with
        # E8M0 scales per 32 elements
        Workload("qwen3_235b_prefill_mxfp4", 8, T=8192, D=4096, E=128, k=8, I=1536,
                 quant="mxfp4", logit_recipe="normal_bias"),
        Workload("deepseek_r1_mxfp4", 9, T=4096, D=7168, E=256, k=8, I=2048,
                 quant="mxfp4", scoring="sigmoid_grouped", n_groups=8,
                 topk_groups=4, route_scale=2.5, n_shared=1),
        # the 32-token decode batch of the Qwen3-235B shape in MXFP4
        Workload("qwen3_235b_decode_mxfp4", 10, T=32, D=4096, E=128, k=8, I=1536,
                 quant="mxfp4", logit_recipe="zipf"),
    ]
}

# tensor ids in the seed
_X, _NOISE, _BIAS, _WR, _W13, _W2, _RANK = 0, 1, 2, 3, 4, 5, 6


def get(name: str) -> Workload:
    return WORKLOADS[name]


def seed_of(cid: int, tensor: int, expert: int = 0, salt: int = 0) -> int:
    """Distinct 63-bit seed per (workload, tensor, expert, salt)."""
    return ((salt & 0xFFFF) << 44) | ((cid & 0xFF) << 36) | ((tensor & 0xF) << 32) | (expert & 0xFFFFFFFF)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def gen_normal_f32(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)
    return t * std if std != 1.0 else t


def gen_uniform_bf16(shape, lo: float, hi: float, seed: int, device="cpu") -> torch.Tensor:
    t = torch.rand(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)
    return (t * (hi - lo) + lo).to(torch.bfloat16)


def gen_x(w: Workload, device="cpu", salt: int = 0) -> torch.Tensor:
    """Hidden states x ~ N(0,1), bf16 [T, D]."""
    return gen_normal_f32((w.T, w.D), 1.0, seed_of(w.cid, _X, 0, salt), device).to(torch.bfloat16)


def gen_router_w(w: Workload, device="cpu") -> torch.Tensor:
    """Router weight ~ N(0, 0.02), fp32 [E, D]."""
    return gen_normal_f32((w.E, w.D), 0.02, seed_of(w.cid, _WR), device)


def gen_logits(w: Workload, device="cpu", salt: int = 0) -> Optional[torch.Tensor]:
    """Router logits fp32 [T, E] per the workload's recipe (None: router GEMM)."""
    if w.router == "gemm":
        return None
    noise = gen_normal_f32((w.T, w.E), 1.0, seed_of(w.cid, _NOISE, 0, salt), device)
    if w.logit_recipe == "normal":
        return noise
    if w.logit_recipe == "normal_bias":
        b = gen_normal_f32((w.E,), w.bias_std, seed_of(w.cid, _BIAS), device)
        return noise + b[None, :]
    if w.logit_recipe == "zipf":
        g = _gen("cpu", seed_of(w.cid, _RANK))
        rank = (torch.randperm(w.E, generator=g) + 1).to(torch.float64)
        b = (-w.zipf_s * torch.log(rank)).to(torch.float32).to(device)
        return noise + b[None, :]
    raise ValueError(w.logit_recipe)


def gen_expert_master(w: Workload, e: int, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """Master weights of expert e (e = E is the shared expert), bf16:
    W13 [2I, D] (gate rows 0..I-1, up rows I..2I-1) and W2 [D, I]."""
    w13 = gen_normal_f32((2 * w.I, w.D), w.w13_std(), seed_of(w.cid, _W13, e), device)
    w2 = gen_normal_f32((w.D, w.I), w.w2_std(), seed_of(w.cid, _W2, e), device)
    return w13.to(torch.bfloat16), w2.to(torch.bfloat16)


def gen_masters(w: Workload, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """All master weights stacked: W13 [E', 2I, D], W2 [E', D, I], bf16."""
    Ep = w.E_total
    w13 = torch.empty((Ep, 2 * w.I, w.D), dtype=torch.bfloat16, device=device)
    w2 = torch.empty((Ep, w.D, w.I), dtype=torch.bfloat16, device=device)
    for e in range(Ep):
        a, b = gen_expert_master(w, e, device)
        w13[e].copy_(a)
        w2[e].copy_(b)
    return w13, w2


def bf16_to_f32_np(t: torch.Tensor) -> np.ndarray:
    """Host float32 numpy copy of a bf16 tensor (exact widening)."""
    return t.detach().to("cpu").to(torch.float32).numpy()
