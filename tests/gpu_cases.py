"""Shared set-up of the GPU parity tests and the bench: a workload's seeded
inputs on the GPU, the HIP layer built from them, and the oracle's view of
the same data (host copies, fetched per expert on demand)."""

from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import oracle as O
import synth

# Reduced shapes with the recipes of the full workloads: several M tiles per
# expert, ragged tails, and every mode.  Full sizes are in synth.WORKLOADS.
REDUCED = {
    "tiny_bf16": synth.get("tiny_bf16"),
    "qwen3_30b_a3b_ptpc": synth.get("qwen3_30b_a3b_ptpc"),
    "qwen3_235b_prefill_ptpc_r": synth.get("qwen3_235b_prefill_ptpc").replace(T=1000, D=1024, I=512, E=32),
    "qwen3_235b_decode_ptpc": synth.get("qwen3_235b_decode_ptpc"),
    "deepseek_r1_block_fp8_r": synth.get("deepseek_r1_block_fp8").replace(T=300, D=1024, I=256, E=32),
    "bf16_multi_tile_r": synth.get("tiny_bf16").replace(T=700, D=512, I=256, E=16, k=4),
    # small batches for the weight-streaming kernels (block_m 16: T <= 64, or at most 24 rows per expert)
    "deepseek_r1_block_fp8_small": synth.get("deepseek_r1_block_fp8").replace(T=40, D=1024, I=256, E=32),
    "qwen3_235b_decode_ptpc_t64": synth.get("qwen3_235b_decode_ptpc").replace(T=64, D=1024, I=512, E=16),
    "bf16_small_t20": synth.get("tiny_bf16").replace(T=20, D=512, I=256, E=16, k=4),
    # weight rows that do not split into 4 x 128 per wave column (2I = 768,
    # D = 1280): the PTPC kernels fall back to 64-row wave tiles
    "qwen3_30b_a3b_ptpc_i384": synth.get("qwen3_30b_a3b_ptpc").replace(T=200, D=1280, I=384, E=16),
    # 512-expert top-10 layer with a shared expert, reduced: top-10 of 64
    "e512_top10_shared_r": synth.get("e512_top10_shared_ptpc").replace(T=500, D=1024, I=256, E=64),
    # MXFP4 (A4W4) layers: several tiles and ragged tails, softmax and
    # grouped routing with a shared expert, a small batch (32-row tiles)
    "qwen3_235b_prefill_mxfp4_r": synth.get("qwen3_235b_prefill_mxfp4").replace(T=1000, D=1024, I=512, E=32),
    "deepseek_r1_mxfp4_r": synth.get("deepseek_r1_mxfp4").replace(T=300, D=1024, I=256, E=32),
    "deepseek_r1_mxfp4_small": synth.get("deepseek_r1_mxfp4").replace(T=40, D=1024, I=256, E=32),
    # the MXFP4 decode batch (T=32 over 128 experts: the weight-streaming launch of 32 rows per expert)
    "qwen3_235b_decode_mxfp4_r": synth.get("qwen3_235b_decode_mxfp4").replace(D=1024, I=512),
    # the weight-streaming path's in-kernel permutation at its limits: 256
    # tokens, top-16 plus the shared expert (4352 rows) over 1023 + 1 experts
    "perm_limits_t256_k16": synth.get("e512_top10_shared_ptpc").replace(T=256, D=256, I=128, E=1023, k=16),
}


def say(*a) -> None:
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def spec_of(w: synth.Workload) -> O.LayerSpec:
    return O.LayerSpec(D=w.D, I=w.I, E=w.E, top_k=w.k, n_shared=w.n_shared, scoring=w.scoring,
                       n_groups=w.n_groups, topk_groups=w.topk_groups, route_scale=w.route_scale, quant=w.quant)


@dataclass
class Case:
    w: synth.Workload
    layer: object                 # moe_layer_router_amd.MoELayer
    x: torch.Tensor               # [T, D] bf16 on the GPU
    logits: Optional[torch.Tensor]
    router_w: Optional[torch.Tensor]
    w13: torch.Tensor             # bf16 masters on the GPU
    w2: torch.Tensor
    spec: O.LayerSpec
    bank: O.ExpertBank

    def x_np(self) -> np.ndarray:
        return synth.bf16_to_f32_np(self.x)

    def logits_np(self) -> Optional[np.ndarray]:
        return None if self.logits is None else self.logits.cpu().numpy()


def build_case(w: synth.Workload, device="cuda", cache_experts: bool = True, keep_masters: bool = True,
               weight_layout=None) -> Case:
    import moe_layer_router_amd as mlr
    x = synth.gen_x(w, device)
    logits = synth.gen_logits(w, device)
    router_w = synth.gen_router_w(w, device) if w.router == "gemm" else None
    w13, w2 = synth.gen_masters(w, device)
    layer = mlr.MoELayer.from_masters(w13, w2, w.quant, router_w=router_w, E=w.E, top_k=w.k,
                                      n_shared=w.n_shared, scoring=w.scoring, n_groups=w.n_groups,
                                      topk_groups=w.topk_groups, route_scale=w.route_scale,
                                      weight_layout=weight_layout)
    spec = spec_of(w)

    def master(e):
        return synth.bf16_to_f32_np(w13[e]), synth.bf16_to_f32_np(w2[e])
    bank = O.ExpertBank(spec, master, cache=cache_experts)
    if not keep_masters and w.quant != "bf16":
        # the layer holds its own quantized copies; free the masters early
        # (the oracle then needs them again: regenerate per expert)
        def master_regen(e):
            a, b = synth.gen_expert_master(w, e, device)
            return synth.bf16_to_f32_np(a), synth.bf16_to_f32_np(b)
        bank = O.ExpertBank(spec, master_regen, cache=cache_experts)
        del w13, w2
        torch.cuda.empty_cache()
        w13 = w2 = None
    return Case(w, layer, x, logits, router_w, w13, w2, spec, bank)


def check_router_logits(lg_gpu: np.ndarray, x_np: np.ndarray, wr_np: np.ndarray) -> np.ndarray:
    """The GPU's router logits against the oracle's float64 projection.  The
    per-token fp64 kernel (small batches) rounds once, so it is within one
    fp32 ulp; the fused matrix-core kernel has exact products and fp32
    accumulation, so |error| <= n u sum_d |x[d] w[d]| for n additions; both
    are inside 1e-6 sum_d |x[d] w[d]| plus half an ulp of the stored value.
    Returns the oracle's logits."""
    ref = O.router_logits(x_np, wr_np)
    cond = np.abs(x_np.astype(np.float64)) @ np.abs(wr_np.astype(np.float64)).T
    err = np.abs(lg_gpu.astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= 1e-6 * cond + np.abs(ref.astype(np.float64)) * 2.0 ** -24), float(np.max(err / cond))
    return ref


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """E2M1 codes [rows, K] (0..15) as the GPU stores them: [rows, K/2] bytes,
    element 2i in the low nibble of byte i."""
    c = np.asarray(codes, np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, np.uint8)
    out = np.empty((b.shape[0], 2 * b.shape[1]), np.uint8)
    out[:, 0::2] = b & 15
    out[:, 1::2] = b >> 4
    return out


def quant_act_ref(quant: str, a: np.ndarray):
    """The oracle's quantization of activation rows in the GPU's storage
    layout: (codes, scales) with codes [rows, K] e4m3 or [rows, K/2] packed
    E2M1, scales fp32 [rows] / [rows, K/128] or E8M0 bytes [rows, K/32]."""
    if quant == "mxfp4":
        q, sc = O.mxfp4_quant(a, 32)
        return pack_nibbles(q), sc
    return O.quant_rows(a, 128 if quant == "block128_fp8" else 0)


def dequant_act(quant: str, q: np.ndarray, sc: np.ndarray) -> np.ndarray:
    """float64 values of GPU-layout activation codes (see quant_act_ref)."""
    if quant == "mxfp4":
        return O.mxfp4_dequant(unpack_nibbles(q), sc, 32)
    return O.dequant_rows(q, sc, 128 if quant == "block128_fp8" else 0)


def same_scales(a: np.ndarray, b: np.ndarray) -> bool:
    """Bitwise equality of fp32 or E8M0 scale arrays."""
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.float32:
        return a.shape == b.shape and np.array_equal(a.view(np.uint32), np.asarray(b, np.float32).view(np.uint32))
    return np.array_equal(a, b)


def rel_l2(a, b) -> float:
    return O.relative_l2(np.asarray(a, np.float64), np.asarray(b, np.float64))


def tol_of(quant: str) -> float:
    """Relative L2 bound on y: 2e-3 for the bf16 path, 1e-2 for the quantized
    (FP8 and MXFP4) paths."""
    return 2e-3 if quant == "bf16" else 1e-2


# Bound on one token's y against the oracle end to end in the quantized
# modes.  The GPU's act (fp32 sums) and the oracle's (fp64) round to the same
# bf16 except where a sum lies next to a rounding boundary; when that is a
# row's largest element the row's scale moves by 2^-8 and about
# 2^-8 / 2^-3.5 = 1/23 of its e4m3 codes move by one step (2^-4 .. 2^-3 of
# their value): about 2e-2 of that row's contribution, which can carry most
# of a token's y.  Over many tokens such rows are rare and the tensor stays
# within tol_of; a token alone is held to this bound, and tightly to the
# oracle's down GEMM and combine fed the GPU's own act codes.
TOKEN_TOL_FP8 = 5e-2


def zero_pad_rows(perm: dict, block_m: int, use_counts: bool = True) -> np.ndarray:
    """Boolean mask over rows [0, offsets[-1]) of the pad rows a GEMM writes
    as 0: every pad row for the streaming kernels (block_m 16) or without
    expert counts; otherwise the pads inside a 32-row tile that also holds
    routed rows (pad-only tiles are not written and their rows are
    unspecified, as every pad row's contents are for the layer)."""
    offs = perm["offsets"].cpu().numpy()
    cnts = perm["counts"].cpu().numpy()
    mask = np.zeros(int(offs[-1]), bool)
    for e in range(len(cnts)):
        lo, hi, end = int(offs[e]), int(offs[e]) + int(cnts[e]), int(offs[e + 1])
        top = end if (block_m == 16 or not use_counts) else min(end, lo + -(-int(cnts[e]) // 32) * 32)
        mask[hi:top] = True
    return mask

