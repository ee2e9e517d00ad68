"""End-to-end GPU parity of moe_forward against the oracle: routing,
permutation and x codes bit-exact; y within relative L2 2e-3 (bf16 path) or
1e-2 (FP8 paths); determinism and token-order invariance, on reduced shapes
with several tiles and ragged tails in every mode and tile size (the full
sizes are in test_gpu_fullsize.py)."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_cases import (REDUCED, TOKEN_TOL_FP8, build_case, check_router_logits, dequant_act, quant_act_ref, rel_l2,
                              same_scales, say, tol_of)

pytestmark = pytest.mark.gpu

mlr = pytest.importorskip("moe_layer_router_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mlr.lib()


def _run(c, block_m=0):
    y = c.layer.forward(c.x, c.logits, block_m=block_m)
    torch.cuda.synchronize()
    return y, c.layer.intermediates(c.w.T, block_m)


def _check_exact(inter, ref, quant):
    assert np.array_equal(inter["topk_ids"].cpu().numpy(), ref["ids"])
    p = ref["perm"]
    for key in ("counts", "offsets", "sorted_ids", "block_expert", "inv_perm"):
        assert np.array_equal(inter[key].cpu().numpy(), p[key]), key
    if quant != "bf16":
        assert np.array_equal(inter["xq"].cpu().numpy(), ref["xq"])
        assert np.array_equal(inter["xs"].cpu().numpy().view(np.uint32), ref["sx"].view(np.uint32))


@pytest.mark.parametrize("name,block_m", [("tiny_bf16", 0), ("tiny_bf16", 64), ("bf16_multi_tile_r", 0),
                                          ("qwen3_30b_a3b_ptpc", 0), ("qwen3_30b_a3b_ptpc", 128),
                                          ("qwen3_235b_prefill_ptpc_r", 0), ("qwen3_235b_prefill_ptpc_r", 32),
                                          ("qwen3_235b_prefill_ptpc_r", 256), ("bf16_multi_tile_r", 256),
                                          ("qwen3_30b_a3b_ptpc_i384", 0),
                                          ("qwen3_235b_decode_ptpc", 0), ("deepseek_r1_block_fp8_r", 0),
                                          ("deepseek_r1_block_fp8_r", 32), ("deepseek_r1_block_fp8_r", 64),
                                          ("deepseek_r1_block_fp8_r", 128), ("deepseek_r1_block_fp8_r", 256),
                                          ("deepseek_r1_block_fp8_small", 0),
                                          ("qwen3_235b_decode_ptpc_t64", 0), ("qwen3_235b_decode_ptpc", 32),
                                          ("bf16_small_t20", 0), ("qwen3_235b_prefill_ptpc_r", 16),
                                          ("deepseek_r1_block_fp8_r", 16), ("e512_top10_shared_r", 0),
                                          ("e512_top10_shared_r", 128), ("e512_top10_shared_r", 16),
                                          ("qwen3_235b_prefill_ptpc_r", 192), ("deepseek_r1_block_fp8_r", 192),
                                          ("perm_limits_t256_k16", 0)])
def test_forward_matches_oracle(name, block_m):
    w = REDUCED[name]
    say("forward", name, block_m)
    c = build_case(w)
    y, inter = _run(c, block_m)
    B = inter["block_m"]
    lg = c.logits_np()
    if w.router == "gemm":
        # routing is bit-exact given the same fp32 logits: the oracle routes
        # the GPU's logits once they are within the projection's bound
        lg = inter["logits"].cpu().numpy()
        check_router_logits(lg, c.x_np(), c.router_w.cpu().numpy())
    ref = O.moe_forward(c.spec, c.bank, c.x_np(), lg, block_m=B)
    _check_exact(inter, ref, w.quant)
    err = rel_l2(y.float().cpu().numpy(), ref["y"])
    say("rel_l2", err)
    assert err <= tol_of(w.quant)
    total = int(ref["perm"]["offsets"][-1])
    real = ref["perm"]["sorted_ids"][:total] != w.T * (w.k + w.n_shared)     # pad rows are unspecified
    assert rel_l2(inter["act"][:total].float().cpu().numpy()[real], ref["act"][:total][real]) < 2e-3


@pytest.mark.parametrize("name,block_m", [("qwen3_235b_decode_ptpc", 0), ("deepseek_r1_block_fp8_small", 0),
                                          ("qwen3_235b_prefill_ptpc_r", 0), ("deepseek_r1_block_fp8_r", 16)])
def test_act_codes_are_the_quantized_act(name, block_m):
    """The act codes the down GEMM reads (row-major for the tiled GEMMs, in
    16-row x 128-byte blocks for the streaming one) are the oracle's
    quantization of the GPU's own act, bit for bit, on every routed row."""
    w = REDUCED[name]
    say("act codes", name, block_m)
    c = build_case(w)
    _, inter = _run(c, block_m)
    total = int(inter["offsets"][-1].item())
    real = inter["sorted_ids"][:total].cpu().numpy() != w.T * (w.k + w.n_shared)
    act = inter["act"][:total].float().cpu().numpy()[real]
    q, sc = O.quant_rows(act, 128 if w.quant == "block128_fp8" else 0)
    assert np.array_equal(inter["aq"][:total].cpu().numpy()[real], q)
    assert np.array_equal(inter["as"][:total].cpu().numpy()[real].view(np.uint32), sc.view(np.uint32))


def test_forward_is_deterministic_and_row_independent():
    w = REDUCED["qwen3_235b_prefill_ptpc_r"]
    say("determinism")
    c = build_case(w)
    y1 = c.layer.forward(c.x, c.logits).clone()
    y2 = c.layer.forward(c.x, c.logits).clone()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    perm = torch.randperm(w.T, generator=torch.Generator().manual_seed(3)).cuda()
    y3 = c.layer.forward(c.x[perm].contiguous(), c.logits[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y1[perm].view(torch.int16), y3.view(torch.int16))


@pytest.mark.parametrize("name,block_m", [("qwen3_235b_prefill_ptpc_r", 0), ("qwen3_235b_prefill_ptpc_r", 16),
                                          ("deepseek_r1_block_fp8_r", 0), ("deepseek_r1_block_fp8_r", 16),
                                          ("qwen3_30b_a3b_ptpc", 32)])
def test_row_major_weights_match_blocked(name, block_m):
    """The same codes stored row-major or in 16-row x 128-byte blocks give
    bitwise the same layer output (only the addresses differ)."""
    w = REDUCED[name]
    say("weight layouts", name, block_m)
    cb = build_case(w)
    cr = build_case(w, weight_layout="rows")
    assert cb.layer.weight_layout == "blocked" and cr.layer.weight_layout == "rows"
    yb = cb.layer.forward(cb.x, cb.logits, block_m=block_m)
    yr = cr.layer.forward(cr.x, cr.logits, block_m=block_m)
    torch.cuda.synchronize()
    assert torch.equal(yb.view(torch.int16), yr.view(torch.int16))


@pytest.mark.parametrize("name", ["deepseek_r1_block_fp8_r", "qwen3_235b_decode_ptpc"])
def test_forward_small_batches_and_empty(name):
    """Batches of 1-7 tokens take the weight-streaming path whose gate/up
    kernel builds the permutation itself: routing, every permutation array
    and the x codes bit-exact; the act codes the oracle's quantization of
    the GPU's own act; y within tol_of of the oracle's down GEMM and combine
    fed those codes, and within the per-token bound end to end (a few
    tokens are a few rows, each able to carry an act scale one bf16 step
    off the oracle's)."""
    w = REDUCED[name]
    fp8 = w.quant != "bf16"
    c = build_case(w)
    for T in (1, 2, 3, 7):
        say("small batch", name, T)
        x, lg = c.x[:T].contiguous(), c.logits[:T].contiguous()
        y = c.layer.forward(x, lg)
        torch.cuda.synchronize()
        inter = c.layer.intermediates(T)
        assert inter["block_m"] == 16
        act = inter["act"].float().cpu().numpy()
        aq = inter["aq"].cpu().numpy() if fp8 else None
        sc = inter["as"].cpu().numpy() if fp8 else None
        o_fed = np.zeros(tuple(inter["out_perm"].shape), np.float64)
        codes_bad = []

        def fed(e, lo, hi, w13, w2, rows):
            if fp8:
                q, s = quant_act_ref(w.quant, act[lo:hi])
                if not (np.array_equal(aq[lo:hi], q) and same_scales(sc[lo:hi], s)):
                    codes_bad.append(e)
                a_in = dequant_act(w.quant, aq[lo:hi], sc[lo:hi])
            else:
                a_in = act[lo:hi].astype(np.float64)
            o_fed[lo:hi] = O.expert_down(a_in, w2, fp8)

        ref = O.moe_forward(c.spec, c.bank, c.x_np()[:T], c.logits_np()[:T], block_m=16, on_expert=fed)
        _check_exact(inter, ref, w.quant)
        assert not codes_bad, codes_bad
        k, inv = w.k, ref["perm"]["inv_perm"].astype(np.int64)
        y_fed = O.combine(o_fed[inv[:T * k]].reshape(T, k, w.D), ref["w"],
                          o_fed[inv[T * k:]] if w.n_shared else None)
        y_np = y.float().cpu().numpy()
        say("y vs the oracle fed the GPU's act codes", rel_l2(y_np, y_fed), "end to end", rel_l2(y_np, ref["y"]))
        assert rel_l2(y_np, y_fed) <= tol_of(w.quant)
        assert rel_l2(y_np, ref["y"]) <= (TOKEN_TOL_FP8 if fp8 else tol_of(w.quant))
    y0 = c.layer.forward(c.x[:0], c.logits[:0])
    assert y0.shape == (0, w.D)


def test_forward_zero_tokens_rows_and_one_hot_routing():
    """All-zero x rows (amax 0 -> scale 1) and every token on one expert."""
    w = REDUCED["qwen3_235b_prefill_ptpc_r"].replace(T=300)
    say("zero rows / one expert")
    c = build_case(w)
    x = c.x.clone()
    x[::7] = 0
    lg = torch.full_like(c.logits, -5.0)
    lg[:, 3] = 5.0
    lg[:, 9] = 4.0
    y = c.layer.forward(x, lg)
    torch.cuda.synchronize()
    inter = c.layer.intermediates(w.T)
    ref = O.moe_forward(c.spec, c.bank, synth.bf16_to_f32_np(x), lg.cpu().numpy(), block_m=inter["block_m"])
    _check_exact(inter, ref, w.quant)
    assert rel_l2(y.float().cpu().numpy(), ref["y"]) <= tol_of(w.quant)
    assert np.all(y[::7].float().cpu().numpy() == 0)
