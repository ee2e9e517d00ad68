"""GPU parity of the MXFP4 (A4W4) path: the row quantizer for activations
and weights bit-exact against the oracle (every bf16 value, zero blocks,
both weight layouts), and moe_forward on reduced MXFP4 layers (among them
a 32-token decode batch over 128 experts) in every tile size and the
weight-streaming path: routing, permutation and x codes bit-exact, act within 2e-3 relative
L2 on routed rows, act codes and scales the oracle's quantization of the
GPU's act, out_perm against the oracle's down GEMM fed those codes, y within
1e-2 (the quantized paths' bound)."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_cases import (REDUCED, build_case, dequant_act, pack_nibbles, quant_act_ref, rel_l2, say,
                             tol_of, zero_pad_rows)

pytestmark = pytest.mark.gpu

mlr = pytest.importorskip("moe_layer_router_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mlr.lib()


def test_mx_rows_every_bf16_value():
    """Every finite bf16 value, 31 per block with a block maximum of 6 * 2^k
    for several k (so each value is scaled by a power of two from -8 to 8
    and goes through the E2M1 rounding at every magnitude), plus all-zero
    and single-value blocks."""
    say("mx every bf16")
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals)]
    rows = []
    for k in (-8, -3, 0, 4, 8):
        top = np.float32(6.0 * 2.0 ** k)
        v = vals[np.abs(vals) <= top]
        nb = -(-v.size // 31)
        blk = np.zeros((nb, 32), np.float32)
        blk[:, 0] = top
        flat = blk[:, 1:].reshape(-1)
        flat[:v.size] = v
        blk[:, 1:] = flat.reshape(nb, 31)
        rows.append(blk.reshape(-1))
    x = np.concatenate(rows)
    x = np.concatenate([x, np.zeros(64, np.float32), np.array([3.0] + [0.0] * 31, np.float32)])
    K = 4096
    x = np.concatenate([x, np.zeros((-x.size) % K, np.float32)]).reshape(-1, K)
    xt = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(xt.float().numpy(), x)
    q, s = mlr.quant_mxfp4(xt.cuda())
    torch.cuda.synchronize()
    rq, rs = O.mxfp4_quant(x, 32)
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), pack_nibbles(rq))


@pytest.mark.parametrize("layout", ["rows", "blocked"])
def test_mx_weights(layout):
    say("mx weights", layout)
    w = synth.get("deepseek_r1_mxfp4").replace(D=1024, I=256, E=3)
    w13, _ = synth.gen_masters(w, "cuda")
    q, s = mlr.quant_weight_mxfp4(w13, layout)
    torch.cuda.synchronize()
    codes = mlr.unblock_weights(q) if layout == "blocked" else q
    for e in range(w13.shape[0]):
        rq, rs = O.mxfp4_quant(synth.bf16_to_f32_np(w13[e]), 32)
        assert np.array_equal(codes[e].cpu().numpy(), pack_nibbles(rq)), e
        assert np.array_equal(s[e].cpu().numpy(), rs), e


@pytest.mark.parametrize("name,block_m", [("qwen3_235b_prefill_mxfp4_r", 0), ("qwen3_235b_prefill_mxfp4_r", 32),
                                          ("qwen3_235b_prefill_mxfp4_r", 64), ("deepseek_r1_mxfp4_r", 0),
                                          ("deepseek_r1_mxfp4_r", 32), ("deepseek_r1_mxfp4_r", 128),
                                          ("qwen3_235b_prefill_mxfp4_r", 192), ("deepseek_r1_mxfp4_r", 192),
                                          ("deepseek_r1_mxfp4_small", 0), ("deepseek_r1_mxfp4_small", 16),
                                          ("qwen3_235b_decode_mxfp4_r", 16), ("qwen3_235b_decode_mxfp4_r", 0), ("qwen3_235b_prefill_mxfp4_r", 16),
                                          ("deepseek_r1_mxfp4_r", 16)])
def test_forward_mxfp4(name, block_m):
    w = REDUCED[name]
    say("mxfp4 forward", name, block_m)
    c = build_case(w)
    y = c.layer.forward(c.x, c.logits, block_m=block_m)
    torch.cuda.synchronize()
    inter = c.layer.intermediates(w.T, block_m)
    B = inter["block_m"]
    assert B in (16, 32, 64, 128, 192)
    ref = O.moe_forward(c.spec, c.bank, c.x_np(), c.logits_np(), block_m=B)
    assert np.array_equal(inter["topk_ids"].cpu().numpy(), ref["ids"])
    for key in ("counts", "offsets", "sorted_ids", "block_expert", "inv_perm"):
        assert np.array_equal(inter[key].cpu().numpy(), ref["perm"][key]), key
    assert np.array_equal(inter["xq"].cpu().numpy(), pack_nibbles(ref["xq"]))
    assert np.array_equal(inter["xs"].cpu().numpy(), ref["sx"])
    total = int(ref["perm"]["offsets"][-1])
    real = ref["perm"]["sorted_ids"][:total] != w.T * (w.k + w.n_shared)
    act = inter["act"][:total].float().cpu().numpy()[real]
    assert rel_l2(act, ref["act"][:total][real]) < 2e-3
    q, s = quant_act_ref("mxfp4", act)
    aq = inter["aq"][:total].cpu().numpy()[real]
    as_ = inter["as"][:total].cpu().numpy()[real]
    assert np.array_equal(aq, q) and np.array_equal(as_, s)
    # out_perm of the routed rows against the oracle's down GEMM on the GPU's act codes
    a_in = dequant_act("mxfp4", aq, as_)
    rows = np.nonzero(real)[0]
    out = inter["out_perm"][:total].float().cpu().numpy()[real]
    ref_out = np.zeros_like(out)
    be = inter["block_expert"].cpu().numpy()
    for e in np.unique(be[rows // B]):
        m = be[rows // B] == e
        ref_out[m] = O.expert_down(a_in[m], c.bank.dequantized(int(e))[1], True)
    assert rel_l2(out, ref_out) < 2e-3
    err = rel_l2(y.float().cpu().numpy(), ref["y"])
    say("y rel_l2", err)
    assert err <= tol_of(w.quant)


@pytest.mark.parametrize("name,block_m", [("deepseek_r1_mxfp4_small", 16), ("deepseek_r1_mxfp4_small", 32),
                                          ("qwen3_235b_decode_mxfp4_r", 16)])
def test_mxfp4_step_entries(name, block_m):
    """The gate/up and down step entries on MXFP4 codes from the library's
    row quantizer (the row-major act codes the public down entry takes; the
    fused forward hands the streaming down GEMM blocked ones): act against
    the oracle's act, the act codes the oracle's quantization of it, out_perm
    against the oracle's down GEMM fed those codes, pad rows written 0."""
    w = REDUCED[name]
    say("mxfp4 step entries", name, block_m)
    c = build_case(w)
    ids, _ = (mlr.route_topk(c.logits, w.k) if w.scoring == "softmax" else
              mlr.route_topk(c.logits, w.k, w.scoring, w.n_groups, w.topk_groups, None, True, w.route_scale))
    perm = mlr.permute_align(ids, w.E, w.n_shared, block_m)
    xq, xs = mlr.quant_mxfp4(c.x)
    act = c.layer.gateup_silu(xq, xs, w.T, block_m, perm)
    torch.cuda.synchronize()
    ref = O.moe_forward(c.spec, c.bank, c.x_np(), c.logits_np(), block_m=block_m)
    total = int(perm["offsets"][-1].item())
    real = perm["sorted_ids"][:total].cpu().numpy() != w.T * (w.k + w.n_shared)
    got = act[:total].float().cpu().numpy()
    assert rel_l2(got[real], ref["act"][:total][real]) < 2e-3
    assert np.all(got[zero_pad_rows(perm, block_m)] == 0)

    aq, sc = mlr.quant_mxfp4(act)
    out = c.layer.down(aq, sc, w.T, block_m, perm)
    torch.cuda.synchronize()
    aq_np, sc_np, out_np = aq.cpu().numpy(), sc.cpu().numpy(), out.float().cpu().numpy()
    q, s = quant_act_ref("mxfp4", got[real])
    assert np.array_equal(aq_np[:total][real], q) and np.array_equal(sc_np[:total][real], s)
    offs, cnts = perm["offsets"].cpu().numpy(), perm["counts"].cpu().numpy()
    pairs = []
    for e in range(w.E + w.n_shared):
        lo, hi = int(offs[e]), int(offs[e]) + int(cnts[e])
        if hi > lo:
            a_in = dequant_act("mxfp4", aq_np[lo:hi], sc_np[lo:hi])
            pairs.append((out_np[lo:hi], O.expert_down(a_in, c.bank.dequantized(e)[1], True)))
    assert rel_l2(np.concatenate([g for g, _ in pairs]), np.concatenate([r for _, r in pairs])) < 2e-3
    zp = zero_pad_rows(perm, block_m)
    assert np.all(out_np[:len(zp)][zp] == 0)


def test_mxfp4_rejects_256_row_tiles():
    w = REDUCED["deepseek_r1_mxfp4_small"]
    c = build_case(w)
    with pytest.raises(mlr.MoEError):
        c.layer.forward(c.x, c.logits, block_m=256)
