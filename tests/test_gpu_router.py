"""GPU parity of the router projection fused with top-k and x quantization
(moe_router_front, and moe_forward without logits above the small-batch
sizes): logits within the fp32-accumulation bound of the oracle's float64
projection; ids and weights bit for bit (weights within one fp32 ulp) as the
oracle routes the GPU's logits (the routing contract is bit-exact given the
same fp32 logits); x codes and scales bit-exact.

Logit bound: every product x[d] * piece is exact (x is bf16 and each fp32
router weight is split exactly into three bf16 pieces), so the GPU differs
from the float64 sum only by fp32 accumulation: |error| <= n u sum_d
|x[d] w[d]| for n additions (u = 2^-24), which the test caps at
1e-6 sum_d |x[d] w[d]| plus half an ulp of the stored fp32 value."""

import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_cases import REDUCED, build_case, check_router_logits, rel_l2, say, tol_of

pytestmark = pytest.mark.gpu

mlr = pytest.importorskip("moe_layer_router_amd")
from moe_layer_router_amd import _lib as L  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mlr.lib()


def _check_logits(lg_gpu, x_np, wr_np):
    ref = check_router_logits(lg_gpu, x_np, wr_np)
    cond = np.abs(x_np.astype(np.float64)) @ np.abs(wr_np.astype(np.float64)).T
    err = np.abs(lg_gpu.astype(np.float64) - ref.astype(np.float64))
    say(f"logits: max |err| / sum|x w| = {np.max(err / cond):.2e}; fraction not bit-equal: {np.mean(err > 0):.3f}")
    return ref


def _route_ref(w, lg):
    if w.scoring == "softmax":
        return O.route_softmax_topk(lg, w.k)
    return O.route_sigmoid_grouped(lg, w.k, w.n_groups, w.topk_groups, None, w.route_scale)


def _front(c, T, desc=None):
    w = c.w
    desc = c.layer.desc if desc is None else desc
    fp8 = w.quant != "bf16"
    blk = w.quant == "block128_fp8"
    dev = c.x.device
    lg = torch.empty((T, w.E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, w.k), dtype=torch.int32, device=dev)
    wt = torch.empty((T, w.k), dtype=torch.float32, device=dev)
    xq = torch.empty((T, w.D), dtype=torch.uint8, device=dev) if fp8 else None
    xs = torch.empty((T, w.D // 128) if blk else (T,), dtype=torch.float32, device=dev) if fp8 else None
    nws = int(L.lib().moe_router_front_workspace_size(ctypes.byref(desc)))
    assert nws > 0
    ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
    st = L.lib().moe_router_front(ctypes.byref(desc), c.x.data_ptr(), T, lg.data_ptr(), ids.data_ptr(),
                                  wt.data_ptr(), None if xq is None else xq.data_ptr(),
                                  None if xs is None else xs.data_ptr(), ws.data_ptr(), nws,
                                  torch.cuda.current_stream().cuda_stream)
    L.check("moe_router_front", st)
    torch.cuda.synchronize()
    return lg, ids, wt, xq, xs


ROUTED = {
    # E = 128 (one 32-expert tile per wave), softmax, PTPC x codes
    "prefill_e128": synth.get("qwen3_235b_prefill_router").replace(T=1000, D=1024, I=512),
    # E = 256 grouped sigmoid with blockwise x codes (two tiles per wave)
    "r1_e256": synth.get("deepseek_r1_block_fp8").replace(T=333, D=1024, I=256, router="gemm"),
    # E = 512, top-10 (four tiles per wave); ragged token tail
    "e512": synth.get("e512_top10_shared_ptpc").replace(T=517, D=512, I=256, router="gemm"),
    # E = 8 (one partial tile), bf16 layer: no x codes
    "tiny": synth.get("tiny_bf16").replace(T=70),
    # E = 60, not a multiple of 32
    "e60": synth.get("qwen3_30b_a3b_ptpc").replace(T=129, D=256, I=128, E=60, k=6, router="gemm"),
}


@pytest.mark.parametrize("name", sorted(ROUTED))
def test_router_front(name):
    w = ROUTED[name]
    say("router front", name)
    c = build_case(w)
    lg, ids, wt, xq, xs = _front(c, w.T)
    x_np = c.x_np()
    wr = c.router_w.cpu().numpy()
    _check_logits(lg.cpu().numpy(), x_np, wr)
    lg_np = lg.cpu().numpy()
    rid, rw = _route_ref(w, lg_np)
    assert np.array_equal(ids.cpu().numpy(), rid)
    d = np.abs(wt.cpu().numpy().view(np.int32).astype(np.int64) - rw.view(np.int32).astype(np.int64))
    assert d.max() <= 1
    if w.quant != "bf16":
        q, s = O.quant_rows(x_np, 128 if w.quant == "block128_fp8" else 0)
        assert np.array_equal(xq.cpu().numpy(), q)
        assert np.array_equal(xs.cpu().numpy().view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("name,renorm,bias", [("prefill_e128", False, False), ("e512", False, False),
                                               ("r1_e256", False, True), ("r1_e256", True, True)])
def test_router_front_routing_options(name, renorm, bias):
    """The other branches of the four-tokens-per-wave routing: soft-max weights
    over all experts (not renormalized over the picks) and a selection bias in
    grouped scoring.  ids bit-exact, weights within one fp32 ulp of the oracle
    routing the GPU's logits."""
    w = ROUTED[name]
    say("router front options", name, renorm, bias)
    c = build_case(w)
    desc = L.LayerDesc.from_buffer_copy(c.layer.desc)
    desc.renormalize = int(renorm)
    b = synth.gen_normal_f32((w.E,), 0.05, 11, "cuda") if bias else None
    if b is not None:
        desc.sel_bias = b.data_ptr()
    lg, ids, wt, _, _ = _front(c, w.T, desc)
    lg_np = lg.cpu().numpy()
    if w.scoring == "softmax":
        rid, rw = O.route_softmax_topk(lg_np, w.k, renormalize=renorm)
    else:
        rid, rw = O.route_sigmoid_grouped(lg_np, w.k, w.n_groups, w.topk_groups,
                                          None if b is None else b.cpu().numpy(), w.route_scale, renormalize=renorm)
    assert np.array_equal(ids.cpu().numpy(), rid)
    d = np.abs(wt.cpu().numpy().view(np.int32).astype(np.int64) - rw.view(np.int32).astype(np.int64))
    assert d.max() <= 1


def test_router_front_full_size():
    """The Qwen3-235B-shaped prefill batch (T = 8192, D = 4096, E = 128)."""
    w = synth.get("qwen3_235b_prefill_router")
    say("router front full size")
    c = build_case(w, cache_experts=False)
    lg, ids, wt, xq, xs = _front(c, w.T)
    x_np = c.x_np()
    _check_logits(lg.cpu().numpy(), x_np, c.router_w.cpu().numpy())
    rid, rw = _route_ref(w, lg.cpu().numpy())
    assert np.array_equal(ids.cpu().numpy(), rid)
    d = np.abs(wt.cpu().numpy().view(np.int32).astype(np.int64) - rw.view(np.int32).astype(np.int64))
    assert d.max() <= 1
    q, s = O.quant_rows(x_np, 0)
    assert np.array_equal(xq.cpu().numpy(), q)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("name,block_m", [("prefill_e128", 0), ("r1_e256", 0), ("e512", 128), ("tiny", 32)])
def test_forward_without_logits(name, block_m):
    """moe_forward given no logits routes through the fused kernel (T above
    the small-batch sizes): its logits, routing and x codes are those of
    moe_router_front, and y matches the oracle run on the GPU's logits."""
    w = ROUTED[name]
    say("forward without logits", name, block_m)
    c = build_case(w)
    y = c.layer.forward(c.x, None, block_m=block_m)
    torch.cuda.synchronize()
    inter = c.layer.intermediates(w.T, block_m)
    lg, ids, wt, xq, _ = _front(c, w.T)
    assert torch.equal(inter["logits"].view(torch.int32), lg.view(torch.int32))
    assert torch.equal(inter["topk_ids"], ids)
    assert torch.equal(inter["topk_w"].view(torch.int32), wt.view(torch.int32))
    if xq is not None:
        assert torch.equal(inter["xq"], xq)
    ref = O.moe_forward(c.spec, c.bank, c.x_np(), lg.cpu().numpy(), block_m=inter["block_m"])
    assert np.array_equal(inter["sorted_ids"].cpu().numpy(), ref["perm"]["sorted_ids"])
    err = rel_l2(y.float().cpu().numpy(), ref["y"])
    say("y rel_l2", err)
    assert err <= tol_of(w.quant)


def test_router_front_validation():
    w = ROUTED["prefill_e128"]
    c = build_case(w.replace(T=4))
    d = L.LayerDesc.from_buffer_copy(c.layer.desc)
    d.router_w = None
    assert L.lib().moe_router_front(ctypes.byref(d), 1, 4, 1, 1, 1, 1, 1, 256, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    d = L.LayerDesc.from_buffer_copy(c.layer.desc)
    assert L.lib().moe_router_front(ctypes.byref(d), 1, 4, 1, 1, 1, None, None, 256, 1 << 30, None) \
        == L.MOE_ERR_INVALID_ARG
    need = int(L.lib().moe_router_front_workspace_size(ctypes.byref(d)))
    assert need == (w.E + 31) // 32 * (w.D // 64) * 12 * 1024
    assert L.lib().moe_router_front(ctypes.byref(d), 1, 4, 1, 1, 1, 1, 1, 256, need - 1, None) == L.MOE_ERR_WORKSPACE
    assert L.lib().moe_router_front(ctypes.byref(d), None, 0, None, None, None, None, None, None, 0, None) == L.MOE_OK
