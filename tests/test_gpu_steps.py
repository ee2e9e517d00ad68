"""GPU parity of each C-ABI entry point against the oracle, on the same
seeded inputs: bit-exact for routing ids, permutation and FP8 codes; within
a stated tolerance for floating-point outputs."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_cases import zero_pad_rows, REDUCED, build_case, rel_l2, say

pytestmark = pytest.mark.gpu

mlr = pytest.importorskip("moe_layer_router_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mlr.lib()


def _ulp_diff_f32(a, b):
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ai - bi)


# ------------------------------------------------------------------ routing

@pytest.mark.parametrize("name", ["qwen3_30b_a3b_ptpc", "qwen3_235b_prefill_ptpc", "qwen3_235b_decode_ptpc"])
def test_route_softmax_full_size(name):
    w = synth.get(name)
    say("route_softmax", name)
    logits = synth.gen_logits(w, "cuda")
    ids, wt = mlr.route_topk(logits, w.k)
    torch.cuda.synchronize()
    rid, rw = O.route_softmax_topk(logits.cpu().numpy(), w.k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    d = _ulp_diff_f32(wt.cpu().numpy(), rw)
    assert d.max() <= 1 and (d > 0).mean() < 1e-3


def test_route_softmax_not_renormalized_and_k_equals_e():
    say("route_softmax variants")
    logits = synth.gen_normal_f32((300, 16), 2.0, 99, "cuda")
    for k, renorm in [(16, True), (8, False), (1, True)]:
        ids, wt = mlr.route_topk(logits, k, renormalize=renorm)
        torch.cuda.synchronize()
        rid, rw = O.route_softmax_topk(logits.cpu().numpy(), k, renorm)
        assert np.array_equal(ids.cpu().numpy(), rid)
        assert _ulp_diff_f32(wt.cpu().numpy(), rw).max() <= 1


def test_route_ties_and_signed_zero():
    say("route ties")
    g = torch.Generator().manual_seed(5)
    logits = torch.randint(-2, 3, (1000, 128), generator=g).to(torch.float32)
    logits[0] = 0.0
    logits[0, 1::2] = -0.0
    logits[1] = 1.0
    lg = logits.cuda()
    ids, _ = mlr.route_topk(lg, 8)
    rid, _ = O.route_softmax_topk(logits.numpy(), 8)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert list(ids[0].cpu().numpy()) == list(range(8)) == list(ids[1].cpu().numpy())
    ids, w = mlr.route_topk(lg, 8, "sigmoid_grouped", 8, 4, None, True, 2.5)
    rid, rw = O.route_sigmoid_grouped(logits.numpy(), 8, 8, 4, None, 2.5)
    assert np.array_equal(ids.cpu().numpy(), rid)


@pytest.mark.parametrize("bias", [False, True])
def test_route_sigmoid_grouped_full_size(bias):
    w = synth.get("deepseek_r1_block_fp8")
    say("route_sigmoid_grouped", bias)
    logits = synth.gen_logits(w, "cuda")
    sb = synth.gen_normal_f32((w.E,), 0.05, 1234, "cuda") if bias else None
    ids, wt = mlr.route_topk(logits, w.k, "sigmoid_grouped", w.n_groups, w.topk_groups, sb, True, w.route_scale)
    torch.cuda.synchronize()
    rid, rw = O.route_sigmoid_grouped(logits.cpu().numpy(), w.k, w.n_groups, w.topk_groups,
                                      None if sb is None else sb.cpu().numpy(), w.route_scale)
    assert np.array_equal(ids.cpu().numpy(), rid)
    d = _ulp_diff_f32(wt.cpu().numpy(), rw)
    assert d.max() <= 1 and (d > 0).mean() < 1e-3


def test_router_logits():
    w = synth.get("tiny_bf16")
    say("router_logits")
    x = synth.gen_x(w, "cuda")
    wr = synth.gen_router_w(w, "cuda")
    lg = mlr.router_logits(x, wr)
    torch.cuda.synchronize()
    ref = O.router_logits(synth.bf16_to_f32_np(x), wr.cpu().numpy())
    assert _ulp_diff_f32(lg.cpu().numpy(), ref).max() <= 1
    # a larger projection exercises the D split
    x2 = synth.gen_normal_f32((50, 4096), 1.0, 3, "cuda").to(torch.bfloat16)
    wr2 = synth.gen_normal_f32((128, 4096), 0.02, 4, "cuda")
    lg2 = mlr.router_logits(x2, wr2)
    ref2 = O.router_logits(synth.bf16_to_f32_np(x2), wr2.cpu().numpy())
    assert _ulp_diff_f32(lg2.cpu().numpy(), ref2).max() <= 1


# ------------------------------------------------------------------ permutation

def _rand_ids(T, k, E, seed, skew=False):
    g = torch.Generator().manual_seed(seed)
    if skew:
        p = 1.0 / torch.arange(1, E + 1, dtype=torch.float64) ** 1.2
        rows = [torch.multinomial(p, k, replacement=False, generator=g) for _ in range(T)]
    else:
        rows = [torch.randperm(E, generator=g)[:k] for _ in range(T)]
    return torch.stack(rows).to(torch.int32) if T else torch.zeros((0, k), dtype=torch.int32)


@pytest.mark.parametrize("T,k,E,ns,B,skew", [
    (64, 2, 8, 0, 32, False), (256, 8, 128, 0, 32, False), (8192, 8, 128, 0, 128, True),
    (32, 8, 128, 0, 32, True), (4096, 8, 256, 1, 64, False), (1, 8, 256, 1, 64, False),
    (333, 10, 512, 1, 64, True), (3000, 4, 16, 0, 128, False), (700, 3, 1000, 1, 32, True)])
def test_permute_align(T, k, E, ns, B, skew):
    say("permute", T, k, E, ns, B)
    ids = _rand_ids(T, k, E, T * 7 + k, skew)
    p = mlr.permute_align(ids.cuda(), E, ns, B)
    torch.cuda.synchronize()
    r = O.permute_align(ids.numpy(), E, ns, B)
    for key in ("counts", "offsets", "sorted_ids", "block_expert", "inv_perm"):
        assert np.array_equal(p[key].cpu().numpy(), r[key]), key


def test_permute_degenerate_routing():
    say("permute degenerate")
    T, k, E = 2000, 1, 64
    ids = torch.full((T, k), 17, dtype=torch.int32)
    p = mlr.permute_align(ids.cuda(), E, 0, 64)
    r = O.permute_align(ids.numpy(), E, 0, 64)
    for key in ("counts", "offsets", "sorted_ids", "block_expert", "inv_perm"):
        assert np.array_equal(p[key].cpu().numpy(), r[key]), key
    # ids outside [0, E) get no row and inv_perm -1, as in the oracle
    for ns in (0, 1):
        ids = _rand_ids(50, 4, 16, 3)
        ids[5, 1] = 16
        ids[7, 0] = -3
        ids[49, 3] = 1000
        p = mlr.permute_align(ids.cuda(), 16, ns, 32)
        r = O.permute_align(ids.numpy(), 16, ns, 32)
        for key in ("counts", "offsets", "sorted_ids", "block_expert", "inv_perm"):
            assert np.array_equal(p[key].cpu().numpy(), r[key]), (ns, key)
        inv = p["inv_perm"].cpu().numpy()
        assert inv[5 * 4 + 1] == -1 and inv[7 * 4] == -1 and inv[49 * 4 + 3] == -1
        assert int(p["counts"].sum()) == 50 * (4 + ns) - 3


# ------------------------------------------------------------------ quantization

def _quant_inputs(M, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g) * torch.exp(torch.randn((M, 1), generator=g) * 3)
    x[0] = 0.0
    x[1] = -0.0
    x[2, :] = 0.0
    x[2, 5] = -1e-30
    # values whose scaled image sits on e4m3 rounding midpoints
    codes = torch.arange(0, 126, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
    mids = (codes[:-1] + codes[1:]) / 2
    row = torch.cat([mids, -mids, torch.tensor([448.0])])
    x[3, :row.numel()] = row[:K]
    x[4] = torch.linspace(-3, 3, K)
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("M,K,group", [(300, 2048, 0), (77, 4096, 0), (64, 7168, 0), (40, 7168, 128),
                                       (513, 1536, 0), (129, 2048, 128), (33, 256, 0), (10, 16384, 0)])
def test_quant_rows(M, K, group):
    say("quant", M, K, group)
    x = _quant_inputs(M, K, M + K)
    q, s = mlr.quant_ptpc_fp8(x.cuda(), group)
    torch.cuda.synchronize()
    rq, rs = O.quant_rows(x.to(torch.float32).numpy(), group)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("amax", [448.0, 300.0])
def test_quant_every_bf16_value(amax):
    """Every finite bf16 value of magnitude at most amax goes through the
    encoder in rows whose first element is amax, so the scale is amax/448 and
    each value is multiplied by fp32(448/amax): 1 (the bf16 values themselves)
    or a factor that is not a power of two (fp32 inputs with all mantissa bits
    in use).  Codes and scales bit-exact against the oracle's encoder."""
    say("quant every bf16", amax)
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= amax)]
    K = 4096
    n = -(-vals.size // (K - 1))
    rows = np.zeros((n, K), np.float32)
    rows[:, 0] = amax
    flat = rows[:, 1:].reshape(-1)
    flat[:vals.size] = vals
    rows[:, 1:] = flat.reshape(n, K - 1)
    x = torch.from_numpy(rows).to(torch.bfloat16)
    assert np.array_equal(x.to(torch.float32).numpy(), rows)       # exact: every value is bf16
    q, sc = mlr.quant_ptpc_fp8(x.cuda(), 0)
    torch.cuda.synchronize()
    rq, rs = O.quant_rows(rows, 0)
    assert np.all(rs == np.float32(amax) / np.float32(448.0))
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), rq)


def test_quant_valid_rows_leaves_the_rest():
    say("quant valid_rows")
    x = _quant_inputs(100, 512, 1).cuda()
    q = torch.full((100, 512), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((100,), -5.0, device="cuda")
    nv = torch.tensor([37], dtype=torch.int32, device="cuda")
    mlr._lib.check("q", mlr.lib().moe_quant_ptpc_fp8(x.data_ptr(), 100, 512, 0, nv.data_ptr(), q.data_ptr(),
                                                     s.data_ptr(), torch.cuda.current_stream().cuda_stream))
    rq, rs = O.quant_rows(x[:37].float().cpu().numpy())
    assert np.array_equal(q[:37].cpu().numpy(), rq)
    assert np.all(q[37:].cpu().numpy() == 0xAB) and np.all(s[37:].cpu().numpy() == -5.0)


@pytest.mark.parametrize("quant,layout", [("ptpc_fp8", "rows"), ("block128_fp8", "rows"),
                                          ("ptpc_fp8", "blocked"), ("block128_fp8", "blocked")])
def test_quant_weights(quant, layout):
    """Codes and scales bit-exact against the oracle; blocked codes are the
    row-major ones moved as whole 16-row x 128-byte blocks."""
    say("quant weights", quant, layout)
    w = synth.get("deepseek_r1_block_fp8").replace(D=1024, I=256, E=3)
    w13, _ = synth.gen_masters(w, "cuda")
    w13[1, :128, :128] *= 1000.0
    w13[2, 128:256, 256:384] = 0.0
    q, s = mlr.quant_weight_fp8(w13, quant, layout)
    torch.cuda.synchronize()
    if layout == "blocked":
        raw = q.cpu().numpy().reshape(-1)
        n, N, K = w13.shape
        # the documented byte order: block (g, kb) of matrix e starts at byte
        # 2048 j, j = (e*N/16 + g) * K/128 + kb; inside it code (r, c) sits at
        # (r//2 + 8*(c//64))*128 + ((r%2)*4 + (c%64)//16)*16 + c%16
        e_, r_, k_ = np.meshgrid(np.arange(n), np.arange(N), np.arange(K), indexing="ij")
        r16, c = r_ % 16, k_ % 128
        pos = (((e_ * (N // 16) + r_ // 16) * (K // 128) + k_ // 128) * 2048
               + (r16 // 2 + 8 * (c // 64)) * 128 + ((r16 % 2) * 4 + (c % 64) // 16) * 16 + c % 16)
        rowmajor = torch.from_numpy(raw[pos])
        assert torch.equal(mlr.unblock_weights(q).cpu(), rowmajor)
        q = rowmajor
    for e in range(3):
        m = synth.bf16_to_f32_np(w13[e])
        rq, rs = O.quant_rows(m) if quant == "ptpc_fp8" else O.quant_weight_blocks(m)
        assert np.array_equal(q[e].cpu().numpy(), rq)
        assert np.array_equal(s[e].cpu().numpy().view(np.uint32), rs.view(np.uint32))


# ------------------------------------------------------------------ expert GEMMs and combine

@pytest.mark.parametrize("name,block_m", [("tiny_bf16", 32), ("bf16_multi_tile_r", 64), ("qwen3_30b_a3b_ptpc", 32),
                                          ("qwen3_235b_prefill_ptpc_r", 128), ("qwen3_235b_prefill_ptpc_r", 64),
                                          ("qwen3_235b_prefill_ptpc_r", 256), ("bf16_multi_tile_r", 256),
                                          ("qwen3_30b_a3b_ptpc_i384", 64), ("qwen3_30b_a3b_ptpc_i384", 256),
                                          ("deepseek_r1_block_fp8_r", 32), ("deepseek_r1_block_fp8_r", 64),
                                          ("deepseek_r1_block_fp8_r", 128), ("deepseek_r1_block_fp8_r", 256),
                                          ("deepseek_r1_block_fp8_r", 192),
                                          ("tiny_bf16", 16), ("bf16_small_t20", 16), ("qwen3_235b_decode_ptpc", 16),
                                          ("qwen3_30b_a3b_ptpc", 16), ("qwen3_235b_prefill_ptpc_r", 16),
                                          ("deepseek_r1_block_fp8_r", 16), ("bf16_multi_tile_r", 16),
                                          ("qwen3_235b_decode_ptpc_t64", 16), ("deepseek_r1_block_fp8_small", 16)])
def test_gateup_silu_entry(name, block_m):
    """act rows of the gate/up GEMM vs the oracle's, from the same x, routing
    and weights (routing and x codes are bit-exact upstream)."""
    w = REDUCED[name]
    say("gateup", name, block_m)
    c = build_case(w)
    x = c.x
    if w.router == "gemm":
        logits = mlr.router_logits(x, c.router_w)
    else:
        logits = c.logits
    ids, wt = (mlr.route_topk(logits, w.k) if w.scoring == "softmax" else
               mlr.route_topk(logits, w.k, w.scoring, w.n_groups, w.topk_groups, None, True, w.route_scale))
    perm = mlr.permute_align(ids, w.E, w.n_shared, block_m)
    group = 128 if w.quant == "block128_fp8" else 0
    if w.quant == "bf16":
        a, sa = x, None
    else:
        a, sa = mlr.quant_ptpc_fp8(x, group)
    act = c.layer.gateup_silu(a, sa, w.T, block_m, perm)
    torch.cuda.synchronize()
    rw = None if c.router_w is None else c.router_w.cpu().numpy()
    ref = O.moe_forward(c.spec, c.bank, c.x_np(), c.logits_np(), router_w=rw, block_m=block_m)
    total = int(perm["offsets"][-1].item())
    got = act[:total].float().cpu().numpy()
    want = ref["act"][:total]
    real = perm["sorted_ids"][:total].cpu().numpy() != w.T * (w.k + w.n_shared)
    assert rel_l2(got[real], want[real]) < 2e-3
    # pad rows inside tiles with routed rows are zero (pad-only tiles are not written)
    assert np.all(got[zero_pad_rows(perm, block_m)] == 0)


@pytest.mark.parametrize("name,block_m", [("tiny_bf16", 32), ("qwen3_235b_prefill_ptpc_r", 128),
                                          ("qwen3_235b_prefill_ptpc_r", 256), ("bf16_multi_tile_r", 256),
                                          ("qwen3_30b_a3b_ptpc_i384", 128), ("qwen3_30b_a3b_ptpc_i384", 256),
                                          ("qwen3_30b_a3b_ptpc", 64), ("deepseek_r1_block_fp8_r", 32),
                                          ("deepseek_r1_block_fp8_r", 64), ("deepseek_r1_block_fp8_r", 128),
                                          ("deepseek_r1_block_fp8_r", 256), ("deepseek_r1_block_fp8_r", 192),
                                          ("tiny_bf16", 16), ("qwen3_235b_decode_ptpc", 16),
                                          ("qwen3_235b_decode_ptpc_t64", 16), ("deepseek_r1_block_fp8_small", 16),
                                          ("qwen3_30b_a3b_ptpc", 16), ("qwen3_235b_prefill_ptpc_r", 16)])
def test_down_entry(name, block_m):
    """out_perm of the down GEMM on a synthetic act buffer (same values on both
    sides), quantized per row / 1x128 by each side."""
    w = REDUCED[name]
    say("down", name, block_m)
    c = build_case(w)
    ids = torch.stack([torch.randperm(w.E, generator=torch.Generator().manual_seed(t))[:w.k]
                       for t in range(w.T)]).to(torch.int32)
    perm = mlr.permute_align(ids.cuda(), w.E, w.n_shared, block_m)
    R = perm["max_rows"]
    act = synth.gen_normal_f32((R, w.I), 0.5, 77, "cuda").to(torch.bfloat16)
    group = 128 if w.quant == "block128_fp8" else 0
    if w.quant == "bf16":
        a, sa = act, None
    else:
        a, sa = mlr.quant_ptpc_fp8(act, group)
    out = c.layer.down(a, sa, w.T, block_m, perm)
    torch.cuda.synchronize()
    act_np = synth.bf16_to_f32_np(act)
    offs = perm["offsets"].cpu().numpy()
    cnts = perm["counts"].cpu().numpy()
    got = out.float().cpu().numpy()
    # pad rows inside tiles with routed rows come out 0 (their act here is
    # not); pad-only tiles are not written
    zp = zero_pad_rows(perm, block_m)
    assert np.all(got[:len(zp)][zp] == 0)
    errs = []
    for e in range(w.E + w.n_shared):
        lo, hi = int(offs[e]), int(offs[e]) + int(cnts[e])
        if hi == lo:
            continue
        _, w2 = c.bank.dequantized(e)
        if w.quant == "bf16":
            ain = act_np[lo:hi].astype(np.float64)
        else:
            q, s = O.quant_rows(act_np[lo:hi], group)
            ain = O.dequant_rows(q, s, group)
        want = O.expert_down(ain, w2, w.quant != "bf16")
        errs.append((got[lo:hi], want))
    g = np.concatenate([a for a, _ in errs])
    r = np.concatenate([b for _, b in errs])
    assert rel_l2(g, r) < (1e-5 if w.quant == "bf16" else 2e-3)


@pytest.mark.parametrize("name,block_m", [("qwen3_235b_prefill_ptpc_r", 256), ("qwen3_235b_prefill_ptpc_r", 128),
                                          ("deepseek_r1_block_fp8_r", 256), ("bf16_multi_tile_r", 256),
                                          ("deepseek_r1_block_fp8_r", 192),
                                          ("qwen3_30b_a3b_ptpc", 64), ("qwen3_30b_a3b_ptpc", 16),
                                          ("qwen3_235b_prefill_ptpc_r", 16)])
def test_gemm_counts_skip_pad_tiles(name, block_m):
    """With expert_counts the LDS-tiled GEMMs skip the 32-row tiles that hold
    only pads (no operand reads, MFMAs or stores); the routed rows must come
    out bitwise equal to the run without counts, pad rows 0 without counts
    and wherever a tile also holds routed rows with them."""
    w = REDUCED[name]
    say("counts", name, block_m)
    c = build_case(w)
    logits = mlr.router_logits(c.x, c.router_w) if w.router == "gemm" else c.logits
    ids, _ = (mlr.route_topk(logits, w.k) if w.scoring == "softmax" else
              mlr.route_topk(logits, w.k, w.scoring, w.n_groups, w.topk_groups, None, True, w.route_scale))
    perm = mlr.permute_align(ids, w.E, w.n_shared, block_m)
    group = 128 if w.quant == "block128_fp8" else 0
    a, sa = (c.x, None) if w.quant == "bf16" else mlr.quant_ptpc_fp8(c.x, group)
    act1 = c.layer.gateup_silu(a, sa, w.T, block_m, perm, use_counts=True)
    act0 = c.layer.gateup_silu(a, sa, w.T, block_m, perm, use_counts=False)
    torch.cuda.synchronize()
    total = int(perm["offsets"][-1].item())
    counts = perm["counts"].cpu().numpy()
    assert np.sum((-(-counts // block_m)) * block_m - counts) > 0, "the case must have pad rows"
    real = perm["sorted_ids"][:total] != w.T * (w.k + w.n_shared)
    # routed rows bitwise; written pad rows are zeros (of either sign)
    zp1 = torch.from_numpy(zero_pad_rows(perm, block_m)).cuda()
    zp0 = torch.from_numpy(zero_pad_rows(perm, block_m, use_counts=False)).cuda()
    assert torch.equal(act1[:total][real].view(torch.int16), act0[:total][real].view(torch.int16))
    assert bool((act1[:total][zp1] == 0).all()) and bool((act0[:total][zp0] == 0).all())
    # the down GEMM on act0 (every pad row 0, so the run without counts,
    # which cannot tell pads from rows, writes 0 there too)
    b, sb = (act0, None) if w.quant == "bf16" else mlr.quant_ptpc_fp8(act0, group)
    o1 = c.layer.down(b, sb, w.T, block_m, perm, use_counts=True)
    o0 = c.layer.down(b, sb, w.T, block_m, perm, use_counts=False)
    torch.cuda.synchronize()
    assert torch.equal(o1[:total][real], o0[:total][real])
    assert bool((o1[:total][zp1] == 0).all()) and bool((o0[:total][zp0] == 0).all())


@pytest.mark.parametrize("T,k,ns,D,dt", [(64, 2, 0, 256, 0), (300, 8, 1, 1024, 1), (17, 8, 0, 7168, 1),
                                         (129, 10, 1, 512, 1), (70, 11, 1, 2048, 1), (40, 12, 1, 512, 1),
                                         (33, 10, 1, 256, 0)])
def test_combine_entry(T, k, ns, D, dt):
    say("combine", T, k, ns, D, dt)
    E = 16
    ids = torch.stack([torch.randperm(E, generator=torch.Generator().manual_seed(t))[:k]
                       for t in range(T)]).to(torch.int32)
    perm = mlr.permute_align(ids.cuda(), E, ns, 32)
    R = perm["max_rows"]
    op = synth.gen_normal_f32((R, D), 1.0, 5, "cuda")
    if dt == 1:
        op = op.to(torch.bfloat16)
    wt = torch.rand((T, k), generator=torch.Generator().manual_seed(9)).cuda()
    y = mlr.unpermute_combine(op, perm["inv_perm"], wt, T, k, ns)
    torch.cuda.synchronize()
    opn = op.float().cpu().numpy()
    inv = perm["inv_perm"].cpu().numpy().astype(np.int64)
    o_rows = opn[inv[:T * k]].reshape(T, k, D)
    o_sh = opn[inv[T * k:]] if ns else None
    ref = O.combine(o_rows, wt.cpu().numpy(), o_sh)
    got = y.float().cpu().numpy()
    # fp32 vs fp64 accumulation: the fp32 sum is within (k+1) * 2^-24 of the
    # summed term magnitudes; after that one bf16 step of the larger result
    mag = np.abs(wt.cpu().numpy())[:, :, None] * np.abs(o_rows)
    S = mag.sum(axis=1) + (np.abs(o_sh) if ns else 0.0)
    diff = np.abs(got - ref)
    bound = np.maximum(np.abs(got), np.abs(ref)) * 2.0 ** -7 + (k + 2) * 2.0 ** -24 * S + 1e-30
    assert np.all(diff <= bound)
    assert (diff > 0).mean() < 0.01
