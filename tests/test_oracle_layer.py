"""Pins of the whole-layer oracle: a dense SwiGLU MLP (one expert, top-1),
a per-token pure-Python evaluation on tiny inputs, identical-expert and
token-order invariances, and agreement of the full and per-token paths."""

import numpy as np
import pytest
import torch

import oracle as O


def _bank(spec, seed, same=False):
    rng = np.random.default_rng(seed)
    n = spec.E + spec.n_shared
    w13 = [O.bf16_round((rng.standard_normal((2 * spec.I, spec.D)) / np.sqrt(spec.D)).astype(np.float32))
           for _ in range(n)]
    w2 = [O.bf16_round((rng.standard_normal((spec.D, spec.I)) / np.sqrt(spec.I)).astype(np.float32))
          for _ in range(n)]
    if same:
        w13 = [w13[0]] * n
        w2 = [w2[0]] * n
    return O.ExpertBank(spec, lambda e: (w13[e], w2[e])), w13, w2


def _x(T, D, seed):
    return O.bf16_round(np.random.default_rng(seed).standard_normal((T, D)).astype(np.float32))


def _torch_dense_swiglu(x, w13, w2, I, fp8):
    """Dense MLP in torch (CPU, float64), quantizing with torch's float8 cast
    when fp8 is set: y = down(silu(gate(x)) * up(x))."""
    def q(m):                                   # per-row fp8 through torch's encoder
        amax = m.abs().amax(dim=1).to(torch.float32)
        inv = torch.where(amax == 0, torch.ones_like(amax), torch.full_like(amax, 448.0) / amax)
        sc = torch.where(amax == 0, torch.ones_like(amax), amax / torch.full_like(amax, 448.0))
        codes = (m.to(torch.float32) * inv[:, None]).to(torch.float8_e4m3fn)
        return codes.to(torch.float64) * sc.to(torch.float64)[:, None]
    xt = torch.from_numpy(x).to(torch.float64)
    W13 = torch.from_numpy(w13).to(torch.float64)
    W2 = torch.from_numpy(w2).to(torch.float64)
    if fp8:
        xt, W13, W2 = q(xt), q(W13), q(W2)
    g = xt @ W13[:I].T
    u = xt @ W13[I:].T
    act = (torch.nn.functional.silu(g) * u).to(torch.float32).to(torch.bfloat16).to(torch.float64)
    if fp8:
        act = q(act)
    o = (act @ W2.T).to(torch.float32)
    if fp8:
        o = o.to(torch.bfloat16).to(torch.float32)
    return o.to(torch.bfloat16).to(torch.float32).numpy()


@pytest.mark.parametrize("quant", ["bf16", "ptpc_fp8"])
def test_one_expert_top1_is_dense_swiglu(quant):
    spec = O.LayerSpec(D=64, I=48, E=1, top_k=1, quant=quant)
    bank, w13, w2 = _bank(spec, 1)
    x = _x(37, 64, 2)
    logits = np.zeros((37, 1), np.float32)
    out = O.moe_forward(spec, bank, x, logits, block_m=8)
    ref = _torch_dense_swiglu(x, w13[0], w2[0], 48, quant != "bf16")
    # both sides round act and y to bf16; their float64 sums may differ in the
    # last fp64 bits, which can flip a rare rounding: allow 1 bf16 step there
    d = np.abs(out["y"] - ref)
    step = np.abs(ref) * 2.0 ** -7 + 1e-30
    assert np.all(d <= step * 1.01)
    assert np.mean(d > 0) < 0.01
    assert O.relative_l2(out["y"], ref) < 1e-3


def test_one_expert_block_fp8_is_dense_mlp_with_block_quant():
    spec = O.LayerSpec(D=256, I=128, E=1, top_k=1, quant="block128_fp8")
    bank, w13, w2 = _bank(spec, 3)
    x = _x(20, 256, 4)
    out = O.moe_forward(spec, bank, x, np.zeros((20, 1), np.float32), block_m=4)
    # same MLP written with independent torch block quantization
    def qrow(m, g):
        m = m.reshape(m.shape[0], -1, g)
        amax = m.abs().amax(dim=2).to(torch.float32)
        inv = torch.where(amax == 0, torch.ones_like(amax), torch.full_like(amax, 448.0) / amax)
        sc = torch.where(amax == 0, torch.ones_like(amax), amax / torch.full_like(amax, 448.0))
        c = (m.to(torch.float32) * inv[..., None]).to(torch.float8_e4m3fn).to(torch.float64)
        return (c * sc.to(torch.float64)[..., None]).reshape(m.shape[0], -1)
    def qblk(w):
        N, K = w.shape
        t = w.reshape(N // 128, 128, K // 128, 128).permute(0, 2, 1, 3).reshape(-1, 128 * 128)
        d = qrow(t, 128 * 128)
        return d.reshape(N // 128, K // 128, 128, 128).permute(0, 2, 1, 3).reshape(N, K)
    xt = qrow(torch.from_numpy(x), 128)
    W13 = qblk(torch.from_numpy(w13[0]))
    W2 = qblk(torch.from_numpy(w2[0]))
    h = xt @ W13.T
    act = (torch.nn.functional.silu(h[:, :128]) * h[:, 128:]).to(torch.float32).to(torch.bfloat16).to(torch.float64)
    o = (qrow(act, 128) @ W2.T).to(torch.float32).to(torch.bfloat16)
    ref = o.to(torch.float32).numpy()
    assert O.relative_l2(out["y"], ref) < 1e-3


def _py_layer(spec, x, logits, w13, w2, sel_bias=None):
    """Per-token evaluation with Python loops over d and i (tiny shapes),
    straight from the layer's definition, no permutation involved."""
    T = x.shape[0]
    ids, w = (O.route_softmax_topk(logits, spec.top_k) if spec.scoring == "softmax" else
              O.route_sigmoid_grouped(logits, spec.top_k, spec.n_groups, spec.topk_groups,
                                      sel_bias, spec.route_scale))
    y = np.zeros((T, spec.D), np.float32)
    for t in range(T):
        acc = [0.0] * spec.D
        experts = [(int(e), float(wt)) for e, wt in zip(ids[t], w[t])]
        if spec.n_shared:
            experts.append((spec.E, 1.0))
        for e, wt in experts:
            act = []
            for i in range(spec.I):
                g = sum(float(x[t, d]) * float(w13[e][i, d]) for d in range(spec.D))
                u = sum(float(x[t, d]) * float(w13[e][spec.I + i, d]) for d in range(spec.D))
                act.append(float(O.bf16_round(np.float32(g / (1.0 + np.exp(-g)) * u))))
            for d in range(spec.D):
                o = float(np.float32(sum(act[i] * float(w2[e][d, i]) for i in range(spec.I))))
                acc[d] += wt * o
        y[t] = O.bf16_round(np.array(acc, np.float32))
    return y


def test_tiny_layer_vs_python_loops_softmax():
    spec = O.LayerSpec(D=12, I=6, E=5, top_k=2)
    bank, w13, w2 = _bank(spec, 5)
    x = _x(9, 12, 6)
    logits = np.random.default_rng(7).standard_normal((9, 5)).astype(np.float32)
    out = O.moe_forward(spec, bank, x, logits, block_m=4)
    ref = _py_layer(spec, x, logits, w13, w2)
    assert O.relative_l2(out["y"], ref) < 1e-6


def test_tiny_layer_vs_python_loops_grouped_shared():
    spec = O.LayerSpec(D=10, I=4, E=8, top_k=3, n_shared=1, scoring="sigmoid_grouped",
                       n_groups=4, topk_groups=2, route_scale=2.5)
    bank, w13, w2 = _bank(spec, 8)
    x = _x(11, 10, 9)
    logits = np.random.default_rng(10).standard_normal((11, 8)).astype(np.float32)
    bias = np.random.default_rng(11).standard_normal(8).astype(np.float32) * 0.1
    out = O.moe_forward(spec, bank, x, logits, sel_bias=bias, block_m=2)
    ref = _py_layer(spec, x, logits, w13, w2, bias)
    assert O.relative_l2(out["y"], ref) < 1e-6


@pytest.mark.parametrize("quant", ["bf16", "ptpc_fp8"])
def test_identical_experts_give_dense_mlp(quant):
    spec = O.LayerSpec(D=128, I=64, E=8, top_k=3, quant=quant)
    bank, w13, w2 = _bank(spec, 12, same=True)
    x = _x(30, 128, 13)
    logits = np.random.default_rng(14).standard_normal((30, 8)).astype(np.float32)
    out = O.moe_forward(spec, bank, x, logits, block_m=4)
    one = O.LayerSpec(D=128, I=64, E=1, top_k=1, quant=quant)
    dense = O.moe_forward(one, O.ExpertBank(one, lambda e: (w13[0], w2[0])), x,
                          np.zeros((30, 1), np.float32), block_m=4)
    # sum_j w_j = 1, so y = bf16(o) up to the fp32 weight sum and a rounding
    assert O.relative_l2(out["y"], dense["y"]) < 3e-3


def test_token_order_permutation_is_bitwise():
    spec = O.LayerSpec(D=64, I=32, E=16, top_k=4, n_shared=1, scoring="sigmoid_grouped",
                       n_groups=4, topk_groups=2, route_scale=2.5, quant="ptpc_fp8")
    bank, _, _ = _bank(spec, 15)
    x = _x(40, 64, 16)
    logits = np.random.default_rng(17).standard_normal((40, 16)).astype(np.float32)
    perm = np.random.default_rng(18).permutation(40)
    a = O.moe_forward(spec, bank, x, logits, block_m=8)
    b = O.moe_forward(spec, bank, x[perm], logits[perm], block_m=8)
    assert np.array_equal(a["y"][perm].view(np.uint32), b["y"].view(np.uint32))


@pytest.mark.parametrize("quant,block_m", [("bf16", 4), ("ptpc_fp8", 16), ("block128_fp8", 8)])
def test_full_path_equals_per_token_path(quant, block_m):
    spec = O.LayerSpec(D=256, I=128, E=6, top_k=2, n_shared=1 if quant == "block128_fp8" else 0,
                       quant=quant)
    bank, _, _ = _bank(spec, 19)
    x = _x(25, 256, 20)
    x[3] = 0.0
    logits = np.random.default_rng(21).standard_normal((25, 6)).astype(np.float32)
    a = O.moe_forward(spec, bank, x, logits, block_m=block_m)
    b = O.moe_forward_tokens(spec, bank, x, logits)
    assert np.array_equal(a["y"].view(np.uint32), b["y"].view(np.uint32))
    assert np.array_equal(a["ids"], b["ids"])


def test_block_m_does_not_change_y():
    spec = O.LayerSpec(D=128, I=64, E=8, top_k=2, quant="ptpc_fp8")
    bank, _, _ = _bank(spec, 22)
    x = _x(33, 128, 23)
    logits = np.random.default_rng(24).standard_normal((33, 8)).astype(np.float32)
    ys = [O.moe_forward(spec, bank, x, logits, block_m=b)["y"] for b in (1, 16, 64)]
    assert all(np.array_equal(ys[0], y) for y in ys[1:])


def test_empty_batch():
    spec = O.LayerSpec(D=128, I=64, E=8, top_k=2, quant="ptpc_fp8")
    bank, _, _ = _bank(spec, 25)
    out = O.moe_forward(spec, bank, np.zeros((0, 128), np.float32), np.zeros((0, 8), np.float32))
    assert out["y"].shape == (0, 128)


# ------------------------------------------------------------ FP8 storage points

def _bf16_t(v: float) -> float:
    """bf16 rounding through torch's own cast (independent of the oracle's codec)."""
    return float(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).to(torch.float32)[0])


def _fp8_dequant_groups(vals, group):
    """Dequantized values of a list of fp32 values, quantized in consecutive
    groups of ``group`` elements: scale = fp32(amax / 448), codes through
    torch's float8_e4m3fn cast of fp32(v * fp32(448 / amax)); value = code * scale."""
    out = []
    for g0 in range(0, len(vals), group):
        grp = [np.float32(v) for v in vals[g0:g0 + group]]
        amax = max(abs(v) for v in grp)
        if amax == 0:
            scale, inv = 1.0, np.float32(1.0)
        else:
            scale, inv = float(np.float32(amax) / np.float32(448.0)), np.float32(448.0) / np.float32(amax)
        t = torch.tensor([float(v * inv) for v in grp], dtype=torch.float32)
        out += [c * scale for c in t.to(torch.float8_e4m3fn).to(torch.float64).tolist()]
    return out


def _fp8_weight(w, block):
    """Dequantized weight [N][K] as nested lists: one scale per output row
    (block None) or per block x block tile."""
    N, K = w.shape
    if block is None:
        return [_fp8_dequant_groups(w[n].tolist(), K) for n in range(N)]
    deq = [[0.0] * K for _ in range(N)]
    for n0 in range(0, N, block):
        for k0 in range(0, K, block):
            tile = [float(w[n, k]) for n in range(n0, n0 + block) for k in range(k0, k0 + block)]
            d = _fp8_dequant_groups(tile, block * block)
            for i, n in enumerate(range(n0, n0 + block)):
                deq[n][k0:k0 + block] = d[i * block:(i + 1) * block]
    return deq


def _py_layer_fp8(spec, x, logits, w13, w2, sel_bias=None):
    """The FP8 layer token by token with Python loops, rounding at every
    storage point the layer declares: x codes (per row, or per 1x128 group),
    fp64 dot products, act = bf16(fp32(silu(g) * u)), act re-quantized (per
    row, or per 1x128 group), expert output o = bf16(fp32(act . W2)), then
    y = bf16(fp32(sum_j w_j o_j + o_shared)) with the sum in order j = 0..k-1
    and the shared expert last.  Rounding goes through torch's casts."""
    blk = 128 if spec.quant == "block128_fp8" else None
    T = x.shape[0]
    ids, w = (O.route_softmax_topk(logits, spec.top_k) if spec.scoring == "softmax" else
              O.route_sigmoid_grouped(logits, spec.top_k, spec.n_groups, spec.topk_groups,
                                      sel_bias, spec.route_scale))
    W13 = {e: _fp8_weight(w13[e], blk) for e in range(spec.E + spec.n_shared)}
    W2 = {e: _fp8_weight(w2[e], blk) for e in range(spec.E + spec.n_shared)}
    y = np.zeros((T, spec.D), np.float32)
    for t in range(T):
        a = _fp8_dequant_groups(x[t].tolist(), blk or spec.D)
        experts = [(int(e), float(wt)) for e, wt in zip(ids[t], w[t])]
        if spec.n_shared:
            experts.append((spec.E, 1.0))
        acc = [0.0] * spec.D
        for e, wt in experts:
            act = []
            for i in range(spec.I):
                g = sum(a[d] * W13[e][i][d] for d in range(spec.D))
                u = sum(a[d] * W13[e][spec.I + i][d] for d in range(spec.D))
                act.append(_bf16_t(float(np.float32(g / (1.0 + np.exp(-g)) * u))))
            aq = _fp8_dequant_groups(act, blk or spec.I)
            for d in range(spec.D):
                o = _bf16_t(float(np.float32(sum(aq[i] * W2[e][d][i] for i in range(spec.I)))))
                acc[d] += wt * o
        y[t] = [_bf16_t(float(np.float32(v))) for v in acc]
    return y


def test_tiny_ptpc_layer_top3_shared_vs_python_loops():
    """PTPC-FP8, k = 3 plus a shared expert: every storage point (x codes, bf16
    act, act codes, bf16 expert outputs, combine order) against the loops."""
    spec = O.LayerSpec(D=16, I=8, E=6, top_k=3, n_shared=1, quant="ptpc_fp8")
    bank, w13, w2 = _bank(spec, 31)
    x = _x(7, 16, 32)
    x[2] = 0.0                                    # amax 0 -> scale 1
    logits = np.random.default_rng(33).standard_normal((7, 6)).astype(np.float32)
    out = O.moe_forward(spec, bank, x, logits, block_m=4)
    ref = _py_layer_fp8(spec, x, logits, w13, w2)
    assert O.relative_l2(out["y"], ref) <= 1e-6
    assert np.all(out["y"][2] == 0)


def test_tiny_block_fp8_layer_grouped_shared_vs_python_loops():
    """Blockwise FP8 (1x128 activations, 128x128 weights), grouped-sigmoid
    top-2 of 4 groups, x 2.5, plus a shared expert, against the loops."""
    spec = O.LayerSpec(D=256, I=128, E=4, top_k=2, n_shared=1, scoring="sigmoid_grouped",
                       n_groups=2, topk_groups=1, route_scale=2.5, quant="block128_fp8")
    bank, w13, w2 = _bank(spec, 34)
    x = _x(3, 256, 35)
    x[1, 128:] = 0.0                              # one all-zero 1x128 group
    logits = np.random.default_rng(36).standard_normal((3, 4)).astype(np.float32)
    out = O.moe_forward(spec, bank, x, logits, block_m=2)
    ref = _py_layer_fp8(spec, x, logits, w13, w2)
    assert O.relative_l2(out["y"], ref) <= 1e-6


# ------------------------------------------------------------ the error metric

def test_relative_l2_closed_forms():
    """relative_l2(a, ref) = ||a - ref||_2 / ||ref||_2 (||a||_2 when ref is all
    zero), on vectors whose norms are known exactly."""
    ref = np.array([3.0, 4.0])                                   # ||ref|| = 5
    assert O.relative_l2(ref, ref) == 0.0
    assert O.relative_l2(np.array([3.0, 4.0 + 5e-3]), ref) == pytest.approx(1e-3, rel=1e-12)
    assert O.relative_l2(np.array([0.0, 0.0]), ref) == pytest.approx(1.0, rel=1e-15)
    assert O.relative_l2(-ref, ref) == pytest.approx(2.0, rel=1e-15)
    # 2-D arrays: the norm over every element (Frobenius), not per row
    a2 = np.array([[1.0, 2.0], [2.0, 0.0]])                      # ||.|| = 3
    r2 = np.array([[1.0, 2.0], [2.0, 4.0]])                      # ||.|| = 5, difference 4
    assert O.relative_l2(a2, r2) == pytest.approx(0.8, rel=1e-15)
    # zero reference: the absolute norm of a
    assert O.relative_l2(np.array([1.0, 2.0, 2.0]), np.zeros(3)) == pytest.approx(3.0, rel=1e-15)
    # a NaN anywhere makes the result NaN, so no `err <= tol` gate can pass it
    assert np.isnan(O.relative_l2(np.array([3.0, np.nan]), ref))
    assert not (O.relative_l2(np.array([3.0, np.nan]), ref) <= 1e-2)


def test_expert_map_and_hook_do_not_change_the_forward():
    """moe_forward over a thread pool (pmap) equals the plain loop bitwise, and
    the per-expert hook sees exactly that expert's rows."""
    from concurrent.futures import ThreadPoolExecutor
    spec = O.LayerSpec(D=256, I=128, E=6, top_k=2, n_shared=1, quant="block128_fp8")
    bank, _, _ = _bank(spec, 41)
    x = _x(30, 256, 42)
    logits = np.random.default_rng(43).standard_normal((30, 6)).astype(np.float32)
    a = O.moe_forward(spec, bank, x, logits, block_m=8)
    seen = {}

    def hook(e, lo, hi, w13, w2, rows):
        seen[e] = (lo, hi, rows["act"].copy(), rows["aq"].copy(), rows["out"].copy(), w2.shape)

    with ThreadPoolExecutor(4) as ex:
        b = O.moe_forward(spec, bank, x, logits, block_m=8, pmap=ex.map, on_expert=hook)
    for key in ("y", "act", "out_perm"):
        assert np.array_equal(a[key].view(np.uint32), b[key].view(np.uint32)), key
    assert np.array_equal(a["aq"], b["aq"])
    counts, offs = a["perm"]["counts"], a["perm"]["offsets"]
    assert sorted(seen) == [e for e in range(7) if counts[e] > 0]
    for e, (lo, hi, act, aq, out, w2s) in seen.items():
        assert (lo, hi) == (offs[e], offs[e] + counts[e]) and w2s == (256, 128)
        assert np.array_equal(act, a["act"][lo:hi]) and np.array_equal(aq, a["aq"][lo:hi])
        assert np.array_equal(out.view(np.uint32), a["out_perm"][lo:hi].view(np.uint32))


# ------------------------------------------------------------ MXFP4 layers

_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _mx_dequant_py(vals):
    """MXFP4 round trip of a list of values in blocks of 32 (OCP MX v1.0),
    written out per element: shared scale X = 2^(floor(log2 amax) - 2), each
    element the nearest E2M1 magnitude of |v| / X (ties to the even mantissa
    bit, above 6 saturating), sign kept; returns the values code * X."""
    import math
    out = []
    for b0 in range(0, len(vals), 32):
        blk = [float(v) for v in vals[b0:b0 + 32]]
        amax = max(abs(v) for v in blk)
        if amax == 0.0:
            out += [0.0] * len(blk)
            continue
        _, ex = math.frexp(amax)                 # amax = m 2^ex, m in [0.5, 1)
        X = 2.0 ** max(-127, min(127, ex - 1 - 2))
        for v in blk:
            a = abs(v) / X
            best = min(range(8), key=lambda i: (abs(a - _E2M1_MAG[i]), i % 2))
            out.append(math.copysign(_E2M1_MAG[best] * X, v))
    return out


def _py_layer_mx(spec, x, logits, w13, w2):
    """The MXFP4 layer token by token with Python loops: x, the weight rows
    and each act row in MXFP4 (blocks of 32 along the reduction dimension),
    fp64 dot products, act = bf16(fp32(silu(g) u)), expert outputs stored
    bf16, combine j = 0..k-1 then the shared expert, one bf16 rounding."""
    T = x.shape[0]
    ids, w = O.route_softmax_topk(logits, spec.top_k)
    W13 = {e: [_mx_dequant_py(w13[e][n].tolist()) for n in range(2 * spec.I)] for e in range(spec.E + spec.n_shared)}
    W2 = {e: [_mx_dequant_py(w2[e][d].tolist()) for d in range(spec.D)] for e in range(spec.E + spec.n_shared)}
    y = np.zeros((T, spec.D), np.float32)
    for t in range(T):
        a = _mx_dequant_py(x[t].tolist())
        experts = [(int(e), float(wt)) for e, wt in zip(ids[t], w[t])]
        if spec.n_shared:
            experts.append((spec.E, 1.0))
        acc = [0.0] * spec.D
        for e, wt in experts:
            act = []
            for i in range(spec.I):
                g = sum(a[d] * W13[e][i][d] for d in range(spec.D))
                u = sum(a[d] * W13[e][spec.I + i][d] for d in range(spec.D))
                act.append(_bf16_t(float(np.float32(g / (1.0 + np.exp(-g)) * u))))
            aq = _mx_dequant_py(act)
            for d in range(spec.D):
                acc[d] += wt * _bf16_t(float(np.float32(sum(aq[i] * W2[e][d][i] for i in range(spec.I)))))
        y[t] = [_bf16_t(float(np.float32(v))) for v in acc]
    return y


def test_mx_quantizer_matches_the_elementwise_definition():
    rng = np.random.default_rng(51)
    x = (rng.standard_normal((6, 96)) * np.exp(rng.standard_normal((6, 1)) * 4)).astype(np.float32)
    x[1] = 0.0
    x[2, :32] = 6.0 * 2.0 ** -3                   # an exact block maximum
    x[3, :32] = np.linspace(-1, 1, 32)
    codes, sc = O.mxfp4_quant(x, 32)
    got = O.mxfp4_dequant(codes, sc, 32)
    ref = np.array([_mx_dequant_py(r.tolist()) for r in x])
    assert np.array_equal(got, ref)


def test_tiny_mxfp4_layer_top2_shared_vs_python_loops():
    spec = O.LayerSpec(D=64, I=32, E=5, top_k=2, n_shared=1, quant="mxfp4")
    bank, w13, w2 = _bank(spec, 52)
    x = _x(6, 64, 53)
    x[4] = 0.0
    logits = np.random.default_rng(54).standard_normal((6, 5)).astype(np.float32)
    out = O.moe_forward(spec, bank, x, logits, block_m=4)
    ref = _py_layer_mx(spec, x, logits, w13, w2)
    assert O.relative_l2(out["y"], ref) <= 1e-6
    assert np.all(out["y"][4] == 0)
    # the intermediates are codes in 0..15 and E8M0 scale bytes
    assert out["xq"].max() <= 15 and out["sx"].shape == (6, 2) and out["aq"].max() <= 15


def test_mxfp4_identical_experts_give_dense_mlp():
    spec = O.LayerSpec(D=128, I=64, E=8, top_k=3, quant="mxfp4")
    bank, w13, w2 = _bank(spec, 55, same=True)
    x = _x(20, 128, 56)
    logits = np.random.default_rng(57).standard_normal((20, 8)).astype(np.float32)
    out = O.moe_forward(spec, bank, x, logits, block_m=4)
    one = O.LayerSpec(D=128, I=64, E=1, top_k=1, quant="mxfp4")
    dense = O.moe_forward(one, O.ExpertBank(one, lambda e: (w13[0], w2[0])), x,
                          np.zeros((20, 1), np.float32), block_m=4)
    assert O.relative_l2(out["y"], dense["y"]) < 3e-3
