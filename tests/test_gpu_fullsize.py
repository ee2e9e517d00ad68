"""Full-size GPU parity of moe_forward, element by element, in the launch
configuration the bench times (block_m chosen by the library).

For each workload at its full size the oracle runs the whole layer once,
expert by expert on a thread pool (the host side of the GPU machine), and:
  - routing ids, counts, offsets, sorted ids, block map, inverse map and x
    codes / scales are compared whole and bit-exact;
  - every routed row of act is compared with the oracle's act (per-row
    relative L2 and over the expert);
  - FP8 modes: every routed row's act codes and scales are the oracle's
    quantization of the GPU's own act, bit for bit;
  - every routed row of out_perm is compared with the oracle's down GEMM fed
    the GPU's own act codes (or bf16 act), so a down-GEMM fault is not hidden
    behind act rounding;
  - y is compared for every token: relative L2 over the tensor within
    2e-3 (bf16 path) or 1e-2 (FP8 paths); per token against the oracle's
    down GEMM and combine fed the GPU's own act codes (the same bounds), and
    per token against the oracle end to end (reported; bound below).
Per-row bound of act and out_perm: 2^-7.  Both sides round the same fp32 /
fp64 value to bf16 and differ only where the GPU's fp32 accumulation moves a
value across a rounding boundary; an element that does so moves by one bf16
step, at most 2^-7 of its value, so a row stays within 2^-7 of the oracle's
even if every element moved (elements that differ more are tiny values whose
fp32 sum cancelled).  Over all rows the same bounds as y apply.
End to end per token the quantized modes are held to TOKEN_TOL_FP8 (5e-2:
one act row's scale moving by a bf16 step re-rounds about 1/23 of its codes;
the derivation is beside the constant), the bf16 path to 2e-3 (no
re-quantization there).
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_cases import (TOKEN_TOL_FP8, build_case, check_router_logits, dequant_act, pack_nibbles, quant_act_ref,
                              same_scales, say, tol_of)

pytestmark = pytest.mark.gpu

mlr = pytest.importorskip("moe_layer_router_amd")

ROW_TOL = 2.0 ** -7


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mlr.lib()


def _host_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _np(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    return synth.bf16_to_f32_np(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _row_rel(a: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Relative L2 of each row (rows with a zero reference: absolute)."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref, axis=1)
    return np.linalg.norm(a - ref, axis=1) / np.where(den > 0, den, 1.0)


@pytest.mark.parametrize("name", ["tiny_bf16", "qwen3_30b_a3b_ptpc", "qwen3_235b_prefill_ptpc",
                                  "qwen3_235b_decode_ptpc", "deepseek_r1_block_fp8", "e512_top10_shared_ptpc",
                                  "qwen3_235b_prefill_mxfp4"])
def test_full_size_every_row(name):
    w = synth.get(name)
    say("full size", name)
    c = build_case(w, cache_experts=False)
    y = c.layer.forward(c.x, c.logits)          # block_m 0: the library's choice, as the bench runs it
    torch.cuda.synchronize()
    inter = c.layer.intermediates(w.T, 0)
    B = inter["block_m"]
    fp8 = w.quant != "bf16"
    say("block_m", B, "max_rows", inter["max_rows"])

    act_g = _np(inter["act"])
    out_g = _np(inter["out_perm"])
    aq_g = inter["aq"].cpu().numpy() if fp8 else None
    as_g = inter["as"].cpu().numpy() if fp8 else None
    y_g = _np(y)
    x_np = c.x_np()
    rw = None if c.router_w is None else c.router_w.cpu().numpy()

    stats = {}
    o_fed = np.zeros(out_g.shape, np.float32)     # oracle down GEMM on the GPU's act codes

    def check(e, lo, hi, w13, w2, rows):
        """This expert's routed rows against the oracle (runs in a worker)."""
        a = act_g[lo:hi]
        r_act = _row_rel(a, rows["act"])
        codes_ok = True
        if fp8:
            q, sc = quant_act_ref(w.quant, a)
            codes_ok = bool(np.array_equal(aq_g[lo:hi], q) and same_scales(as_g[lo:hi], sc))
            a_in = dequant_act(w.quant, aq_g[lo:hi], as_g[lo:hi])
        else:
            a_in = a.astype(np.float64)
        o_ref = O.expert_down(a_in, w2, fp8)
        o_fed[lo:hi] = o_ref
        r_out = _row_rel(out_g[lo:hi], o_ref)
        stats[e] = dict(rows=hi - lo, act_max=float(r_act.max()), out_max=float(r_out.max()),
                        act_ss=(float(np.sum((a.astype(np.float64) - rows["act"]) ** 2)),
                                float(np.sum(rows["act"].astype(np.float64) ** 2))),
                        codes_ok=codes_ok)

    lg = c.logits_np()
    if w.router == "gemm":
        # routing is bit-exact given the same fp32 logits: the oracle routes
        # the GPU's logits once they are within the projection's bound
        lg = inter["logits"].cpu().numpy()
        check_router_logits(lg, x_np, rw)
    with ThreadPoolExecutor(_host_threads()) as ex:
        ref = O.moe_forward(c.spec, c.bank, x_np, lg, block_m=B, pmap=ex.map, on_expert=check)

    # routing, permutation and x codes: whole and bit-exact
    assert np.array_equal(inter["topk_ids"].cpu().numpy(), ref["ids"])
    for key in ("counts", "offsets", "sorted_ids", "block_expert", "inv_perm"):
        assert np.array_equal(inter[key].cpu().numpy(), ref["perm"][key]), key
    if fp8:
        xq_ref = pack_nibbles(ref["xq"]) if w.quant == "mxfp4" else ref["xq"]
        assert np.array_equal(inter["xq"].cpu().numpy(), xq_ref)
        assert same_scales(inter["xs"].cpu().numpy(), ref["sx"])

    # every routed row of every expert
    counts = ref["perm"]["counts"]
    assert sorted(stats) == [e for e in range(w.E_total) if counts[e] > 0]
    bad_codes = [e for e, s in stats.items() if not s["codes_ok"]]
    assert not bad_codes, f"act codes differ from the quantized GPU act for experts {bad_codes[:8]}"
    act_max = max(s["act_max"] for s in stats.values())
    out_max = max(s["out_max"] for s in stats.values())
    num = sum(s["act_ss"][0] for s in stats.values())
    den = sum(s["act_ss"][1] for s in stats.values())
    hot = max(stats, key=lambda e: stats[e]["rows"])
    cold = min(stats, key=lambda e: stats[e]["rows"])
    say(f"rows {int(counts.sum())} experts {len(stats)} (hottest {hot}: {stats[hot]['rows']} rows, "
        f"coldest {cold}: {stats[cold]['rows']}); act rel_l2 {np.sqrt(num / den):.2e} "
        f"row max {act_max:.2e}; out_perm row max {out_max:.2e}")
    assert np.sqrt(num / den) <= tol_of(w.quant)
    assert act_max <= ROW_TOL, [(e, s["act_max"]) for e, s in stats.items() if s["act_max"] > ROW_TOL][:8]
    assert out_max <= ROW_TOL, [(e, s["out_max"]) for e, s in stats.items() if s["out_max"] > ROW_TOL][:8]

    # y: every token
    k, T = w.k, w.T
    inv = ref["perm"]["inv_perm"].astype(np.int64)
    y_fed = O.combine(o_fed[inv[:T * k]].reshape(T, k, w.D), ref["w"], o_fed[inv[T * k:]] if w.n_shared else None)
    per_fed = _row_rel(y_g, y_fed)
    err = O.relative_l2(y_g, ref["y"])
    per_tok = _row_rel(y_g, ref["y"])
    worst = int(np.argmax(per_tok))
    say(f"y rel_l2 {err:.2e}; per token vs the oracle fed the GPU's act codes: max {per_fed.max():.2e}; "
        f"end to end: max {per_tok[worst]:.2e} (token {worst}), median {np.median(per_tok):.2e}")
    if per_tok[worst] > tol_of(w.quant):
        rows_w = [int(r) for r in inv[worst * k:(worst + 1) * k]] + ([int(inv[T * k + worst])] if w.n_shared else [])
        say("rows of the worst token and their act error:",
            [(r, float(_row_rel(act_g[r:r + 1], ref["act"][r:r + 1])[0])) for r in rows_w])
    assert err <= tol_of(w.quant)
    assert per_fed.max() <= tol_of(w.quant)
    assert per_tok.max() <= (TOKEN_TOL_FP8 if fp8 else tol_of(w.quant))

    # the layer's quantized weights of the hottest expert are the oracle's codes
    if fp8:
        q13, s13, q2, s2 = c.bank.quantized(hot)
        if w.quant == "mxfp4":
            q13, q2 = pack_nibbles(q13), pack_nibbles(q2)
        assert c.layer.weight_layout == "blocked"
        assert np.array_equal(mlr.unblock_weights(c.layer.weights.w13[hot]).cpu().numpy(), q13)
        assert np.array_equal(mlr.unblock_weights(c.layer.weights.w2[hot]).cpu().numpy(), q2)
        assert same_scales(c.layer.weights.w13_scale[hot].cpu().numpy(), s13)
        assert same_scales(c.layer.weights.w2_scale[hot].cpu().numpy(), s2)
