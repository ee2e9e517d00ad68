"""Benchmark of the fused MoE layer forward on one MI355X.

One step = one pass of the whole routed-expert path over one batch of
synthetic input, resident in HBM: top-k routing -> permutation -> x
quantization -> gate/up grouped GEMM with SwiGLU -> act quantization -> down
grouped GEMM -> weighted combine (plus the router projection when the
workload has one).  The timed loop calls the fused moe_forward entry; a
second loop calls the C-ABI step entries one by one (the same kernels, with
routing and x quantization as separate launches) with HIP events around the
two grouped GEMMs, for the per-kernel figures and the roofline of the
dominant kernel, and checks that both paths give the same bits.

Prints ONE JSON line.  Default workload: the Qwen3-235B-A22B-shaped prefill
layer (T=8192, D=4096, E=128, top-8, I=1536, PTPC-FP8).  Further legs of the
same line time the decode batch (T=32; PTPC-FP8, and MXFP4 as
``decode_mxfp4``) eagerly and from captured graphs, the
other layer shapes (tiny bf16, Qwen3-30B-A3B-shaped, DeepSeek-R1-shaped with
blockwise FP8, 512 experts top-10 plus a shared expert, the Qwen3-235B and
DeepSeek-R1 shapes in MXFP4, the Qwen3-235B prefill routed by its own router
gate) and the expert-parallel payload kernels; ``cpu_baseline`` runs the CPU oracle over
the whole default batch once, on the host's cores, and its output gates the
GPU number on every token.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer TFLOP/s (prefill) and expert-weight GB/s (decode), % of roofline"
PEAK_TFLOPS = {"ptpc_fp8": 5000.0, "block128_fp8": 5000.0, "bf16": 2500.0, "mxfp4": 10100.0}
PEAK_HBM_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def measured_traffic(workload: str):
    """HBM bytes per launch of the gate/up GEMM from the committed rocprofv3
    counter record, or None when the kernel source changed since (or the
    record is for another workload)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "grouped_gemm_gateup_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.strip() and not line.startswith("#") and ":" in line:
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    src = os.path.join(ROOT, rec.get("kernel_source", ""))
    if rec.get("workload") != workload or not os.path.exists(src):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec.get("source_sha256"):
        return None
    kib = float(rec["fetch_kib"]) * float(rec["fetch_factor"]) + float(rec["write_kib"]) * float(rec["write_factor"])
    return int(kib * 1024)


class Case:
    """A workload's seeded inputs on the GPU and the layer built from them
    (FP8 weights quantized on the GPU from the bf16 masters)."""

    def __init__(self, mlr, synth, w, keep_masters=True):
        self.w = w
        self.x = synth.gen_x(w, "cuda")
        self.logits = synth.gen_logits(w, "cuda")
        self.router_w = synth.gen_router_w(w, "cuda") if w.router == "gemm" else None
        w13, w2 = synth.gen_masters(w, "cuda")
        self.layer = mlr.MoELayer.from_masters(w13, w2, w.quant, router_w=self.router_w, E=w.E, top_k=w.k,
                                               n_shared=w.n_shared, scoring=w.scoring, n_groups=w.n_groups,
                                               topk_groups=w.topk_groups, route_scale=w.route_scale)
        self.w13, self.w2 = (w13, w2) if keep_masters else (None, None)


class Steps:
    """The path through the step entries, on buffers carved from the layer's
    workspace (the same layout moe_forward uses)."""

    def __init__(self, layer, w, x, logits, block_m):
        import torch
        from moe_layer_router_amd import _lib as L
        self.L, self.lib, self.layer, self.w = L, L.lib(), layer, w
        self.x, self.logits = x, logits
        self.T = w.T
        self.lay = layer.layout(w.T, block_m)
        self.B = self.lay["block_m"]
        self.ws = layer.workspace(w.T, block_m)
        self.y = torch.empty((w.T, w.D), dtype=torch.bfloat16, device=x.device)
        base = self.ws.data_ptr()
        self.p = {k: (base + v if isinstance(v, int) and v >= 0 else None) for k, v in self.lay.items()}
        self.stream = torch.cuda.current_stream().cuda_stream

    def run(self, ev=None):
        L, lib, w, p, s = self.L, self.lib, self.w, self.p, self.stream
        d = ctypes.byref(self.layer.desc)
        fp8 = w.quant != "bf16"
        group = 128 if w.quant == "block128_fp8" else 0
        Ep = w.E + w.n_shared
        lg = self.logits.data_ptr() if self.logits is not None else p["logits"]
        if self.logits is None:
            L.check("router", lib.moe_router_logits(self.x.data_ptr(), self.layer.weights.router_w.data_ptr(),
                                                    self.T, w.D, w.E, lg, s))
        sc = 0 if w.scoring == "softmax" else 1
        L.check("route", lib.moe_route_topk(lg, self.T, w.E, w.k, sc, w.n_groups, w.topk_groups, None, 1,
                                            w.route_scale, p["topk_ids"], p["topk_w"], s))
        L.check("permute", lib.moe_permute_align(p["topk_ids"], self.T, w.k, w.E, w.n_shared, self.B, p["counts"],
                                                 p["offsets"], p["sorted_ids"], p["block_expert"], p["inv_perm"],
                                                 p["scratch"], s))
        mx = w.quant == "mxfp4"
        a, a_s = self.x.data_ptr(), None
        if mx:
            L.check("quant x", lib.moe_quant_mxfp4(self.x.data_ptr(), self.T, w.D, None, p["xq"], p["xs"], s))
            a, a_s = p["xq"], p["xs"]
        elif fp8:
            L.check("quant x", lib.moe_quant_ptpc_fp8(self.x.data_ptr(), self.T, w.D, group, None, p["xq"], p["xs"], s))
            a, a_s = p["xq"], p["xs"]
        if ev is not None:
            ev[0].record()
        L.check("gateup", lib.moe_grouped_gemm_gateup_silu(d, a, a_s, self.T, self.B, p["sorted_ids"],
                                                           p["block_expert"], p["offsets"], p["counts"], p["act"], s))
        if ev is not None:
            ev[1].record()
        act, act_s = p["act"], None
        if mx:
            L.check("quant act", lib.moe_quant_mxfp4(p["act"], self.lay["max_rows"], w.I, p["offsets"] + 4 * Ep,
                                                     p["aq"], p["as_"], s))
            act, act_s = p["aq"], p["as_"]
        elif fp8:
            L.check("quant act", lib.moe_quant_ptpc_fp8(p["act"], self.lay["max_rows"], w.I, group,
                                                        p["offsets"] + 4 * Ep, p["aq"], p["as_"], s))
            act, act_s = p["aq"], p["as_"]
        if ev is not None:
            ev[2].record()
        L.check("down", lib.moe_grouped_gemm_down(d, act, act_s, self.T, self.B, p["block_expert"], p["offsets"],
                                                  p["counts"], p["out_perm"], s))
        if ev is not None:
            ev[3].record()
        L.check("combine", lib.moe_unpermute_combine(p["out_perm"], 1 if fp8 else 0, p["inv_perm"], p["topk_w"],
                                                     self.T, w.k, w.n_shared, w.D, self.y.data_ptr(), s))


def gateup_bytes(w, ids_np):
    """Algorithmic HBM bytes of one gate/up launch: W13 codes and scales of
    the experts the batch uses, the activation rows read once, act written once."""
    import numpy as np
    used = len(np.unique(ids_np)) + w.n_shared
    if w.quant == "mxfp4":           # E2M1 codes (half a byte) + one E8M0 byte per 32
        wb = 2 * w.I * w.D // 2 + 2 * w.I * w.D // 32
        ab = w.T * w.D // 2 + w.T * w.D // 32
        return used * wb + ab + w.T * (w.k + w.n_shared) * w.I * 2
    elem = 2 if w.quant == "bf16" else 1
    wb = 2 * w.I * w.D * elem
    if w.quant == "ptpc_fp8":
        wb += 4 * 2 * w.I
    elif w.quant == "block128_fp8":
        wb += 4 * (2 * w.I // 128) * (w.D // 128)
    ab = w.T * w.D * elem + (0 if w.quant == "bf16" else 4 * w.T * (1 if w.quant == "ptpc_fp8" else w.D // 128))
    return used * wb + ab + w.T * (w.k + w.n_shared) * w.I * 2


def active_expert_bytes(w, ids_np):
    """Weight bytes of the experts the batch routes to (codes + scales)."""
    import numpy as np
    used = len(np.unique(ids_np)) + w.n_shared
    if w.quant == "mxfp4":
        return used * (3 * w.I * w.D // 2 + 3 * w.I * w.D // 32), used
    elem = 2 if w.quant == "bf16" else 1
    per = 3 * w.I * w.D * elem
    if w.quant == "ptpc_fp8":
        per += 4 * (2 * w.I + w.D)
    elif w.quant == "block128_fp8":
        per += 4 * 3 * (w.I // 128) * (w.D // 128)
    return used * per, used


def timed_calls(torch, call, steps, warmup):
    """Median, p10 and p90 (microseconds) of `steps` calls, each bracketed by
    HIP events on the current stream."""
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        call(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    pick = lambda f: t[min(len(t) - 1, int(f * len(t)))]
    return pick(0.5), pick(0.1), pick(0.9)


def sclk_during(torch, call, seconds=2.0):
    """The shader clock under the timed workload: `call` runs back to back for
    `seconds` (after the timed region, which the sampling never overlaps)
    while a host thread polls the SMU metrics of the GPU at cuda:0's PCI
    address through amdsmi.  The SMU refreshes them every 100-200 ms (its
    gfx activity accumulator advances at each refresh): each refresh counts
    once, the one current when the calls start is dropped, and so is any
    whose average gfx activity is under 50 %.  A reading is the mean of the
    XCDs' current gfx clocks.  Without amdsmi or a fresh busy reading the
    figure is None, with the reason."""
    import threading
    try:
        import amdsmi
    except Exception as e:                                  # noqa: BLE001 - reported, not fatal
        return {"mhz_median": None, "reason": f"amdsmi not importable: {e}"}
    prop = torch.cuda.get_device_properties(0)
    bdf = f"{prop.pci_domain_id:04x}:{prop.pci_bus_id:02x}:{prop.pci_device_id:02x}"
    try:
        amdsmi.amdsmi_init()
    except Exception as e:                                  # noqa: BLE001
        return {"mhz_median": None, "reason": f"amdsmi_init: {e}"}
    try:
        h = next((h for h in amdsmi.amdsmi_get_processor_handles()
                  if amdsmi.amdsmi_get_gpu_device_bdf(h).lower().startswith(bdf)), None)
        if h is None:
            return {"mhz_median": None, "reason": f"no amdsmi device at {bdf}"}
        seen, readings, errors, stop = set(), [], [], threading.Event()

        def poll():
            while not stop.is_set():
                try:
                    m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                except Exception as e:                      # noqa: BLE001
                    errors.append(str(e))
                    return
                acc, act, per = m.get("gfx_activity_acc"), m.get("average_gfx_activity"), m.get("current_gfxclks")
                if acc not in seen:
                    fresh = bool(seen)
                    seen.add(acc)
                    v = [c for c in per if isinstance(c, (int, float)) and c > 0] if isinstance(per, list) else []
                    if fresh and v and isinstance(act, (int, float)) and act >= 50:
                        readings.append(sum(v) / len(v))
                stop.wait(0.01)

        torch.cuda.synchronize()
        th = threading.Thread(target=poll, daemon=True)
        th.start()
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < seconds:
            call()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        stop.set()
        th.join()
        if not readings:
            return {"mhz_median": None, "calls": n,
                    "reason": errors[0] if errors else "no fresh metrics with the GPU busy"}
        r = sorted(readings)
        return {"mhz_median": round(r[len(r) // 2], 1), "mhz_min": round(r[0], 1), "mhz_max": round(r[-1], 1),
                "readings": len(r), "calls": n, "seconds": seconds,
                "source": "amdsmi gpu_metrics current_gfxclks (mean over XCDs), fresh SMU refreshes only"}
    finally:
        amdsmi.amdsmi_shut_down()


def weight_copies(mlr, layer):
    """The layer plus identical copies of its weights when they are under
    1 GiB (part of them could stay in the 256 MB MALL between steps): steps
    use the copies in turn, so every step reads its weights from HBM as a
    layer of a deep model would."""
    wt = layer.weights
    wbytes = sum(t.numel() * t.element_size() for t in (wt.w13, wt.w2, wt.w13_scale, wt.w2_scale) if t is not None)
    ncopy = 1 if wbytes >= (1 << 30) else int(min(4, -(-(1 << 30) // wbytes)))
    return [layer] + [
        layer.with_weights(mlr.LayerWeights(*(None if t is None else t.clone()
                                              for t in (wt.w13, wt.w2, wt.w13_scale, wt.w2_scale)),
                                            router_w=wt.router_w, sel_bias=wt.sel_bias))
        for _ in range(ncopy - 1)]


def time_decode(torch, mlr, synth, steps, warmup, name="qwen3_235b_decode_ptpc"):
    """Decode layer (T=32, Zipf-skewed routing): full forward, weights rotated
    over copies so each step streams its experts from HBM.  Timed per call
    (median, p10, p90), eagerly and replayed from a captured HIP graph of the
    forwards over every weight copy (per-forward figures; the replayed output
    must equal the eager one)."""
    w = synth.get(name)
    c = Case(mlr, synth, w, keep_masters=False)
    ncopy = 4
    layers = [c.layer]
    for _ in range(ncopy - 1):
        wt = c.layer.weights
        lw = mlr.LayerWeights(wt.w13.clone(), wt.w2.clone(), wt.w13_scale.clone(), wt.w2_scale.clone())
        layers.append(c.layer.with_weights(lw))
    y = torch.empty((w.T, w.D), dtype=torch.bfloat16, device="cuda")
    ws = layers[0].workspace(w.T)

    med, p10, p90 = timed_calls(torch, lambda i: layers[i % ncopy].forward(c.x, c.logits, y=y, workspace=ws),
                                steps, warmup)
    y_eager = y.clone()
    ids = layers[0].intermediates(w.T, 0, ws)["topk_ids"].cpu().numpy()
    nbytes, used = active_expert_bytes(w, ids)
    out = dict(workload=w.name, calls=steps, us_per_step=round(med, 2), p10_us=round(p10, 2), p90_us=round(p90, 2),
               active_experts=int(used), expert_weight_bytes=int(nbytes),
               GBps=round(nbytes / (med * 1e-6) / 1e9, 1), hbm_frac=round(nbytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4))
    # One graph holds the forwards over the ncopy weight copies in turn (as a
    # decode step of a model holds its layers): a replay launches ncopy
    # forwards, so the host's per-launch cost of a graph, larger on this
    # runtime than one forward's GPU time, is paid once per ncopy forwards.
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(ncopy):
            layers[i].forward(c.x, c.logits, y=y, workspace=ws)
    torch.cuda.synchronize()
    gsteps = max(1, steps // ncopy)
    gmed, gp10, gp90 = (v / ncopy for v in timed_calls(torch, lambda i: g.replay(), gsteps, max(1, warmup // ncopy)))
    same = bool(torch.equal(y, y_eager))
    out.update(graph_us_per_step=round(gmed, 2), graph_p10_us=round(gp10, 2), graph_p90_us=round(gp90, 2),
               graph_GBps=round(nbytes / (gmed * 1e-6) / 1e9, 1),
               graph_hbm_frac=round(nbytes / (gmed * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), graph_output_equal=same)
    if not same:
        raise SystemExit("graph replay of the decode forward differs from the eager forward")
    del g, layers, c
    torch.cuda.empty_cache()
    return out


def time_layer(torch, mlr, synth, name, steps, warmup):
    """One more layer shape: the fused forward over `steps` calls (weights
    rotated over copies when under 1 GiB), and the two grouped GEMMs through
    the step entries with HIP events around them."""
    w = synth.get(name)
    c = Case(mlr, synth, w, keep_masters=False)
    torch.cuda.empty_cache()
    layers = weight_copies(mlr, c.layer)
    ws = c.layer.workspace(w.T)
    y = torch.empty((w.T, w.D), dtype=torch.bfloat16, device="cuda")
    med, p10, p90 = timed_calls(torch, lambda i: layers[i % len(layers)].forward(c.x, c.logits, y=y, workspace=ws),
                                steps, warmup)
    inter = c.layer.intermediates(w.T, 0, ws)
    ids = inter["topk_ids"].cpu().numpy()
    st = Steps(c.layer, w, c.x, c.logits, 0)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(warmup):
        st.layer = layers[i % len(layers)]
        st.run()
    for i in range(steps):
        st.layer = layers[i % len(layers)]
        st.run(ev[i])
    torch.cuda.synchronize()
    gu_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    dn_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / steps
    rows = w.T * (w.k + w.n_shared)
    gu_f, dn_f = 2.0 * rows * 2 * w.I * w.D, 2.0 * rows * w.D * w.I
    wbytes, used = active_expert_bytes(w, ids)
    lbytes = wbytes + w.T * w.D * 4 + (0 if c.logits is None else 4 * w.T * w.E)
    ms = med * 1e-3
    peak = PEAK_TFLOPS[w.quant]
    out = dict(workload=name, T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, n_shared=w.n_shared, quant=w.quant,
               block_m=int(inter["block_m"]), calls=steps, weight_copies=len(layers),
               ms_per_step=round(ms, 4), p10_ms=round(p10 * 1e-3, 4), p90_ms=round(p90 * 1e-3, 4),
               tflops=round(w.flops() / (ms * 1e-3) / 1e12, 1), frac_mfma=round(w.flops() / (ms * 1e-3) / 1e12 / peak, 4),
               active_experts=int(used), algorithmic_bytes=int(lbytes), GBps=round(lbytes / (ms * 1e-3) / 1e9, 1),
               frac_hbm=round(lbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
               floor_ms=round(max(w.flops() / (peak * 1e12), lbytes / (PEAK_HBM_GBS * 1e9)) * 1e3, 4),
               gateup_ms=round(gu_ms, 4), down_ms=round(dn_ms, 4),
               gemms_frac_of_peak=round((gu_f + dn_f) / ((gu_ms + dn_ms) * 1e-3) / 1e12 / peak, 4),
               tokens_per_s=round(w.T / (ms * 1e-3), 1))
    out["frac_of_floor"] = round(out["floor_ms"] / ms, 4)
    if c.logits is None and w.T > 64:
        # the fused router front alone (projection, top-k, x quantization),
        # into the workspace's slots
        from moe_layer_router_amd import _lib as L
        lay = c.layer.layout(w.T, 0)
        base = ws.data_ptr()
        sp = torch.cuda.current_stream().cuda_stream

        def front(i):
            L.check("router_front", L.lib().moe_router_front(
                ctypes.byref(c.layer.desc), c.x.data_ptr(), w.T, base + lay["logits"], base + lay["topk_ids"],
                base + lay["topk_w"], base + lay["xq"], base + lay["xs"], base + lay["router"],
                ws.numel() - lay["router"], sp))
        rmed, _, _ = timed_calls(torch, front, steps, warmup)
        rflops = 3 * 2.0 * w.T * w.E * w.D          # three exact bf16 pieces of the router weight
        out["router_front"] = dict(us=round(rmed, 2), tflops=round(rflops / (rmed * 1e-6) / 1e12, 1),
                                   frac_bf16_peak=round(rflops / (rmed * 1e-6) / 1e12 / 2500.0, 4),
                                   note="router projection (3 exact bf16 pieces), top-k and x quantization "
                                        "in one launch")
    del st, layers, c, inter
    torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(case, y_gpu):
    """The CPU oracle as it stands over the whole batch, once: routing,
    permutation, x quantization, quantization of every used expert's weights
    from its bf16 masters, the expert GEMMs in float64 (experts mapped over a
    pool of host threads), act quantization and combine.  Its y gates the GPU
    number: every token must match within the parity bound."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle as O
    import synth
    w = case.w
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    spec = O.LayerSpec(D=w.D, I=w.I, E=w.E, top_k=w.k, n_shared=w.n_shared, scoring=w.scoring,
                       n_groups=w.n_groups, topk_groups=w.topk_groups, route_scale=w.route_scale, quant=w.quant)
    bank = O.ExpertBank(spec, lambda e: (synth.bf16_to_f32_np(case.w13[e]), synth.bf16_to_f32_np(case.w2[e])),
                        cache=False)
    x = synth.bf16_to_f32_np(case.x)
    lg = None if case.logits is None else case.logits.cpu().numpy()
    rw = None if case.router_w is None else case.router_w.cpu().numpy()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        ref = O.moe_forward(spec, bank, x, lg, router_w=rw, block_m=16, pmap=ex.map)
    dt = time.perf_counter() - t0
    yg = y_gpu.float().cpu().numpy().astype(np.float64)
    err = O.relative_l2(yg, ref["y"])
    den = np.linalg.norm(ref["y"].astype(np.float64), axis=1)
    per_tok = np.linalg.norm(yg - ref["y"], axis=1) / np.where(den > 0, den, 1.0)
    # over the tensor: 2e-3 (bf16 path) / 1e-2 (FP8 paths); per token (FP8
    # paths): 5e-2, the effect of one act row whose largest element crosses a
    # bf16 rounding boundary on the GPU, which moves that row's FP8 scale by
    # 2^-8 and about 1/23 of its codes by one e4m3 step
    tol = 2e-3 if w.quant == "bf16" else 1e-2
    ok = bool(err <= tol and per_tok.max() <= (tol if w.quant == "bf16" else 5e-2))
    used = len(np.unique(ref["ids"])) + w.n_shared
    cb = dict(value=round(w.flops() / dt / 1e12, 6), unit="TFLOP/s", cores=threads, kind="oracle",
              sample=f"the whole {w.T}-token batch, once: routing, permutation, x quantization, quantization of "
                     f"the {used} used experts' weights from bf16 masters, float64 expert GEMMs (experts mapped "
                     f"over {threads} host threads), act quantization, combine; {dt:.1f} s",
              seconds=round(dt, 2), tokens_per_s=round(w.T / dt, 1), cpu_model=cpu_model())
    return cb, ok, dict(rel_l2=err, per_token_max=float(per_tok.max()), tokens=int(w.T))


def time_payloads(torch, mlr, x, steps, warmup):
    """Pack and unpack of the expert-parallel payloads (MXFP4 dispatch, FP8
    blockwise combine) of the workload's x rows: HIP events on the current
    stream; bytes = bf16 rows + payload rows per call."""
    T, D = x.shape
    res = {"T": T, "D": D}
    for fmt in ("mxfp4", "fp8_block"):
        n = mlr.ep_payload_bytes(D, fmt)
        p = torch.empty((T, n), dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        r = {"row_bytes": n}
        for name, fn in (("pack", lambda: mlr.ep_pack(x, fmt, out=p)), ("unpack", lambda: mlr.ep_unpack(p, D, fmt, out=y))):
            for _ in range(warmup):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / steps * 1e3
            gbs = (T * D * 2 + T * n) / (us * 1e-6) / 1e9
            r[name + "_us"] = round(us, 2)
            r[name + "_GBps"] = round(gbs, 1)
            r[name + "_hbm_frac"] = round(gbs / PEAK_HBM_GBS, 4)
        res[fmt] = r
    return res


OTHER_LAYERS = ("tiny_bf16", "qwen3_30b_a3b_ptpc", "deepseek_r1_block_fp8", "e512_top10_shared_ptpc",
                "qwen3_235b_prefill_mxfp4", "deepseek_r1_mxfp4", "qwen3_235b_prefill_router")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_235b_prefill_ptpc")
    ap.add_argument("--block-m", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-layers", action="store_true", help="skip the legs of the other layer shapes")
    ap.add_argument("--no-payload", action="store_true", help="skip the expert-parallel payload leg")
    ap.add_argument("--no-sclk", action="store_true",
                    help="skip the shader-clock sampling after the timed steps (profiled runs)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="launch one device-to-device copy of this many MiB (a known-size kernel for "
                         "calibrating HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (the layer holds every expert on one MI355X); "
              f"--gpus {args.gpus} / WORLD_SIZE {world} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_layer_router_amd as mlr
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mlr.lib()
    w = synth.get(args.workload)
    log("building", w.name)
    case = Case(mlr, synth, w, keep_masters=not args.no_cpu_baseline)
    if args.copy_probe_mib:
        # one elementwise kernel that reads and writes exactly copy_probe_mib MiB
        src = torch.ones((args.copy_probe_mib << 20) // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    st = Steps(case.layer, w, case.x, case.logits, args.block_m)
    log("block_m", st.B, "max_rows", st.lay["max_rows"])

    # the timed steps: the fused entry, over weight copies in turn when the
    # layer's weights are under 1 GiB
    y_fused = torch.empty_like(st.y)
    ws = case.layer.workspace(w.T, args.block_m)
    layers = weight_copies(mlr, case.layer)
    ncopy = len(layers)
    turn = [0]

    def fwd():
        layers[turn[0] % ncopy].forward(case.x, case.logits, block_m=args.block_m, y=y_fused, workspace=ws)
        turn[0] += 1

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    for _ in range(args.steps):
        fwd()
    f1.record()
    torch.cuda.synchronize()
    ms = f0.elapsed_time(f1) / args.steps
    sclk = None if args.no_sclk else sclk_during(torch, fwd)
    log("sclk", sclk)

    # the step entries, HIP events around the grouped GEMMs (over the same
    # weight copies in turn)
    for i in range(args.warmup):
        st.layer = layers[i % ncopy]
        st.run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(args.steps):
        st.layer = layers[i % ncopy]
        st.run(ev[i])
    t_end.record()
    torch.cuda.synchronize()
    steps_ms = t_start.elapsed_time(t_end) / args.steps
    gu_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    dn_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / args.steps
    log(f"step {ms:.3f} ms (step entries {steps_ms:.3f} ms)  gate_up {gu_ms:.3f} ms  down {dn_ms:.3f} ms")
    same = bool(torch.equal(y_fused.view(torch.int16), st.y.view(torch.int16)))
    inter = case.layer.intermediates(w.T, args.block_m, ws)
    ids = inter["topk_ids"].cpu().numpy()
    counts = inter["counts"].cpu().numpy()
    routed = counts[:w.E]
    # expert load of the batch (the gating load the pages monitor) and the
    # rows the grouped GEMMs run after padding and 32-row pad-tile skipping
    load = {"active_experts": int((routed > 0).sum()), "rows_per_expert_mean": round(float(routed.mean()), 1),
            "rows_per_expert_max": int(routed.max()), "rows_per_expert_min": int(routed.min()),
            "padded_rows": int(inter["offsets"][-1].item()),
            "computed_rows": int((-(-counts // 32) * 32).sum()) if st.B > 16 else int(counts.sum())}

    rows = w.T * (w.k + w.n_shared)
    flops = w.flops()
    gu_flops = 2.0 * rows * 2 * w.I * w.D
    dn_flops = 2.0 * rows * w.D * w.I
    peak = PEAK_TFLOPS[w.quant]
    tflops = flops / (ms * 1e-3) / 1e12
    gu_tf = gu_flops / (gu_ms * 1e-3) / 1e12
    # the gate/up launch is MFMA-bound when its flops per algorithmic byte
    # exceed the ridge (peak flops / 8 TB/s), else HBM-bound
    gu_bytes = gateup_bytes(w, ids)
    if gu_flops / gu_bytes >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "kernel": "grouped_gemm_gateup_silu", "achieved": round(gu_tf, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(gu_tf / peak, 4)}
    else:
        gbs = gu_bytes / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "grouped_gemm_gateup_silu", "achieved": round(gbs, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    roof.update(traffic=measured_traffic(w.name), avg_launch_ms=round(gu_ms, 4), flops_per_launch=gu_flops,
                bytes_per_launch=int(gu_bytes))
    layer_bytes = active_expert_bytes(w, ids)[0] + w.T * w.D * (2 + 2) + (0 if case.logits is None else 4 * w.T * w.E)
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"bf16": "bf16", "mxfp4": "fp4_e2m1"}.get(w.quant, "fp8_e4m3"), "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "D": w.D, "E": w.E, "top_k": w.k, "I": w.I,
                   "n_shared": w.n_shared, "quant": w.quant, "scoring": w.scoring, "block_m": st.B},
        "roofline": roof,
        "kernels": {"gateup_ms": round(gu_ms, 4), "down_ms": round(dn_ms, 4),
                    "down_tflops": round(dn_flops / (dn_ms * 1e-3) / 1e12, 1),
                    "gemms_frac_of_peak": round((gu_flops + dn_flops) / ((gu_ms + dn_ms) * 1e-3) / 1e12 / peak, 4),
                    "rest_ms": round(ms - gu_ms - dn_ms, 4)},
        "layer": {"tflops": round(tflops, 1), "frac_mfma": round(tflops / peak, 4), "algorithmic_bytes": int(layer_bytes),
                  "weight_copies": ncopy,
                  "GBps": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
                  "frac_hbm": round(layer_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "routing": load,
        "sclk": sclk,
        "step_entries_ms_per_step": round(steps_ms, 4), "step_entries_equal_fused": same,
        "tokens_per_s": round(w.T / (ms * 1e-3), 1),
    }
    del st, layers
    if w.D % 128 == 0 and not args.no_payload:
        log("expert-parallel payloads")
        out["ep_payload"] = time_payloads(torch, mlr, case.x, args.steps, args.warmup)
    if not args.no_decode and w.name != "qwen3_235b_decode_ptpc":
        log("decode leg")
        out["decode"] = time_decode(torch, mlr, synth, max(args.steps, 100), args.warmup)
        log("decode leg, MXFP4")
        out["decode_mxfp4"] = time_decode(torch, mlr, synth, max(args.steps, 100), args.warmup,
                                          name="qwen3_235b_decode_mxfp4")
    if not args.no_cpu_baseline:
        log("cpu baseline: the oracle over the whole batch")
        cb, ok, par = cpu_baseline(case, y_fused)
        out["cpu_baseline"] = cb
        out["parity"] = par
        log(f"oracle {cb['seconds']} s; parity rel_l2 {par['rel_l2']:.2e}, per-token max {par['per_token_max']:.2e}")
        if not ok:
            log("PARITY FAILED against the oracle")
            out["value"] = None
            print(json.dumps(out), flush=True)
            sys.exit(1)
    case.w13 = case.w2 = None
    torch.cuda.empty_cache()
    if not args.no_layers:
        out["layers"] = {}
        for name in OTHER_LAYERS:
            if name == w.name:
                continue
            log("layer leg", name)
            out["layers"][name] = time_layer(torch, mlr, synth, name, args.steps, args.warmup)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
