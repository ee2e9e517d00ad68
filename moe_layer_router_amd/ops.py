"""torch-facing wrappers of the C ABI.

Argument checking and marshalling only: every step of the layer runs in the
HIP kernels of libmoe.so.  torch provides device memory (``torch.empty``) and
the current HIP stream.
"""

from __future__ import annotations

import copy
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L

_U8, _BF16, _F32, _I32 = torch.uint8, torch.bfloat16, torch.float32, torch.int32

# MOE_VALIDATE=1 (read once, at import): MoELayer.forward first counts Inf
# and NaN in x and the logits, and permute_align ids outside [0, E), on the
# GPU (moe_validate_inputs), and raises ValueError if there are any.
VALIDATE = os.environ.get("MOE_VALIDATE", "") == "1"


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, dtype, name: str, shape=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _empty(shape, dtype, like: torch.Tensor) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=like.device)


# ---------------------------------------------------------------- step entries

def validate_inputs(x: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                    ids: Optional[torch.Tensor] = None, E: Optional[int] = None) -> dict:
    """Counts of Inf/NaN in x [T, D] bf16 and logits [T, E] fp32 and of ids
    [T, k] int32 outside [0, E), taken on the GPU (waits for the stream)."""
    ref = next(t for t in (x, logits, ids) if t is not None)
    T = ref.shape[0]
    E = logits.shape[1] if E is None and logits is not None else E
    if x is not None:
        _need(x, _BF16, "x", (T, x.shape[1]))
    if logits is not None:
        _need(logits, _F32, "logits", (T, E))
    if ids is not None:
        _need(ids, _I32, "ids", (T, ids.shape[1]))
    counts = _empty((3,), _I32, ref)
    L.check("moe_validate_inputs", L.lib().moe_validate_inputs(
        _ptr(x), T, 0 if x is None else x.shape[1], _ptr(logits), E or 0, _ptr(ids), 0 if ids is None else ids.shape[1],
        _ptr(counts), _stream()))
    c = counts.tolist()
    return {"x_nonfinite": c[0], "logits_nonfinite": c[1], "ids_out_of_range": c[2]}


def router_logits(x: torch.Tensor, router_w: torch.Tensor) -> torch.Tensor:
    T, D = x.shape
    E = router_w.shape[0]
    _need(x, _BF16, "x")
    _need(router_w, _F32, "router_w", (E, D))
    out = _empty((T, E), _F32, x)
    L.check("moe_router_logits", L.lib().moe_router_logits(_ptr(x), _ptr(router_w), T, D, E, _ptr(out), _stream()))
    return out


def route_topk(logits: torch.Tensor, k: int, scoring: str = "softmax", n_groups: int = 1,
               topk_groups: int = 1, sel_bias: Optional[torch.Tensor] = None, renormalize: bool = True,
               route_scale: float = 1.0):
    T, E = logits.shape
    _need(logits, _F32, "logits")
    if sel_bias is not None:
        _need(sel_bias, _F32, "sel_bias", (E,))
    sc = L.SCORING_SOFTMAX if scoring == "softmax" else L.SCORING_SIGMOID_GROUPED
    ids = _empty((T, k), _I32, logits)
    w = _empty((T, k), _F32, logits)
    L.check("moe_route_topk", L.lib().moe_route_topk(_ptr(logits), T, E, k, sc, n_groups, topk_groups,
                                                      _ptr(sel_bias), int(renormalize), float(route_scale),
                                                      _ptr(ids), _ptr(w), _stream()))
    return ids, w


def permute_max_rows(T: int, k: int, E: int, n_shared: int, block_m: int) -> int:
    return int(L.lib().moe_permute_max_rows(T, k, E, n_shared, block_m))


def permute_align(ids: torch.Tensor, E: int, n_shared: int, block_m: int) -> dict:
    T, k = ids.shape
    if VALIDATE and T > 0:
        bad = validate_inputs(ids=ids, E=E)
        if bad["ids_out_of_range"]:
            raise ValueError(f"MOE_VALIDATE: routed ids outside [0, {E}): {bad['ids_out_of_range']}")
    _need(ids, _I32, "topk_ids")
    R = permute_max_rows(T, k, E, n_shared, block_m)
    Ep = E + n_shared
    out = dict(counts=_empty((Ep,), _I32, ids), offsets=_empty((Ep + 1,), _I32, ids),
               sorted_ids=_empty((R,), _I32, ids), block_expert=_empty((R // block_m,), _I32, ids),
               inv_perm=_empty((T * (k + n_shared),), _I32, ids))
    scratch = _empty((max(1, int(L.lib().moe_permute_scratch_bytes(T, k, n_shared, E))),), _U8, ids)
    L.check("moe_permute_align", L.lib().moe_permute_align(
        _ptr(ids), T, k, E, n_shared, block_m, _ptr(out["counts"]), _ptr(out["offsets"]),
        _ptr(out["sorted_ids"]), _ptr(out["block_expert"]), _ptr(out["inv_perm"]), _ptr(scratch), _stream()))
    out["max_rows"] = R
    return out


def quant_ptpc_fp8(x: torch.Tensor, group: int = 0, valid_rows: Optional[torch.Tensor] = None):
    M, K = x.shape
    _need(x, _BF16, "x")
    q = _empty((M, K), _U8, x)
    s = _empty((M,) if group == 0 else (M, K // group), _F32, x)
    L.check("moe_quant_ptpc_fp8", L.lib().moe_quant_ptpc_fp8(_ptr(x), M, K, group, _ptr(valid_rows), _ptr(q),
                                                              _ptr(s), _stream()))
    return q, s


def quant_weight_fp8(w: torch.Tensor, quant: str, layout: str = "blocked"):
    """w: [n_mats, N, K] bf16 -> codes (n_mats x N x K bytes, row-major or in
    16-row x 128-byte blocks; the tensor keeps the [n_mats, N, K] shape),
    scales per row or 128x128 block."""
    n, N, K = w.shape
    _need(w, _BF16, "w")
    code = L.QUANT_CODES[quant]
    q = _empty((n, N, K), _U8, w)
    s = _empty((n, N) if code == L.QUANT_PTPC_FP8 else (n, N // 128, K // 128), _F32, w)
    L.check("moe_quant_weight_fp8", L.lib().moe_quant_weight_fp8(_ptr(w), n, N, K, code, L.LAYOUT_CODES[layout],
                                                                  _ptr(q), _ptr(s), _stream()))
    return q, s


def quant_mxfp4(x: torch.Tensor, valid_rows: Optional[torch.Tensor] = None):
    """MXFP4 rows: codes [M, K/2] uint8 (two E2M1 per byte), E8M0 scales [M, K/32] uint8."""
    M, K = x.shape
    _need(x, _BF16, "x")
    q = _empty((M, K // 2), _U8, x)
    s = _empty((M, K // 32), _U8, x)
    L.check("moe_quant_mxfp4", L.lib().moe_quant_mxfp4(_ptr(x), M, K, _ptr(valid_rows), _ptr(q), _ptr(s), _stream()))
    return q, s


def quant_weight_mxfp4(w: torch.Tensor, layout: str = "blocked"):
    """w: [n_mats, N, K] bf16 -> E2M1 codes [n_mats, N, K/2] (row-major or in
    16-row x 128-byte blocks) and E8M0 scales [n_mats, N, K/32]."""
    n, N, K = w.shape
    _need(w, _BF16, "w")
    q = _empty((n, N, K // 2), _U8, w)
    s = _empty((n, N, K // 32), _U8, w)
    L.check("moe_quant_weight_mxfp4", L.lib().moe_quant_weight_mxfp4(_ptr(w), n, N, K, L.LAYOUT_CODES[layout], _ptr(q),
                                                                      _ptr(s), _stream()))
    return q, s


def unblock_weights(q: torch.Tensor) -> torch.Tensor:
    """Row-major copy of codes [..., N, K] stored in 16-row x 128-byte blocks
    (inside a block: K half h, line l, row parity p, 16-byte piece c, byte
    -> row 2l + p, byte 64h + 16c + byte)."""
    *lead, N, K = q.shape
    b = q.reshape(*lead, N // 16, K // 128, 2, 8, 2, 4, 16)
    nd = b.dim()
    # [.., g, kb, h, l, p, c, x] -> [.., g, l, p, kb, h, c, x]
    perm = list(range(nd - 7)) + [nd - 7, nd - 4, nd - 3, nd - 6, nd - 5, nd - 2, nd - 1]
    return b.permute(*perm).reshape(*lead, N, K)


# ---------------------------------------------------------------- the layer

@dataclass
class LayerWeights:
    w13: torch.Tensor                      # [E', 2I, D] bf16 or u8
    w2: torch.Tensor                       # [E', D, I]
    w13_scale: Optional[torch.Tensor] = None
    w2_scale: Optional[torch.Tensor] = None
    router_w: Optional[torch.Tensor] = None
    sel_bias: Optional[torch.Tensor] = None


class MoELayer:
    """A routed-expert layer on one GPU (all experts resident)."""

    def __init__(self, D: int, I: int, E: int, top_k: int, weights: LayerWeights, quant: str = "bf16",
                 n_shared: int = 0, scoring: str = "softmax", n_groups: int = 1, topk_groups: int = 1,
                 renormalize: bool = True, route_scale: float = 1.0, weight_layout: Optional[str] = None):
        self.D, self.I, self.E, self.top_k, self.n_shared = D, I, E, top_k, n_shared
        self.quant = quant
        self.weights = weights
        # FP8 codes from quant_weight_fp8 are blocked by default; bf16 weights are row-major
        self.weight_layout = weight_layout or ("rows" if quant == "bf16" else "blocked")
        Ep = E + n_shared
        wdt = _BF16 if quant == "bf16" else _U8
        kdiv = 2 if quant == "mxfp4" else 1            # MXFP4: two codes per byte
        _need(weights.w13, wdt, "w13", (Ep, 2 * I, D // kdiv))
        _need(weights.w2, wdt, "w2", (Ep, D, I // kdiv))
        if quant == "ptpc_fp8":
            _need(weights.w13_scale, _F32, "w13_scale", (Ep, 2 * I))
            _need(weights.w2_scale, _F32, "w2_scale", (Ep, D))
        elif quant == "block128_fp8":
            _need(weights.w13_scale, _F32, "w13_scale", (Ep, 2 * I // 128, D // 128))
            _need(weights.w2_scale, _F32, "w2_scale", (Ep, D // 128, I // 128))
        elif quant == "mxfp4":
            _need(weights.w13_scale, _U8, "w13_scale", (Ep, 2 * I, D // 32))
            _need(weights.w2_scale, _U8, "w2_scale", (Ep, D, I // 32))
        if weights.router_w is not None:
            _need(weights.router_w, _F32, "router_w", (E, D))
        if weights.sel_bias is not None:
            _need(weights.sel_bias, _F32, "sel_bias", (E,))
        self.desc = L.LayerDesc(D=D, I=I, E=E, top_k=top_k, n_shared=n_shared,
                                scoring=L.SCORING_SOFTMAX if scoring == "softmax" else L.SCORING_SIGMOID_GROUPED,
                                n_groups=n_groups, topk_groups=topk_groups, renormalize=int(renormalize),
                                route_scale=float(route_scale), quant=L.QUANT_CODES[quant],
                                weight_layout=L.LAYOUT_CODES[self.weight_layout], w13=_ptr(weights.w13), w13_scale=_ptr(weights.w13_scale), w2=_ptr(weights.w2),
                                w2_scale=_ptr(weights.w2_scale), router_w=_ptr(weights.router_w),
                                sel_bias=_ptr(weights.sel_bias))
        self._ws: Optional[torch.Tensor] = None

    @classmethod
    def from_masters(cls, w13_bf16: torch.Tensor, w2_bf16: torch.Tensor, quant: str, router_w=None,
                     sel_bias=None, weight_layout: Optional[str] = None, **kw) -> "MoELayer":
        """Build the layer from bf16 master weights, quantizing them on the GPU
        (per output channel or per 128x128 block) for the FP8 modes, codes in
        16-row x 128-byte blocks unless weight_layout is "rows"."""
        Ep, I2, D = w13_bf16.shape
        if quant == "bf16":
            w = LayerWeights(w13_bf16.contiguous(), w2_bf16.contiguous(), router_w=router_w, sel_bias=sel_bias)
            weight_layout = "rows"
        elif quant == "mxfp4":
            weight_layout = weight_layout or "blocked"
            q13, s13 = quant_weight_mxfp4(w13_bf16.contiguous(), weight_layout)
            q2, s2 = quant_weight_mxfp4(w2_bf16.contiguous(), weight_layout)
            w = LayerWeights(q13, q2, s13, s2, router_w=router_w, sel_bias=sel_bias)
        else:
            weight_layout = weight_layout or "blocked"
            q13, s13 = quant_weight_fp8(w13_bf16.contiguous(), quant, weight_layout)
            q2, s2 = quant_weight_fp8(w2_bf16.contiguous(), quant, weight_layout)
            w = LayerWeights(q13, q2, s13, s2, router_w=router_w, sel_bias=sel_bias)
        return cls(D=D, I=I2 // 2, weights=w, quant=quant, weight_layout=weight_layout, **kw)

    def with_weights(self, weights: LayerWeights) -> "MoELayer":
        """The same layer over other weight tensors of the same shapes, dtypes
        and layout (e.g. copies of this layer's weights)."""
        other = copy.copy(self)
        other.weights = weights
        other.desc = L.LayerDesc.from_buffer_copy(self.desc)
        other.desc.w13, other.desc.w13_scale = _ptr(weights.w13), _ptr(weights.w13_scale)
        other.desc.w2, other.desc.w2_scale = _ptr(weights.w2), _ptr(weights.w2_scale)
        other.desc.router_w, other.desc.sel_bias = _ptr(weights.router_w), _ptr(weights.sel_bias)
        other._ws = None
        return other

    # ---- host-side sizes
    def default_block_m(self, T: int) -> int:
        return int(L.lib().moe_default_block_m(ctypes.byref(self.desc), T))

    def layout(self, T: int, block_m: int = 0) -> dict:
        lay = L.WsLayout()
        L.check("moe_workspace_layout", L.lib().moe_workspace_layout(ctypes.byref(self.desc), T, block_m,
                                                                      ctypes.byref(lay)))
        return {n: getattr(lay, n) for n, _ in L.WsLayout._fields_}

    def workspace(self, T: int, block_m: int = 0, device=None) -> torch.Tensor:
        n = int(L.lib().moe_forward_workspace_size(ctypes.byref(self.desc), T, block_m))
        if n == 0 and T > 0:
            raise L.MoEError("moe_forward_workspace_size", L.MOE_ERR_UNSUPPORTED)
        dev = device if device is not None else self.weights.w13.device
        if self._ws is None or self._ws.numel() < n or self._ws.device != torch.device(dev):
            self._ws = torch.empty((max(n, 256),), dtype=_U8, device=dev)
        return self._ws

    # ---- the step entries that need the layer
    def gateup_silu(self, a, a_scale, T: int, block_m: int, perm: dict, use_counts: bool = True) -> torch.Tensor:
        act = _empty((perm["max_rows"], self.I), _BF16, a)
        L.check("moe_grouped_gemm_gateup_silu", L.lib().moe_grouped_gemm_gateup_silu(
            ctypes.byref(self.desc), _ptr(a), _ptr(a_scale), T, block_m, _ptr(perm["sorted_ids"]),
            _ptr(perm["block_expert"]), _ptr(perm["offsets"]), _ptr(perm["counts"]) if use_counts else None,
            _ptr(act), _stream()))
        return act

    def down(self, act, act_scale, T: int, block_m: int, perm: dict, use_counts: bool = True) -> torch.Tensor:
        out = _empty((perm["max_rows"], self.D), _F32 if self.quant == "bf16" else _BF16, act)
        L.check("moe_grouped_gemm_down", L.lib().moe_grouped_gemm_down(
            ctypes.byref(self.desc), _ptr(act), _ptr(act_scale), T, block_m, _ptr(perm["block_expert"]),
            _ptr(perm["offsets"]), _ptr(perm["counts"]) if use_counts else None, _ptr(out), _stream()))
        return out

    def forward(self, x: torch.Tensor, logits: Optional[torch.Tensor] = None, block_m: int = 0,
                y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        T = x.shape[0]
        _need(x, _BF16, "x", (T, self.D))
        if logits is not None:
            _need(logits, _F32, "logits", (T, self.E))
        if VALIDATE and T > 0:
            bad = validate_inputs(x, logits, E=self.E)
            if bad["x_nonfinite"] or bad["logits_nonfinite"]:
                raise ValueError(f"MOE_VALIDATE: non-finite forward inputs {bad}")
        if y is None:
            y = _empty((T, self.D), _BF16, x)
        ws = workspace if workspace is not None else self.workspace(T, block_m, x.device)
        L.check("moe_forward", L.lib().moe_forward(ctypes.byref(self.desc), _ptr(x), _ptr(logits), T, block_m,
                                                   _ptr(y), _ptr(ws), ws.numel(), _stream()))
        return y

    def intermediates(self, T: int, block_m: int = 0, workspace: Optional[torch.Tensor] = None) -> dict:
        """Views of the intermediates the last forward left in the workspace."""
        lay = self.layout(T, block_m)
        ws = workspace if workspace is not None else self._ws
        R, B = lay["max_rows"], lay["block_m"]
        k, E, Ep, D, I = self.top_k, self.E, self.E + self.n_shared, self.D, self.I
        A = T * (k + self.n_shared)
        blk = self.quant == "block128_fp8"

        def view(name, n, dtype, shape):
            off = lay[name]
            if off < 0:
                return None
            nbytes = n * torch.tensor([], dtype=dtype).element_size()
            return ws[off:off + nbytes].view(dtype).view(*shape)
        out = dict(
            logits=view("logits", T * E, _F32, (T, E)), topk_ids=view("topk_ids", T * k, _I32, (T, k)),
            topk_w=view("topk_w", T * k, _F32, (T, k)), counts=view("counts", Ep, _I32, (Ep,)),
            offsets=view("offsets", Ep + 1, _I32, (Ep + 1,)), sorted_ids=view("sorted_ids", R, _I32, (R,)),
            block_expert=view("block_expert", R // B, _I32, (R // B,)),
            inv_perm=view("inv_perm", A, _I32, (A,)), act=view("act", R * I, _BF16, (R, I)),
            out_perm=view("out_perm", R * D, _F32 if self.quant == "bf16" else _BF16, (R, D)))
        if self.quant == "mxfp4":
            out["xq"] = view("xq", T * D // 2, _U8, (T, D // 2))
            out["xs"] = view("xs", T * D // 32, _U8, (T, D // 32))
            aq = view("aq", R * I // 2, _U8, (R, I // 2))
            out["aq"] = unblock_weights(aq) if B == 16 else aq      # blocked for the streaming down GEMM
            out["as"] = view("as_", R * I // 32, _U8, (R, I // 32))
        elif self.quant != "bf16":
            out["xq"] = view("xq", T * D, _U8, (T, D))
            out["xs"] = view("xs", T * (D // 128 if blk else 1), _F32, (T, D // 128) if blk else (T,))
            aq = view("aq", R * I, _U8, (R, I))
            # the streaming down GEMM (block_m 16) takes act codes in the
            # blocked order; shown row-major here
            out["aq"] = unblock_weights(aq) if B == 16 else aq
            out["as"] = view("as_", R * (I // 128 if blk else 1), _F32, (R, I // 128) if blk else (R,))
        out["max_rows"], out["block_m"] = R, B
        return out


def unpermute_combine(out_perm: torch.Tensor, inv_perm: torch.Tensor, topk_w: torch.Tensor, T: int, k: int,
                      n_shared: int) -> torch.Tensor:
    D = out_perm.shape[1]
    dt = 0 if out_perm.dtype == _F32 else 1
    y = _empty((T, D), _BF16, out_perm)
    L.check("moe_unpermute_combine", L.lib().moe_unpermute_combine(_ptr(out_perm), dt, _ptr(inv_perm),
                                                                    _ptr(topk_w), T, k, n_shared, D, _ptr(y),
                                                                    _stream()))
    return y


# ---------------------------------------------------------------- expert-parallel payloads

def ep_payload_bytes(D: int, fmt: str) -> int:
    """Bytes of one payload row ("mxfp4" dispatch or "fp8_block" combine)."""
    n = L.lib().moe_ep_payload_bytes(D, L.PAYLOAD_CODES[fmt])
    if n < 0:
        raise ValueError(f"no {fmt} payload for D={D} (D must be a positive multiple of 128)")
    return n


def ep_pack(x: torch.Tensor, fmt: str, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Payload rows [T, ep_payload_bytes(D, fmt)] uint8 of bf16 rows x [T, D]."""
    T, D = x.shape
    _need(x, _BF16, "x")
    n = ep_payload_bytes(D, fmt)
    p = out if out is not None else _empty((T, n), torch.uint8, x)
    _need(p, torch.uint8, "payload", (T, n))
    L.check("moe_ep_pack_payload", L.lib().moe_ep_pack_payload(_ptr(x), T, D, L.PAYLOAD_CODES[fmt], _ptr(p),
                                                                _stream()))
    return p


def ep_unpack(payload: torch.Tensor, D: int, fmt: str, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 rows [T, D] of payload rows [T, ep_payload_bytes(D, fmt)]."""
    T = payload.shape[0]
    _need(payload, torch.uint8, "payload", (T, ep_payload_bytes(D, fmt)))
    y = out if out is not None else _empty((T, D), _BF16, payload)
    _need(y, _BF16, "x", (T, D))
    L.check("moe_ep_unpack_payload", L.lib().moe_ep_unpack_payload(_ptr(payload), T, D, L.PAYLOAD_CODES[fmt],
                                                                    _ptr(y), _stream()))
    return y
