"""ctypes view of ``libmoe.so`` (the C ABI declared in include/moe.h).

Loading fails loudly when the library has not been built: there is no other
implementation of these entry points.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p, c_char_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, 1, 2, 3, 4
SCORING_SOFTMAX, SCORING_SIGMOID_GROUPED = 0, 1
QUANT_NONE_BF16, QUANT_PTPC_FP8, QUANT_BLOCK128_FP8, QUANT_MXFP4 = 0, 1, 2, 3
QUANT_CODES = {"bf16": QUANT_NONE_BF16, "ptpc_fp8": QUANT_PTPC_FP8, "block128_fp8": QUANT_BLOCK128_FP8,
               "mxfp4": QUANT_MXFP4}
WEIGHTS_ROWS, WEIGHTS_BLOCKED = 0, 1
LAYOUT_CODES = {"rows": WEIGHTS_ROWS, "blocked": WEIGHTS_BLOCKED}
PAYLOAD_MXFP4, PAYLOAD_FP8_BLOCK = 0, 1
PAYLOAD_CODES = {"mxfp4": PAYLOAD_MXFP4, "fp8_block": PAYLOAD_FP8_BLOCK}
NOALLOC_SCRATCH_BYTES = 96 << 20      # MOE_NOALLOC_SCRATCH_BYTES


class LayerDesc(ctypes.Structure):
    _fields_ = [("D", c_int32), ("I", c_int32), ("E", c_int32), ("top_k", c_int32), ("n_shared", c_int32),
                ("scoring", c_int32), ("n_groups", c_int32), ("topk_groups", c_int32),
                ("renormalize", c_int32), ("route_scale", c_float), ("quant", c_int32),
                ("weight_layout", c_int32), ("w13", c_void_p), ("w13_scale", c_void_p), ("w2", c_void_p), ("w2_scale", c_void_p),
                ("router_w", c_void_p), ("sel_bias", c_void_p)]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, c_int64) for n in ("logits", "topk_ids", "topk_w", "counts", "offsets", "sorted_ids",
                                       "block_expert", "inv_perm", "xq", "xs", "act", "aq", "as_",
                                       "out_perm", "scratch", "router", "total", "max_rows")] + [("block_m", c_int32)]


# name -> (restype, argtypes)
SIGNATURES = {
    "moe_status_str": (c_char_p, [c_int32]),
    "moe_router_logits": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "moe_router_front_workspace_size": (c_size_t, [POINTER(LayerDesc)]),
    "moe_router_front": (c_int32, [POINTER(LayerDesc), c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_route_topk": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                 c_int32, c_float, c_void_p, c_void_p, c_void_p]),
    "moe_permute_max_rows": (c_int64, [c_int32, c_int32, c_int32, c_int32, c_int32]),
    "moe_permute_scratch_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "moe_permute_align": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_quant_ptpc_fp8": (c_int32, [c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                     c_void_p]),
    "moe_quant_mxfp4": (c_int32, [c_void_p, c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_quant_weight_mxfp4": (c_int32, [c_void_p, c_int64, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                         c_void_p]),
    "moe_quant_weight_fp8": (c_int32, [c_void_p, c_int64, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                       c_void_p, c_void_p]),
    "moe_grouped_gemm_gateup_silu": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_int32,
                                               c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_grouped_gemm_down": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_unpermute_combine": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                        c_int32, c_void_p, c_void_p]),
    "moe_default_block_m": (c_int32, [POINTER(LayerDesc), c_int32]),
    "moe_forward_workspace_size": (c_size_t, [POINTER(LayerDesc), c_int32, c_int32]),
    "moe_workspace_layout": (c_int32, [POINTER(LayerDesc), c_int32, c_int32, POINTER(WsLayout)]),
    "moe_forward": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                              c_size_t, c_void_p]),
    "moe_forward_noalloc": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                      c_void_p]),
    "moe_ep_payload_bytes": (c_int64, [c_int32, c_int32]),
    "moe_ep_pack_payload": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "moe_ep_unpack_payload": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "moe_validate_inputs": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_int32, c_void_p, c_int32, c_void_p,
                                      c_void_p]),
}

_LIB = None


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_str(status)})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m moe_layer_router_amd.build` "
                              "(the MoE layer has no non-HIP implementation)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _LIB = l
    return _LIB


def status_str(s: int) -> str:
    return lib().moe_status_str(s).decode()


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoEError(fn, status)
