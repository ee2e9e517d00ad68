"""Fused Mixture-of-Experts layer forward for AMD Instinct MI355X (gfx950).

Every step runs in the hand-written HIP kernels of ``libmoe.so`` behind the C
ABI in ``include/moe.h``; this package only marshals torch tensors to it.
"""

from ._lib import MoEError, lib  # noqa: F401
from .ops import (LayerWeights, MoELayer, ep_pack, ep_payload_bytes, ep_unpack,  # noqa: F401
                  permute_align, permute_max_rows, quant_mxfp4, quant_ptpc_fp8, quant_weight_fp8,
                  quant_weight_mxfp4, route_topk,
                  router_logits, unblock_weights, unpermute_combine, validate_inputs)
