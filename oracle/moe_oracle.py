"""Plain, slow CPU oracle of the routed Mixture-of-Experts layer forward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use this module.  It shares no code,
table or constant generator with the HIP library, and imports nothing from it.

Sources (the pages this follows; each function cites the passage it uses):

* [QWEN-MI300X] "Unleashing Computational Power: Ultimate Latency Optimization
  of Qwen3 and Qwen3-VL on AMD MI300X Series" (LMSYS blog), section 2.1.1
  "GEMM Quantization Strategy" and Figure 3 (PTPC-FP8: one scale per token for
  activations, one scale per output channel for weights), section 2.1.4
  "MoE Optimization".
* [TPU-QWEN35] "Systems engineering playbook: optimizing Qwen 3.5 397B MoE on
  Ironwood TPU7x" (Google Developers Blog): the MoE paragraph of the model
  description (router gate, soft-max top-k over routed experts, one always-on
  shared expert), the routing-metadata item of the expert-parallel section
  (expert ids and top-k weights as two [tokens, k] arrays), the SparseCore
  permutation item (gather of token rows into a contiguous per-expert
  buffer), the GMM V2 item (grouped GEMM with gate and up packed in one tile
  and SwiGLU fused; bounded per-expert slices with minimal padding), the
  SparseCore unpermutation item (gather plus local weighted reduction) and
  the "Numerical Verification Layer" paragraph.
* [MI355X-MORI] "Win on TCO: How AMD Instinct MI355X Achieves Cost-Competitive
  Distributed Inference Through SGLang with MoRI", section "Hybrid FP4/FP8
  quantized all-to-all" (DeepSeek-R1 hidden size 7168, top-8 routing, FP8
  blockwise quantization with one fp32 scale per 128 elements).

Precision: every contraction and sum is done in float64.  Results are rounded
only at the storage points the layer declares (bf16 act, e4m3fn codes, bf16
or fp32 expert outputs, bf16 y), so that the GPU's own rounding is mirrored.

Readings where the pages are silent (the same list is kept with the design
notes): top-k ties go to the lower expert index and +0 equals -0; the k
outputs are ordered by descending key; routing weights stay fp32; the
quantizer is scale = amax/448 and codes = e4m3fn_rne(x * (448/amax)) with
both divisions IEEE fp32; an all-zero group has scale 1; e4m3fn keeps
subnormals and the sign of zero and saturates to +-448; act is stored bf16;
expert outputs are fp32 in the bf16 mode and bf16 in the FP8 modes; the
combine sums j = 0..k-1 in order, then the shared expert, with one final
bf16 rounding; the grouped-sigmoid group score is the sum of the two largest
selection keys of the group (the DeepSeek-V3/R1 convention).

Pins (tests/test_oracle_*.py): every function here is checked against
something other than itself -- torch CPU dtype casts and brute-force
nearest-code search for the codecs, rank-counting brute force for top-k and
group selection, Python ``sorted`` for the permutation, a dense SwiGLU MLP
(E=1, top-1) and a per-token pure-Python evaluation for the layer, and
invariants (identical experts, token-order permutation).  The pages print no
worked example of a whole layer; moe_forward is pinned by the per-token
evaluation and the dense identities at small sizes and runs the same code at
full size.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Dict, Optional, Tuple

import numpy as np

__all__ = [
    "E4M3_MAX", "bf16_round", "bf16_bits", "bf16_from_bits",
    "e4m3_value", "e4m3_encode", "quant_rows", "quant_weight_blocks",
    "dequant_rows", "dequant_weight_blocks",
    "router_logits", "route_softmax_topk", "route_sigmoid_grouped",
    "permute_max_rows", "permute_align",
    "LayerSpec", "ExpertBank", "expert_gateup_silu", "expert_down", "combine",
    "moe_forward", "moe_forward_tokens", "relative_l2",
    "E2M1_MAGNITUDES", "e2m1_value", "e2m1_encode", "mxfp4_quant", "mxfp4_payload", "mxfp4_unpack",
    "fp8_block_payload", "fp8_block_unpack", "ep_payload_bytes", "mxfp4_dequant",
]

E4M3_MAX = 448.0          # largest finite OCP e4m3fn magnitude (S.1111.110)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def bf16_round(a) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    bfloat16 keeps the upper 16 bits of an IEEE binary32.  Rounding adds
    0x7FFF plus the lowest kept bit before truncating (round half to even).
    Returns float32 values that are exactly representable in bf16.
    """
    a = np.asarray(a, dtype=np.float32)
    f = np.ascontiguousarray(a)
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)
    out = (u << np.uint64(16)).astype(np.uint32)
    return out.view(np.float32).reshape(a.shape)


def bf16_bits(a) -> np.ndarray:
    """uint16 bit patterns of ``bf16_round(a)``."""
    r = bf16_round(a)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(bits) -> np.ndarray:
    """float32 values of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def e4m3_value(codes) -> np.ndarray:
    """float64 value of OCP e4m3fn codes (1 sign, 4 exponent, 3 mantissa bits).

    Exponent bias 7.  Exponent field 0 holds subnormals m * 2^-9; field
    1..15 holds (1 + m/8) * 2^(e-7); only S.1111.111 is NaN (no infinities).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """Encode float32 values as e4m3fn codes: round to nearest, ties to even,
    subnormals kept, sign of zero kept, magnitudes saturated to 448.

    Works on exact float64 copies of the float32 inputs, so every scaling by a
    power of two below is exact and ``np.rint`` (round half to even) performs
    the single rounding.
    """
    f = np.asarray(x, dtype=np.float32)
    neg = np.signbit(f)
    a = np.abs(f.astype(np.float64))
    if np.any(~np.isfinite(a)):
        raise ValueError("e4m3_encode: non-finite input")
    a = np.minimum(a, E4M3_MAX)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: value = m * 2^-9, m = 0..7 (m = 8 is the smallest normal,
    # whose code 0x08 is exactly 8 in this encoding)
    code = np.where(sub, np.rint(a * 2.0 ** 9).astype(np.int64), code)
    # normal range: a = 2^e * (1 + m/8)
    mant, ex = np.frexp(np.where(sub, 1.0, a))        # a = mant * 2^ex, mant in [0.5,1)
    e = ex.astype(np.int64) - 1                       # a = (2*mant) * 2^e
    m = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    ncode = ((e + 7) << 3) | m
    code = np.where(sub, code, ncode)
    code = np.minimum(code, 0x7E)                     # saturate; never 0x7F (NaN)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# PTPC / block FP8 quantization   [QWEN-MI300X] 2.1.1, Fig. 3; [MI355X-MORI]
# --------------------------------------------------------------------------

def _quant_groups(g: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantize each row of ``g`` (float32, [n, len]) with one scale per row."""
    g = np.asarray(g, dtype=np.float32)
    amax = np.max(np.abs(g), axis=1) if g.shape[1] else np.zeros(g.shape[0], np.float32)
    amax = amax.astype(np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    scale = np.where(zero, np.float32(1.0), safe / np.float32(E4M3_MAX)).astype(np.float32)
    inv = np.where(zero, np.float32(1.0), np.float32(E4M3_MAX) / safe).astype(np.float32)
    y = (g * inv[:, None]).astype(np.float32)            # one fp32 multiply
    return e4m3_encode(y), scale


def quant_rows(x, group: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token (group=0) or per-1x``group`` FP8 quantization of a matrix.

    PTPC quantizes each activation row (token) with its own dynamic scale
    ([QWEN-MI300X] 2.1.1, Fig. 3); the blockwise mode uses one fp32 scale per
    128 consecutive elements ([MI355X-MORI], hybrid FP4/FP8 all-to-all).
    The same routine quantizes weights per output channel: a weight matrix
    [N, K] stored row-major has one row per output channel.

    Returns (codes uint8 [M, K], scale float32 [M] or [M, K/group]).
    """
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    if group == 0:
        return _quant_groups(x)
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    codes, scale = _quant_groups(x.reshape(M * (K // group), group))
    return codes.reshape(M, K), scale.reshape(M, K // group)


def quant_weight_blocks(w, blk: int = 128) -> Tuple[np.ndarray, np.ndarray]:
    """Blockwise FP8 weight quantization: one fp32 scale per blk x blk tile of
    a row-major [N, K] weight ([MI355X-MORI] blockwise FP8; block 128 x 128 is
    the DeepSeek-R1 weight layout).  Returns (codes [N, K], scale [N/blk, K/blk]).
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if N % blk or K % blk:
        raise ValueError("N and K must be multiples of the block size")
    tiles = w.reshape(N // blk, blk, K // blk, blk).transpose(0, 2, 1, 3)
    codes, scale = _quant_groups(tiles.reshape(-1, blk * blk))
    codes = codes.reshape(N // blk, K // blk, blk, blk).transpose(0, 2, 1, 3).reshape(N, K)
    return codes, scale.reshape(N // blk, K // blk)


# --------------------------------------------------------------------------
# Expert-parallel payloads   [MI355X-MORI] "Hybrid FP4/FP8 quantized
# all-to-all": tokens go out to their experts as MXFP4 (dispatch) and expert
# outputs come back as FP8 with one fp32 scale per 128 elements (combine);
# for hidden size 7168 the round trip falls from 28,672 to 11,200 bytes per
# token.  MXFP4 is the OCP Microscaling (MX) v1.0 format: blocks of 32
# elements share one E8M0 power-of-two scale; elements are FP4 E2M1
# (1 sign, 2 exponent bits with bias 1, 1 mantissa bit).
# --------------------------------------------------------------------------

E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)   # codes 0..7 (bit 3: sign)


def e2m1_value(codes) -> np.ndarray:
    """float64 value of FP4 E2M1 codes (low 4 bits; bit 3 is the sign)."""
    c = np.asarray(codes, dtype=np.uint8) & 0xF
    exp, man = (c >> 1) & 3, (c & 1).astype(np.float64)
    mag = np.where(exp == 0, man * 0.5, (1.0 + man * 0.5) * np.exp2(exp.astype(np.float64) - 1.0))
    return np.where(c & 8, -mag, mag)


def e2m1_encode(q) -> np.ndarray:
    """Nearest E2M1 code of each value (ties to the even mantissa bit),
    saturating to +-6; the sign bit follows the sign of the input (-0 -> 8).
    Inputs are finite."""
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    mags = np.asarray(E2M1_MAGNITUDES)
    dist = np.abs(a[..., None] - mags)                       # [.., 8]
    best = dist.min(axis=-1, keepdims=True)
    # among the nearest magnitudes take the one whose mantissa bit (code & 1) is 0
    cand = dist == best
    even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    idx = np.where(a > 6.0, 7, idx)
    return (idx | np.where(np.signbit(q), 8, 0)).astype(np.uint8)


def mxfp4_quant(x, block: int = 32) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP4 quantization of the rows of ``x`` [M, K] (K a multiple of 32).

    Per block of 32: amax = max|x|; shared exponent e = floor(log2(amax)) - 2
    (2 is the exponent of E2M1's largest value, 6 = 1.5 * 2^2), clamped to
    [-127, 127]; each element is x / 2^e encoded to E2M1 (round to nearest,
    ties to even, saturating); the scale code is the E8M0 byte e + 127.  An
    all-zero block gets scale code 0 and zero codes.
    Returns (codes uint8 [M, K] in 0..15, scale codes uint8 [M, K/32])."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    b = x.reshape(M, K // block, block)
    amax = np.max(np.abs(b), axis=2)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))           # amax = m * 2^ex, m in [0.5, 1)
    e = np.clip(ex - 1 - 2, -127, 127)
    e = np.where(amax > 0, e, -127)
    q = b / np.exp2(e.astype(np.float64))[:, :, None]          # exact: a power-of-two divisor
    codes = e2m1_encode(q).reshape(M, K)
    return codes, (e + 127).astype(np.uint8)


def mxfp4_payload(x) -> np.ndarray:
    """Dispatch payload of each row of ``x`` [M, K]: K/2 bytes of E2M1 codes
    (element 2i in the low nibble of byte i, 2i+1 in the high nibble), then
    K/32 E8M0 scale bytes.  Returns uint8 [M, K/2 + K/32]."""
    codes, sc = mxfp4_quant(x)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return np.concatenate([packed, sc], axis=1)


def mxfp4_unpack(payload, K: int) -> np.ndarray:
    """float64 values of a dispatch payload [M, K/2 + K/32]: code value *
    2^(scale code - 127)."""
    p = np.asarray(payload, dtype=np.uint8)
    codes = np.empty((p.shape[0], K), np.uint8)
    codes[:, 0::2] = p[:, :K // 2] & 0xF
    codes[:, 1::2] = p[:, :K // 2] >> 4
    e = p[:, K // 2:K // 2 + K // 32].astype(np.float64) - 127.0
    return e2m1_value(codes) * np.repeat(np.exp2(e), 32, axis=1)


def fp8_block_payload(x) -> np.ndarray:
    """Combine payload of each row of ``x`` [M, K]: the K e4m3fn codes of its
    1x128 blockwise quantization, then its K/128 fp32 scales (little-endian
    bytes).  Returns uint8 [M, K + 4 K/128]."""
    codes, sc = quant_rows(x, 128)
    return np.concatenate([codes, np.ascontiguousarray(sc.astype("<f4")).view(np.uint8)], axis=1)


def fp8_block_unpack(payload, K: int) -> np.ndarray:
    """bf16 values (as float32) of a combine payload: fp32(code value *
    scale), one fp32 product, then rounded to bf16."""
    p = np.asarray(payload, dtype=np.uint8)
    v = e4m3_value(p[:, :K]).astype(np.float32)
    sc = np.ascontiguousarray(p[:, K:K + 4 * (K // 128)]).view("<f4").astype(np.float32)
    y = (v * np.repeat(sc, 128, axis=1)).astype(np.float32)
    return bf16_round(y)


def ep_payload_bytes(D: int) -> Dict[str, int]:
    """Bytes per token of the dispatch and combine payloads for hidden size D."""
    return {"bf16": 2 * D, "mxfp4": D // 2 + D // 32, "fp8_block": D + 4 * (D // 128)}


_E4M3_TABLE = None


def _code_values(codes) -> np.ndarray:
    """float64 values of codes through a 256-entry table built by e4m3_value."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = e4m3_value(np.arange(256, dtype=np.uint8))
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def dequant_rows(codes, scale, group: int = 0) -> np.ndarray:
    """float64 values code_value * scale for row/group scales."""
    v = _code_values(codes)
    s = np.asarray(scale, dtype=np.float64)
    if group == 0:
        return v * s[:, None]
    return v * np.repeat(s, group, axis=1)


def dequant_weight_blocks(codes, scale, blk: int = 128) -> np.ndarray:
    v = _code_values(codes)
    s = np.asarray(scale, dtype=np.float64)
    return v * np.repeat(np.repeat(s, blk, axis=0), blk, axis=1)


# --------------------------------------------------------------------------
# router   [TPU-QWEN35] MoE paragraph, routing metadata; roadmap (top-k)
# --------------------------------------------------------------------------

def router_logits(x, router_w) -> np.ndarray:
    """logits[t, e] = sum_d x[t, d] * Wr[e, d]; float64 sum, stored fp32.
    The router gate projects each token onto the experts ([TPU-QWEN35])."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(router_w, dtype=np.float64)
    return (x @ w.T).astype(np.float32)


def _order_desc(keys: np.ndarray) -> np.ndarray:
    """Per row, column indices sorted by key descending, then index ascending.
    Keys compare by value, so +0 and -0 tie and the lower index wins."""
    keys = np.asarray(keys, dtype=np.float64)
    T, E = keys.shape
    idx = np.broadcast_to(np.arange(E), (T, E))
    out = np.empty((T, E), dtype=np.int64)
    for t in range(T):
        out[t] = np.lexsort((idx[t], -keys[t]))
    return out


def route_softmax_topk(logits, k: int, renormalize: bool = True
                       ) -> Tuple[np.ndarray, np.ndarray]:
    """Soft-max top-k routing ([TPU-QWEN35] MoE paragraph: the router selects
    the top routed experts from a soft-max distribution).

    Selection is on the raw fp32 logits (soft-max is strictly increasing, so
    this is the same choice as on probabilities).  ids[t] lists the k experts by
    descending logit, ties to the lower index.  With renormalize the weights
    are the soft-max over the k selected logits (equal to the full soft-max
    divided by the selected mass); without it, the full soft-max values.
    Returns ids int32 [T, k] and w float32 [T, k].
    """
    l = np.asarray(logits, dtype=np.float32)
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = _order_desc(l)[:, :k]
    sel = np.take_along_axis(l.astype(np.float64), order, axis=1)
    lmax = l.astype(np.float64).max(axis=1, keepdims=True) if E else 0.0
    num = np.exp(sel - lmax)
    if renormalize:
        den = num.sum(axis=1, keepdims=True)
    else:
        den = np.exp(l.astype(np.float64) - lmax).sum(axis=1, keepdims=True)
    w = (num / den).astype(np.float32)
    return order.astype(np.int32), w


def route_sigmoid_grouped(logits, k: int, n_groups: int, topk_groups: int,
                          sel_bias=None, route_scale: float = 1.0,
                          renormalize: bool = True
                          ) -> Tuple[np.ndarray, np.ndarray]:
    """Grouped sigmoid routing of the DeepSeek-R1-shaped layer (256 experts in
    8 groups, top-4 groups, top-8 experts, weights normalized then scaled).

    score s = sigmoid(logit) stored fp32; selection key = fp32(s + bias);
    group score = fp32 sum of the two largest keys in the group; keep the
    ``topk_groups`` best groups (ties to the lower group); pick the top-k
    experts by key among kept groups (ties to the lower expert); weights are
    the unbiased s of the picks, divided by their sum when renormalizing, times
    ``route_scale``.  The page on MI355X DeepSeek-R1 serving ([MI355X-MORI])
    fixes top-8 routing over hidden 7168; the group rule is a reading.
    """
    l = np.asarray(logits, dtype=np.float32)
    T, E = l.shape
    if E % n_groups or not 1 <= topk_groups <= n_groups:
        raise ValueError("bad grouping")
    gsz = E // n_groups
    if not 1 <= k <= topk_groups * gsz:
        raise ValueError("k larger than the experts of the kept groups")
    s = (1.0 / (1.0 + np.exp(-l.astype(np.float64)))).astype(np.float32)
    bias = np.zeros(E, np.float32) if sel_bias is None else np.asarray(sel_bias, np.float32)
    key = (s + bias[None, :]).astype(np.float32)
    if gsz >= 2:
        top2 = -np.sort(-key.reshape(T, n_groups, gsz), axis=2)[:, :, :2]
        gscore = (top2[:, :, 0] + top2[:, :, 1]).astype(np.float32)
    else:
        gscore = key.reshape(T, n_groups).astype(np.float32)
    gorder = _order_desc(gscore)[:, :topk_groups]
    keep = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(keep, gorder, True, axis=1)
    keep_e = np.repeat(keep, gsz, axis=1)
    masked = np.where(keep_e, key.astype(np.float64), -np.inf)
    order = _order_desc(masked)[:, :k]
    ssel = np.take_along_axis(s.astype(np.float64), order, axis=1)
    if renormalize:
        w = ssel / ssel.sum(axis=1, keepdims=True) * float(route_scale)
    else:
        w = ssel * float(route_scale)
    return order.astype(np.int32), w.astype(np.float32)


# --------------------------------------------------------------------------
# permutation   [TPU-QWEN35] SparseCore permutation, GMM V2 bounded slices
# --------------------------------------------------------------------------

def permute_max_rows(T: int, k: int, E: int, n_shared: int, block_m: int) -> int:
    """Upper bound on the padded permuted row count.

    Each expert segment is padded to a multiple of block_m, so the block
    count is sum_e ceil(c_e / B) <= (A' + E'(B-1)) / B, and also <= A' because
    a non-empty segment has at least one row per block.
    """
    A = T * (k + n_shared)
    Ep = E + n_shared
    blocks = min((A + Ep * (block_m - 1)) // block_m, A)
    return blocks * block_m


def permute_align(ids, E: int, n_shared: int, block_m: int) -> Dict[str, np.ndarray]:
    """Stable permutation of routed rows by expert, padded per expert.

    Row (t, j) of the routing output has flat index t*k + j.  Shared-expert
    rows (n_shared = 1) are expert E with flat index T*k + t.  Within each
    expert, rows keep ascending flat order.  Each segment is padded to a
    multiple of block_m with the sentinel T*(k + n_shared); padding keeps the
    per-expert slices bounded and contiguous ([TPU-QWEN35] GMM V2 bounded
    slices, SparseCore permutation into a contiguous buffer).

    Returns counts [E'], offsets [E'+1] (padded exclusive prefix sums),
    sorted_ids [max_rows], block_expert [max_rows/B] (-1 past the end) and
    inv_perm [T*(k+n_shared)] (flat index -> permuted row).

    A routed pick outside [0, E) (the pages define no such id) gets no row:
    it is not counted, appears nowhere in sorted_ids and has inv_perm -1.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape if ids.ndim == 2 else (0, 0)
    Ep = E + n_shared
    A = T * (k + n_shared)
    flat_e = ids.reshape(-1)
    if n_shared:
        flat_e = np.concatenate([flat_e, np.full(T, E, dtype=np.int64)])
    valid = np.ones(A, dtype=bool)
    valid[:T * k] = (flat_e[:T * k] >= 0) & (flat_e[:T * k] < E)
    counts = np.bincount(flat_e[valid], minlength=Ep).astype(np.int64)[:Ep]
    padded = (counts + block_m - 1) // block_m * block_m
    offsets = np.zeros(Ep + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    max_rows = permute_max_rows(T, k, E, n_shared, block_m)
    sentinel = A
    sorted_ids = np.full(max_rows, sentinel, dtype=np.int64)
    inv_perm = np.full(A, -1, dtype=np.int64)
    fill = offsets[:-1].copy()
    for f in range(A):                       # ascending flat index => stable
        if not valid[f]:
            continue
        e = flat_e[f]
        sorted_ids[fill[e]] = f
        inv_perm[f] = fill[e]
        fill[e] += 1
    nblocks = max_rows // block_m
    block_expert = np.full(nblocks, -1, dtype=np.int64)
    for e in range(Ep):
        block_expert[offsets[e] // block_m: offsets[e + 1] // block_m] = e
    i32 = lambda a: a.astype(np.int32)
    return dict(counts=i32(counts), offsets=i32(offsets), sorted_ids=i32(sorted_ids),
                block_expert=i32(block_expert), inv_perm=i32(inv_perm),
                max_rows=max_rows, sentinel=sentinel)


# --------------------------------------------------------------------------
# expert computation   [TPU-QWEN35] GMM V2; [QWEN-MI300X] 2.1.1 PTPC
# --------------------------------------------------------------------------

QUANT_NONE, QUANT_PTPC, QUANT_BLOCK, QUANT_MXFP4 = "bf16", "ptpc_fp8", "block128_fp8", "mxfp4"


def mxfp4_dequant(codes, scale_codes, block: int = 32) -> np.ndarray:
    """float64 values of MXFP4 data: E2M1 code value * 2^(scale code - 127),
    one scale per ``block`` consecutive elements of a row ([MI355X-MORI]
    A4W4: 4-bit weights and activations with E8M0 block scales)."""
    v = e2m1_value(codes)
    e = np.asarray(scale_codes, dtype=np.float64) - 127.0
    return v * np.repeat(np.exp2(e), block, axis=-1)


@dataclass
class LayerSpec:
    D: int
    I: int
    E: int
    top_k: int
    n_shared: int = 0
    scoring: str = "softmax"          # or "sigmoid_grouped"
    n_groups: int = 1
    topk_groups: int = 1
    renormalize: bool = True
    route_scale: float = 1.0
    quant: str = QUANT_NONE           # "bf16" | "ptpc_fp8" | "block128_fp8" | "mxfp4"


class ExpertBank:
    """Expert weights as the method uses them.

    ``master(e)`` returns the bf16-valued master weights (W13 [2I, D] with the
    gate rows first and the up rows after them, W2 [D, I]) as float32 arrays.
    In the FP8 modes the bank quantizes them itself, per output channel (PTPC)
    or per 128 x 128 block, and in the MXFP4 mode to E2M1 codes with one E8M0
    scale per 32 elements of each row (along the reduction dimension), and
    keeps the float64 dequantized copies it uses.
    Expert index E is the shared expert when the layer has one.
    """

    def __init__(self, spec: LayerSpec, master: Callable[[int], Tuple[np.ndarray, np.ndarray]],
                 cache: bool = True):
        self.spec, self.master, self.cache = spec, master, cache
        self._deq: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}
        self._codes: Dict[int, tuple] = {}

    def quantized(self, e: int):
        """(w13 codes, w13 scale, w2 codes, w2 scale) of expert e (FP8 modes)."""
        if e in self._codes:
            return self._codes[e]
        w13, w2 = self.master(e)
        if self.spec.quant == QUANT_PTPC:
            q13, s13 = quant_rows(w13, 0)
            q2, s2 = quant_rows(w2, 0)
        elif self.spec.quant == QUANT_BLOCK:
            q13, s13 = quant_weight_blocks(w13, 128)
            q2, s2 = quant_weight_blocks(w2, 128)
        elif self.spec.quant == QUANT_MXFP4:
            q13, s13 = mxfp4_quant(w13, 32)
            q2, s2 = mxfp4_quant(w2, 32)
        else:
            raise ValueError("not a quantized layer")
        out = (q13, s13, q2, s2)
        if self.cache:
            self._codes[e] = out
        return out

    def dequantized(self, e: int) -> Tuple[np.ndarray, np.ndarray]:
        if e in self._deq:
            return self._deq[e]
        if self.spec.quant == QUANT_NONE:
            w13, w2 = self.master(e)
            out = (np.asarray(w13, np.float64), np.asarray(w2, np.float64))
        else:
            q13, s13, q2, s2 = self.quantized(e)
            if self.spec.quant == QUANT_PTPC:
                out = (dequant_rows(q13, s13), dequant_rows(q2, s2))
            elif self.spec.quant == QUANT_MXFP4:
                out = (mxfp4_dequant(q13, s13), mxfp4_dequant(q2, s2))
            else:
                out = (dequant_weight_blocks(q13, s13), dequant_weight_blocks(q2, s2))
        if self.cache:
            self._deq[e] = out
        return out


def _silu(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_gateup_silu(a_rows: np.ndarray, w13: np.ndarray, I: int) -> np.ndarray:
    """act = bf16(fp32(silu(g) * u)) with [g | u] = A @ W13^T in float64.

    Gate and up projections are packed in one [2I, D] weight and SwiGLU is
    applied to the pair ([TPU-QWEN35] GMM V2).  ``a_rows`` are the (dequantized)
    activation rows of the tokens routed to this expert.
    """
    h = np.asarray(a_rows, np.float64) @ np.asarray(w13, np.float64).T
    g, u = h[:, :I], h[:, I:]
    return bf16_round((_silu(g) * u).astype(np.float32))


def expert_down(act_rows: np.ndarray, w2: np.ndarray, out_bf16: bool) -> np.ndarray:
    """o = act @ W2^T in float64, stored fp32 (bf16 mode) or bf16 (FP8 modes)."""
    o = (np.asarray(act_rows, np.float64) @ np.asarray(w2, np.float64).T).astype(np.float32)
    return bf16_round(o) if out_bf16 else o


def combine(o_rows: np.ndarray, w: np.ndarray, o_shared: Optional[np.ndarray]) -> np.ndarray:
    """y = bf16(fp32(sum_j w_j * o_j + o_shared)): gather of the expert outputs
    of a token and their weighted local reduction ([TPU-QWEN35] SparseCore
    unpermutation), summed in float64 in the order j = 0..k-1, then shared.

    o_rows: [T, k, D]; w: [T, k]; o_shared: [T, D] or None.
    """
    acc = np.zeros((o_rows.shape[0], o_rows.shape[2]), dtype=np.float64)
    for j in range(o_rows.shape[1]):
        acc = acc + np.asarray(w[:, j], np.float64)[:, None] * np.asarray(o_rows[:, j], np.float64)
    if o_shared is not None:
        acc = acc + np.asarray(o_shared, np.float64)
    return bf16_round(acc.astype(np.float32))


def relative_l2(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / (den if den > 0 else 1.0))


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------

def _route(spec: LayerSpec, logits, sel_bias):
    if spec.scoring == "softmax":
        return route_softmax_topk(logits, spec.top_k, spec.renormalize)
    return route_sigmoid_grouped(logits, spec.top_k, spec.n_groups, spec.topk_groups,
                                 sel_bias, spec.route_scale, spec.renormalize)


def _act_group(spec: LayerSpec) -> int:
    return 128 if spec.quant == QUANT_BLOCK else 0


def _quant_act(spec: LayerSpec, a):
    """Codes and scales of activation rows: per row / 1x128 group (FP8) or
    MXFP4 per 32 elements."""
    if spec.quant == QUANT_MXFP4:
        return mxfp4_quant(a, 32)
    return quant_rows(a, _act_group(spec))


def _dequant_act(spec: LayerSpec, q, sc):
    if spec.quant == QUANT_MXFP4:
        return mxfp4_dequant(q, sc, 32)
    return dequant_rows(q, sc, _act_group(spec))


def _a_rows_of(spec: LayerSpec, xq, sx, x):
    """Dequantized activation rows the GEMMs consume."""
    if spec.quant == QUANT_NONE:
        return np.asarray(x, np.float64)
    return _dequant_act(spec, xq, sx)


def moe_forward(spec: LayerSpec, bank: ExpertBank, x, logits=None, router_w=None,
                sel_bias=None, block_m: int = 16, pmap=map,
                on_expert: Optional[Callable] = None) -> Dict[str, np.ndarray]:
    """Full routed-expert forward over all T tokens, step by step.

    x: [T, D] float32 holding bf16 values.  logits: [T, E] fp32, or None with
    router_w [E, D] given (then the router projection runs first).
    Returns every intermediate: logits, ids, w, the permutation dict, xq/sx
    (FP8 modes), act [max_rows, I] (pad rows zero), aq/sa, out_perm and y.

    Experts are independent given the permutation (each writes only its own
    rows), so the per-expert step may be mapped with ``pmap`` (for example a
    thread pool's ``map``; the result does not depend on it).  ``on_expert``,
    when given, is called after each expert as
    ``on_expert(e, lo, hi, w13, w2, rows)`` with the expert's routed rows
    [lo, hi), its dequantized weights and ``rows``, a dict of that expert's
    rows of act, aq/sa (FP8 modes) and out_perm, so a caller can inspect them
    while the weights are at hand.
    """
    x = np.asarray(x, np.float32)
    T = x.shape[0]
    if logits is None:
        logits = router_logits(x, router_w)
    ids, w = _route(spec, logits, sel_bias)
    perm = permute_align(ids, spec.E, spec.n_shared, block_m)
    k, I, D = spec.top_k, spec.I, spec.D
    out: Dict[str, np.ndarray] = dict(logits=np.asarray(logits, np.float32), ids=ids, w=w, perm=perm)
    xq = sx = None
    if spec.quant != QUANT_NONE:
        xq, sx = _quant_act(spec, x)
        out["xq"], out["sx"] = xq, sx
    a_all = _a_rows_of(spec, xq, sx, x)
    R = perm["max_rows"]
    g = _act_group(spec)
    fp8 = spec.quant != QUANT_NONE          # a quantized layer (FP8 or MXFP4)
    act = np.zeros((R, I), np.float32)
    out_perm = np.zeros((R, D), np.float32)
    if spec.quant == QUANT_MXFP4:
        aq = np.zeros((R, I), np.uint8)
        sa = np.zeros((R, I // 32), np.uint8)
    elif fp8:
        aq = np.zeros((R, I), np.uint8)
        sa = np.ones((R,) if g == 0 else (R, I // g), np.float32)
    offs, srt = perm["offsets"], perm["sorted_ids"]

    def one_expert(e):
        lo, hi = int(offs[e]), int(offs[e]) + int(perm["counts"][e])
        if hi == lo:
            return
        f = srt[lo:hi].astype(np.int64)
        rows = np.where(f < T * k, f // max(k, 1), f - T * k)
        w13, w2 = bank.dequantized(e)
        act[lo:hi] = expert_gateup_silu(a_all[rows], w13, I)
        if fp8:
            # per-row (or per-group) scales: quantizing one expert's rows
            # alone gives the same codes as quantizing the whole buffer
            aq[lo:hi], sa[lo:hi] = _quant_act(spec, act[lo:hi])
            act_in = _dequant_act(spec, aq[lo:hi], sa[lo:hi])
        else:
            act_in = act[lo:hi].astype(np.float64)
        out_perm[lo:hi] = expert_down(act_in, w2, fp8)
        if on_expert is not None:
            rows_of = dict(act=act[lo:hi], out=out_perm[lo:hi])
            if fp8:
                rows_of.update(aq=aq[lo:hi], sa=sa[lo:hi])
            on_expert(e, lo, hi, w13, w2, rows_of)

    for _ in pmap(one_expert, range(spec.E + spec.n_shared)):
        pass
    out["act"] = act
    if fp8:
        out["aq"], out["sa"] = aq, sa
    out["out_perm"] = out_perm
    inv = perm["inv_perm"].astype(np.int64)
    o_rows = out_perm[inv[:T * k]].reshape(T, k, D) if T else np.zeros((0, k, D), np.float32)
    o_sh = out_perm[inv[T * k:]] if spec.n_shared else None
    out["y"] = combine(o_rows, w, o_sh)
    return out


def moe_forward_tokens(spec: LayerSpec, bank: ExpertBank, x_rows, logits_rows,
                       sel_bias=None) -> Dict[str, np.ndarray]:
    """The forward evaluated token by token, for a subset of tokens.

    Every step of the layer is row-independent given the routing, so the
    output of token t depends only on x[t], logits[t] and the weights of the
    experts it picks.  Used to check sampled tokens of full-size workloads.
    Returns ids, w, xq, sx and y for the given rows.
    """
    x_rows = np.asarray(x_rows, np.float32)
    n = x_rows.shape[0]
    ids, w = _route(spec, logits_rows, sel_bias)
    res = dict(ids=ids, w=w)
    xq = sx = None
    if spec.quant != QUANT_NONE:
        xq, sx = _quant_act(spec, x_rows)
        res["xq"], res["sx"] = xq, sx
    a = _a_rows_of(spec, xq, sx, x_rows)
    out_bf16 = spec.quant != QUANT_NONE
    y = np.zeros((n, spec.D), np.float32)
    for t in range(n):
        experts = list(ids[t]) + ([spec.E] if spec.n_shared else [])
        o = []
        for e in experts:
            w13, w2 = bank.dequantized(int(e))
            act = expert_gateup_silu(a[t:t + 1], w13, spec.I)
            if spec.quant != QUANT_NONE:
                aq, sa = _quant_act(spec, act)
                act = _dequant_act(spec, aq, sa)
            o.append(expert_down(act, w2, out_bf16)[0])
        o = np.stack(o)
        y[t] = combine(o[None, :spec.top_k], w[t:t + 1],
                       o[None, spec.top_k] if spec.n_shared else None)[0]
    res["y"] = y
    return res
