"""Pins of the oracle's PTPC / blockwise FP8 quantizer: closed forms of the
scale and of the rounding error, torch's float8 cast as an independent
encoder, element-by-element pure-Python quantization on small inputs, and the
pages' own layout figures."""

import os

import numpy as np
import torch

import oracle as O
from tests.conftest import GOLDEN


def _bf16_values(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return O.bf16_round((rng.standard_normal(shape) * scale).astype(np.float32))


def _py_quant_row(row):
    """One row quantized element by element in plain Python + fp32 numpy
    scalars, encoding each value by exhaustive nearest-code search."""
    table = [float(v) for v in O.e4m3_value(np.arange(0, 0x7F, dtype=np.uint8))]
    amax = np.float32(0.0)
    for v in row:
        amax = max(amax, np.float32(abs(v)))
    if amax == 0:
        scale, inv = np.float32(1.0), np.float32(1.0)
    else:
        scale = np.float32(amax) / np.float32(448.0)
        inv = np.float32(448.0) / np.float32(amax)
    codes = []
    for v in row:
        y = float(np.float32(np.float32(v) * inv))
        a = min(abs(y), 448.0)
        best, bd = None, None
        for c, tv in enumerate(table):
            d = abs(tv - a)
            if bd is None or d < bd or (d == bd and c % 2 == 0):
                best, bd = c, d
        codes.append(best | (0x80 if np.signbit(y) else 0))
    return np.array(codes, np.uint8), np.float32(scale)


def test_quant_rows_vs_python_elementwise():
    x = _bf16_values((6, 40), 11, 3.0)
    x[2] = 0.0
    x[3, :5] = -0.0
    q, s = O.quant_rows(x)
    for r in range(x.shape[0]):
        qr, sr = _py_quant_row(x[r])
        assert np.array_equal(q[r], qr)
        assert s[r] == sr


def test_quant_rows_with_torch_float8_encoder():
    x = _bf16_values((64, 512), 5)
    q, s = O.quant_rows(x)
    amax = np.abs(x).max(axis=1).astype(np.float32)
    inv = (np.full_like(amax, 448.0) / amax).astype(np.float32)
    y = torch.from_numpy((x * inv[:, None]).astype(np.float32))
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    assert np.array_equal(s, (amax / np.float32(448.0)).astype(np.float32))


def test_quant_closed_forms():
    x = _bf16_values((128, 256), 9, 0.05)
    q, s = O.quant_rows(x)
    # every non-zero row attains the largest code magnitude
    assert np.all((q & 0x7F).max(axis=1) == 0x7E)
    # the scale is amax/448 and dequantized values stay within half an e4m3
    # step (2^-4 relative for normals, 2^-10 absolute below 2^-6) of x/scale
    y = x.astype(np.float64) / s[:, None].astype(np.float64)
    v = O.e4m3_value(q)
    a = np.abs(y)
    bound = np.where(a >= 2.0 ** -6, a * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6) + 1e-9
    assert np.all(np.abs(y - v) <= bound)
    # codes keep the sign of x
    nz = x != 0
    assert np.array_equal(np.signbit(x[nz]), (q[nz] & 0x80) != 0)


def test_quant_zero_rows():
    x = np.zeros((3, 256), np.float32)
    x[1] = -0.0
    q, s = O.quant_rows(x)
    assert np.all(s == 1.0)
    assert np.all(q[0] == 0) and np.all(q[1] == 0x80)


def test_quant_group128_is_rowwise_on_128_chunks():
    x = _bf16_values((16, 7168), 4)
    q, s = O.quant_rows(x, 128)
    assert s.shape == (16, 56)
    q2, s2 = O.quant_rows(x.reshape(-1, 128), 0)
    assert np.array_equal(q, q2.reshape(16, 7168)) and np.array_equal(s.reshape(-1), s2)


def test_quant_weight_blocks_by_loops():
    w = _bf16_values((256, 384), 8)
    w[128:256, 0:128] *= 100.0
    w[0:128, 256:384] = 0.0
    q, s = O.quant_weight_blocks(w, 128)
    assert s.shape == (2, 3)
    for bn in range(2):
        for bk in range(3):
            tile = w[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128]
            qt, st = O.quant_rows(tile.reshape(1, -1), 0)
            assert s[bn, bk] == st[0]
            assert np.array_equal(q[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128],
                                  qt.reshape(128, 128))
    assert s[0, 2] == 1.0


def _pins():
    out = {}
    with open(os.path.join(GOLDEN, "page_shape_pins.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, val, _ = [p.strip() for p in line.split("|", 2)]
                out[name] = int(val)
    return out


def test_page_figures_fix_layouts():
    p = _pins()
    # 192 per-channel scales for one TP8 shard of the 1536-wide expert
    # intermediate: one scale per output row of the gate projection shard
    shard = _bf16_values((1536 // 8, 64), 1)
    assert O.quant_rows(shard)[1].shape == (p["tp8_per_channel_scales"],)
    # the permuted buffer of top-10 routing over 8192 tokens has 81920 rows
    # when no padding is applied (block of 1)
    assert O.permute_max_rows(p["permuted_rows_tokens"], p["permuted_rows_topk"], 512, 0, 1) \
        == p["permuted_rows_total"]
    # 1x128 groups over hidden 7168 give 56 scales per token
    assert O.quant_rows(_bf16_values((2, p["r1_hidden"]), 2), p["fp8_block_elems"])[1].shape[1] \
        == p["r1_scale_dim"]
    # an FP8-blockwise token (codes + fp32 scales) is 7392 bytes; the rest of
    # the quantized round trip is the MXFP4 dispatch (4-bit codes plus one byte
    # of scale per 32 elements): 3584 + 224 = 3808; BF16 round trip = 4 bytes
    # per element
    q, s = O.quant_rows(_bf16_values((1, p["r1_hidden"]), 3), 128)
    fp8_token = q.nbytes + s.nbytes
    mxfp4_token = p["r1_hidden"] // 2 + p["r1_hidden"] // 32
    assert fp8_token + mxfp4_token == p["quantized_round_trip_bytes"]
    assert p["r1_hidden"] * 2 * 2 == p["bf16_round_trip_bytes"]
