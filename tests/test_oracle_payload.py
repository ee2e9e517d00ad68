"""Pins of the oracle's expert-parallel payload formats (MXFP4 dispatch,
FP8-blockwise combine) against things other than the oracle itself: the OCP
E2M1 code table, a nearest-value property check over every midpoint, the
MX shared-exponent rule found by search, closed-form error bounds, exact
round trips of representable values, and the byte counts the MoRI page
prints."""

import os

import numpy as np
import pytest

import oracle as O
from tests.conftest import GOLDEN


def _table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    return rows


def _pins():
    out = {}
    with open(os.path.join(GOLDEN, "page_shape_pins.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, val, _ = [t.strip() for t in line.split("|", 2)]
                out[name] = int(val)
    return out


def test_e2m1_value_matches_spec_table():
    for code, val in _table("e2m1_codes.txt"):
        got = O.e2m1_value(np.array([code], np.uint8))[0]
        assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e2m1_encode_is_nearest_with_ties_to_even_and_saturation():
    mags = np.array([v for c, v in _table("e2m1_codes.txt") if c < 8])
    mids = (mags[1:] + mags[:-1]) / 2
    dense = np.concatenate([mags, mids, np.nextafter(mids, 0), np.nextafter(mids, 10),
                            np.linspace(0, 7.9, 4001), [6.0, 6.5, 7.0, 100.0, 1e30]])
    vals = np.concatenate([dense, -dense])
    codes = O.e2m1_encode(vals)
    got = O.e2m1_value(codes)
    for v, c, g in zip(vals, codes, got):
        a = abs(v)
        if a > 6.0:
            assert abs(g) == 6.0
        else:
            d = np.abs(mags - a)
            assert abs(abs(g) - a) == d.min(), (v, g)
            ties = np.flatnonzero(d == d.min())
            if len(ties) > 1:                       # exact midpoint: even mantissa bit
                assert (c & 1) == 0, (v, c)
        assert bool(c & 8) == bool(np.signbit(v))
    # the midpoints themselves, spelled out from the table
    want = {0.25: 0x0, 0.75: 0x2, 1.25: 0x2, 1.75: 0x4, 2.5: 0x4, 3.5: 0x6, 5.0: 0x6}
    for v, c in want.items():
        assert O.e2m1_encode(np.array([v]))[0] == c
        assert O.e2m1_encode(np.array([-v]))[0] == c | 8


def _blocks(rng, M, K):
    x = rng.standard_normal((M, K)) * np.exp2(rng.integers(-30, 30, size=(M, 1)))
    x[0, :32] = 0.0                                  # all-zero block
    x[1, 32:64] = rng.standard_normal(32) * 1e-40    # bf16/fp32 subnormal range
    x[2, :32] = np.linspace(-5.0, 5.0, 32)           # amax exactly 5
    return x.astype(np.float32).astype(np.float64)


def test_mxfp4_shared_exponent_by_search_and_error_bound():
    rng = np.random.default_rng(11)
    x = _blocks(rng, 6, 128)
    codes, sc = O.mxfp4_quant(x)
    dq = O.e2m1_value(codes) * np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1)
    for m in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            blk = x[m, 32 * b:32 * b + 32]
            amax = np.max(np.abs(blk))
            if amax == 0:
                assert sc[m, b] == 0 and np.all((codes[m, 32 * b:32 * b + 32] & 7) == 0)
                continue
            # the exponent e with 4 <= amax / 2^e < 8, found by search
            e0 = next(e for e in range(-200, 200) if 4.0 <= amax / 2.0 ** e < 8.0)
            e = max(e0, -127)                        # E8M0's smallest scale is 2^-127
            assert sc[m, b] == e + 127
            X = 2.0 ** e
            # error bound: half the local code spacing, or the saturation gap
            q = np.abs(blk) / X
            spacing = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0))
            bound = np.where(q > 6, q - 6, spacing / 2) * X
            assert np.all(np.abs(blk - dq[m, 32 * b:32 * b + 32]) <= bound * (1 + 1e-12))
            # the block's largest element lands on 4 or 6 (amax/X is in [4, 8))
            if e0 >= -127:
                assert np.max(np.abs(dq[m, 32 * b:32 * b + 32])) in (4 * X, 6 * X)


def test_mxfp4_round_trip_of_representable_values_and_nibble_order():
    rng = np.random.default_rng(12)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    vals = rng.choice(mags, size=(3, 96)) * rng.choice([-1.0, 1.0], size=(3, 96))
    vals[:, ::32] = 6.0                              # every block's amax is 6 -> exponent 0
    scale = np.exp2(rng.integers(-20, 20, size=(3, 3)))
    x = vals * np.repeat(scale, 32, axis=1)
    p = O.mxfp4_payload(x)
    assert p.shape == (3, 96 // 2 + 96 // 32)
    assert np.array_equal(O.mxfp4_unpack(p, 96), x)
    # element 2i in the low nibble of byte i, 2i+1 in the high nibble
    row = np.zeros((1, 32))
    row[0, 0], row[0, 1], row[0, 2] = 1.0, 6.0, -0.5
    p = O.mxfp4_payload(row)
    assert p[0, 0] == 0x72 and p[0, 1] == 0x09 and p[0, 16] == 127


def test_fp8_block_payload_layout_and_unpack_bound():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((4, 256)) * 3).astype(np.float32)
    p = O.fp8_block_payload(x)
    codes, sc = O.quant_rows(x, 128)
    assert p.shape == (4, 256 + 8)
    assert np.array_equal(p[:, :256], codes)
    assert np.array_equal(np.ascontiguousarray(p[:, 256:]).view("<f4"), sc)
    y = O.fp8_block_unpack(p, 256)
    # e4m3 keeps 3 mantissa bits: relative error <= 2^-4, plus the bf16 rounding
    big = np.abs(x) > 0.1 * np.repeat(sc, 128, axis=1) * 448
    assert np.all(np.abs(y - x)[big] <= (2.0 ** -4 + 2.0 ** -8) * np.abs(x)[big])


def test_payload_bytes_match_the_page():
    pins = _pins()
    D = pins["r1_hidden"]
    b = O.ep_payload_bytes(D)
    assert 2 * b["bf16"] == pins["bf16_round_trip_bytes"]
    assert b["mxfp4"] + b["fp8_block"] == pins["quantized_round_trip_bytes"]
    assert b["fp8_block"] == D + 4 * pins["r1_scale_dim"]
    x = np.ones((1, D))
    assert O.mxfp4_payload(x).shape[1] == b["mxfp4"] and O.fp8_block_payload(x).shape[1] == b["fp8_block"]
