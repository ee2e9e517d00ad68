"""Pins of the oracle's number formats against things other than itself:
the OCP e4m3fn code table, torch's CPU dtype casts and a brute-force
nearest-code search."""

import os

import numpy as np
import pytest
import torch

import oracle as O
from tests.conftest import GOLDEN


def _golden_codes():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3fn_codes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c, 16), float(v)))
    return rows


def test_e4m3_value_matches_spec_table():
    for code, val in _golden_codes():
        got = O.e4m3_value(np.array([code], np.uint8))[0]
        if np.isnan(val):
            assert np.isnan(got)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e4m3_value_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_value(np.arange(256, dtype=np.uint8))
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(got[~both_nan]))


def _dense_probe_set():
    """fp32 values around every code: the codes, the midpoints between
    neighbours, one fp32 ulp either side of each midpoint, subnormal range,
    saturation range and random magnitudes."""
    vals = O.e4m3_value(np.arange(0, 0x7F, dtype=np.uint8))       # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2.0
    m32 = mids.astype(np.float32)
    pts = [vals.astype(np.float32), m32,
           np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(0)),
           np.array([448.0, 449.0, 463.99, 464.0, 465.0, 480.0, 1e4, 3.0e38], np.float32),
           np.array([2.0 ** -10, 2.0 ** -11, 1e-30, 1e-45, 0.0], np.float32)]
    rng = np.random.default_rng(7)
    pts.append((np.exp(rng.uniform(np.log(1e-4), np.log(500.0), 20000))).astype(np.float32))
    p = np.concatenate(pts).astype(np.float32)
    return np.concatenate([p, -p])


def _brute_force_encode(x):
    """Nearest finite code by exhaustive search; ties go to the code with an
    even mantissa (its lowest bit 0); magnitudes above 448 saturate."""
    table = O.e4m3_value(np.arange(0, 0x7F, dtype=np.uint8))      # magnitudes of 0x00..0x7E
    out = []
    for v in x.astype(np.float64):
        a = min(abs(v), 448.0)
        d = np.abs(table - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
        if np.signbit(v):
            c |= 0x80
        out.append(c)
    return np.array(out, np.uint8)


def test_e4m3_encode_vs_brute_force():
    x = _dense_probe_set()
    assert np.array_equal(O.e4m3_encode(x), _brute_force_encode(x))


def test_e4m3_encode_vs_torch_cast_in_range():
    x = _dense_probe_set()
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), ref)


def test_e4m3_encode_never_nan_and_saturates():
    x = np.array([448.0, 500.0, 1e30, -1e30, -470.0], np.float32)
    c = O.e4m3_encode(x)
    assert list(c) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_e4m3_encode_signed_zero():
    c = O.e4m3_encode(np.array([0.0, -0.0, 1e-40, -1e-40], np.float32))
    assert list(c) == [0x00, 0x80, 0x00, 0x80]


def test_bf16_round_vs_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
        np.array([0.0, -0.0, 1.0, 3.0e38, -3.4e38, 1e-42, 65504.0], np.float32)]).astype(np.float32)
    # values whose low 16 bits are exactly 0x8000 exercise the tie-to-even rule
    ties = (rng.integers(0, 2 ** 31, 5000).astype(np.uint32) & np.uint32(0x7F7F0000)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = O.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(O.bf16_from_bits(O.bf16_bits(x)).view(np.uint32), ref.view(np.uint32))
