"""Pins of the oracle's format layer against definitions that do not come from the oracle:
hand-derived OCP tables, torch's float8 casts, numpy's half-to-even rounding and an
exact rational brute force."""
import os
from fractions import Fraction as Fr

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests import exact_ref as X

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ----------------------------------------------------------------------------- E2M1

def test_e2m1_decode_table_matches_golden():
    rows = _read_golden("e2m1_codes.txt")
    assert len(rows) == 16
    for code, value in rows:
        assert F.e2m1_decode(np.uint8(int(code, 0))) == float(value)


def test_e2m1_decode_matches_field_definition():
    for c in range(8):
        assert F.E2M1_MAGNITUDES[c] == F._e2m1_magnitude_from_bits(c)


def test_e2m1_midpoint_ties_golden():
    # every grid midpoint, both signs, goes to the even code (hand table from the
    # round-half-to-even rule of OCP MX v1.0)
    for value, code in _read_golden("e2m1_midpoints.txt"):
        v = float(value)
        assert F.e2m1_rne(np.float64(v)) == int(code, 0), value
        assert F.e2m1_rne(np.float64(-v)) == (int(code, 0) | 8), value


def _e2m1_by_numpy_round(a):
    """Textbook route: per binade the grid is uniform, so half-to-even rounding of a
    scaled value (numpy.round) gives the magnitude; then look the value up."""
    a = np.asarray(a, dtype=np.float64)
    v = np.where(a < 2, np.round(2 * a) / 2, np.where(a < 4, np.round(a), 2 * np.round(a / 2)))
    v = np.minimum(v, 6.0)
    return np.searchsorted(F.E2M1_MAGNITUDES, v).astype(np.uint8)


def test_e2m1_rne_against_numpy_half_even():
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.uniform(0, 9, 200000),
        np.arange(0, 9, 0.125),                              # all quarter/eighth points
        np.nextafter(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]), 0),
        np.nextafter(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]), 10),
        [0.0, 6.0, 6.5, 7.0, 1e30],
    ])
    assert np.array_equal(F.e2m1_rne(a), _e2m1_by_numpy_round(a))
    assert np.array_equal(F.e2m1_rne(-a) & 7, _e2m1_by_numpy_round(a))
    assert np.all(F.e2m1_rne(-a[a > 0]) & 8)


def test_e2m1_rne_against_exact_bruteforce():
    rng = np.random.default_rng(1)
    vals = rng.uniform(-7, 7, 2000)
    got = F.e2m1_rne(vals)
    for v, g in zip(vals, got):
        fr = Fr(float(v))
        want = (8 if v < 0 else 0) | X.nearest_even(X.E2M1, abs(fr))
        assert g == want, v


def test_e2m1_sign_of_zero():
    assert F.e2m1_rne(np.float64(-0.0)) == 8
    assert F.e2m1_rne(np.float64(0.0)) == 0
    assert F.e2m1_rne(np.float64(-0.1)) == 8


def test_nibble_packing_order():
    codes = np.array([[1, 2, 15, 0]], dtype=np.uint8)
    packed = F.pack_nibbles(codes)
    assert packed.tolist() == [[0x21, 0x0F]]            # element 2j in the low nibble
    assert np.array_equal(F.unpack_nibbles(packed), codes)


# ----------------------------------------------------------------------------- E4M3

def test_e4m3_decode_matches_torch():
    bits = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = bits.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert nan.sum() == 2                                 # 0x7F and 0xFF


def test_e4m3_specials_golden():
    for code, value in _read_golden("e4m3_values.txt"):
        assert F.e4m3_decode(np.uint8(int(code, 0))) == float(Fr(value))


def test_e4m3_rne_against_torch_cast():
    # torch's float8_e4m3fn cast is round-to-nearest-even; compare on binary32 inputs
    # (exact in both) up to the last midpoint below the NaN encoding (464).
    rng = np.random.default_rng(2)
    mids = (F.E4M3_FINITE[:-1] + F.E4M3_FINITE[1:]) / 2
    r = np.concatenate([
        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(464.0), 300000)),
        F.E4M3_FINITE, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
        np.nextafter(mids.astype(np.float32), np.float32(1000)), [0.0, 2.0 ** -10, 464.0],
    ]).astype(np.float32)
    ref = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_rne(r.astype(np.float64))
    assert np.array_equal(ref, got)


def test_e4m3_saturates():
    assert F.e4m3_rne(np.array([448.0, 460.0, 464.0, 500.0, 1e9])).tolist() == [126] * 5


def test_e4m3_against_exact_bruteforce():
    rng = np.random.default_rng(3)
    r = np.exp(rng.uniform(np.log(2.0 ** -11), np.log(500.0), 500))
    for v, g in zip(r, F.e4m3_rne(r)):
        assert g == X.nearest_even(X.E4M3, Fr(float(v)))


# ----------------------------------------------------------------------------- E8M0

def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = F.e8m0_decode(codes)
    nan = np.isnan(ref)
    assert nan.tolist() == [False] * 255 + [True]       # 0xFF is the format's NaN
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_e8m0_from_amax_golden():
    for amax, code in _read_golden("e8m0_from_amax.txt"):
        assert F.e8m0_from_amax(np.float64(float(Fr(amax)))) == int(code), amax


def test_e8m0_brackets_block_max():
    # defining property of X = 2^(floor(log2 amax) - 2): 4 X <= amax < 8 X
    rng = np.random.default_rng(4)
    amax = np.exp(rng.uniform(np.log(1e-30), np.log(1e30), 100000))
    X = F.e8m0_decode(F.e8m0_from_amax(amax))
    assert np.all(4 * X <= amax) and np.all(amax < 8 * X)


def test_e8m0_clamps_and_zero():
    assert F.e8m0_from_amax(np.float64(0.0)) == 0
    assert F.e8m0_from_amax(np.float64(2.0 ** -140)) == 0          # clamped at 2^-127
    assert F.e8m0_from_amax(np.float64(3.0e38)) == 127 + 125        # floor(log2) = 127


# ----------------------------------------------------------------------------- bf16

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f32_to_bf16_bits(v), ref)
    back = F.bf16_bits_to_f64(ref)
    assert np.array_equal(back, torch.from_numpy(v).to(torch.bfloat16).double().numpy())
