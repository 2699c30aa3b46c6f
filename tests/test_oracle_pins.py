"""Pins of the oracle parts that the other CPU tests leave open, and of the tolerance
helpers that decide which GPU decisions the rotated-path comparisons accept.

* RMSNorm with a gain vector: exact rational brute force (squares and the mean in
  Fractions) showing that gamma scales input channel perm[c] before the reorder
  (ARCQuant summary, Méthodologie item 5: one kernel does the reorder and the norm).
* Dual-scale dequantization: fl32(V * s_m * s_g) element by element against exact
  rational rounding, and the unpack's rotation against scipy's H_128 (FP4Quant abstract:
  dual-scale micro-groups, two-level FWHT).
* Boundary distances of the E2M1, E4M3 and E8M0 decisions: hand values at each midpoint
  or power of two, one ulp either side and just inside / outside the 1e-5 band, plus the
  accept / reject behaviour of the checkers on planted differences.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest
import scipy.linalg

from oracle import arcquant, dualscale, formats as F
from tests import exact_ref as X
from tests import parity as P


# ----------------------------------------------------------------------------- RMSNorm gain

def _gamma_case(seed=60, M=3, K=64):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32).astype(np.float64)
    gamma = rng.standard_normal(K).astype(np.float32)
    gamma[[3, 17, 40]] = 0.0                       # zero gains
    assert (gamma < 0).sum() > 10                  # and plenty of negative ones
    perm = rng.permutation(K)
    return x, gamma, perm


def test_rmsnorm_gain_applied_per_input_channel_before_reorder():
    x, gamma, perm = _gamma_case()
    M, K = x.shape
    eps = 1e-6
    r = arcquant.quantize(x, perm, 16, gamma=gamma, eps=eps)
    z = r["z"]
    for i in range(M):
        ms = sum(Fr(float(v)) ** 2 for v in x[i]) / K + Fr(eps)       # exact mean(x^2) + eps
        for c in range(K):
            j = int(perm[c])
            num = Fr(float(x[i, j])) * Fr(float(gamma[j]))           # x gamma of input channel j
            got = Fr(float(z[i, c]))
            if num == 0:
                assert got == 0, (i, c)
                continue
            assert (got > 0) == (num > 0), (i, c)
            want_sq = num * num / ms                                   # z^2 exactly
            assert abs(got * got - want_sq) <= Fr(1, 10 ** 13) * want_sq, (i, c)
    # the reading is distinguishable: gamma taken in output order gives other values
    wrong = arcquant.rmsnorm(x)[:, perm] * gamma.astype(np.float64)
    assert np.max(np.abs(wrong - z)) > 0.1


def test_rmsnorm_gain_mx_flavour_and_unit_gain():
    x, gamma, perm = _gamma_case(seed=61, K=128)
    a = arcquant.quantize(x, perm, 32, gamma=gamma)
    b = arcquant.quantize_mx(x, perm, 32, gamma=gamma)
    assert np.array_equal(a["z"], b["z"])
    one = arcquant.quantize(x, perm, 32, gamma=np.ones(128, np.float32))
    none = arcquant.quantize(x, perm, 32)
    assert np.array_equal(one["z"], none["z"]) and np.array_equal(one["codes"], none["codes"])


# ----------------------------------------------------------------------------- dual scale

def _dual_case(seed=70, M=2, K=256):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, (M, K)).astype(np.uint8)
    sm = rng.integers(0, 127, (M, K // 16)).astype(np.uint8)           # every finite E4M3 code range
    sm[0, :4] = [0, 1, 7, 126]                                          # zero, subnormals, 448
    sg = (rng.standard_normal((M, K // 128)) ** 2 * np.exp(rng.uniform(-30, 2, (M, K // 128))))
    sg = sg.astype(np.float32)
    sg[-1, -1] = np.float32(2.0 ** -135)                                # subnormal products
    return codes, sm, sg


def test_dualscale_dequantized_is_one_binary32_rounding():
    codes, sm, sg = _dual_case()
    M, K = codes.shape
    d = dualscale.dequantized(codes, sm, sg)
    for i in range(M):
        for k in range(K):
            v = X.e2m1_value(int(codes[i, k])) * X.E4M3[int(sm[i, k // 16])] * Fr(float(sg[i, k // 128]))
            assert Fr(float(d[i, k])) == X.f32(v), (i, k)


def test_dualscale_unpack_is_h128_of_the_dequantized_values():
    codes, sm, sg = _dual_case(seed=71, M=3, K=384)
    M, K = codes.shape
    # the message laid out by the header's formula, independently of dualscale.layout
    a256 = lambda n: (n + 255) // 256 * 256                             # noqa: E731
    off_m = a256(M * K // 2)
    off_g = a256(off_m + M * K // 16)
    buf = np.zeros(a256(off_g + 4 * M * K // 128), np.uint8)
    buf[:M * K // 2] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).reshape(-1)
    buf[off_m:off_m + M * K // 16] = sm.reshape(-1)
    buf[off_g:off_g + 4 * M * K // 128] = sg.astype("<f4").reshape(-1).view(np.uint8)
    y = dualscale.unpack(buf, M, K)
    h = scipy.linalg.hadamard(128) / np.sqrt(128.0)
    want = (dualscale.dequantized(codes, sm, sg).reshape(M, K // 128, 128) @ h.T).reshape(M, K)
    assert np.allclose(y, want, rtol=0, atol=1e-12 * np.max(np.abs(want)))
    # the micro and group scales sit at their own positions: moving a group scale by one
    # group moves exactly that group's values
    sg2 = sg.copy()
    sg2[0, 1] *= 2
    d1, d2 = dualscale.dequantized(codes, sm, sg), dualscale.dequantized(codes, sm, sg2)
    changed = np.nonzero(np.any(d1 != d2, axis=0))[0]
    assert changed.min() >= 128 and changed.max() < 256


# ----------------------------------------------------------------------------- boundaries

E2M1_MIDS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def test_e2m1_boundary_distance_hand_values():
    for m in E2M1_MIDS:
        assert F.e2m1_boundary_distance(m) == 0.0
        assert F.e2m1_boundary_distance(-m) == 0.0
        for nb in (np.nextafter(m, 0.0), np.nextafter(m, 10.0)):
            d = F.e2m1_boundary_distance(nb)
            assert 0.0 < d < 1e-15
        assert F.e2m1_boundary_distance(m * (1 + 0.9e-5)) <= 1e-5
        assert F.e2m1_boundary_distance(m * (1 - 0.9e-5)) <= 1e-5
        assert F.e2m1_boundary_distance(m * (1 + 1.1e-5)) > 1e-5
        assert F.e2m1_boundary_distance(m * (1 - 1.1e-5)) > 1e-5
    # grid points sit between two midpoints: 0.5 -> |0.5 - 0.75| / 0.75 = 1/3
    assert F.e2m1_boundary_distance(0.5) == pytest.approx(1 / 3, rel=1e-15)
    assert F.e2m1_boundary_distance(1.0) == pytest.approx(0.2, rel=1e-15)    # 1.25
    assert F.e2m1_boundary_distance(6.0) == pytest.approx(0.2, rel=1e-15)    # 5
    assert F.e2m1_boundary_distance(0.0) == 1.0
    assert F.e2m1_boundary_distance(100.0) == pytest.approx(19.0, rel=1e-15)  # saturated: far


def _e4m3_mids():
    v = np.array([float(e) for e in X.E4M3])
    return (v[:-1] + v[1:]) / 2


def test_e4m3_boundary_distance_hand_values():
    for m in _e4m3_mids():
        assert F.e4m3_boundary_distance(m) == 0.0
        for nb in (np.nextafter(m, 0.0), np.nextafter(m, 1e3)):
            assert 0.0 < F.e4m3_boundary_distance(nb) < 1e-15
        assert F.e4m3_boundary_distance(m * (1 + 0.9e-5)) <= 1e-5
        assert F.e4m3_boundary_distance(m * (1 - 1.1e-5)) > 1e-5
    assert F.e4m3_boundary_distance(1.0) == pytest.approx(1 / 31, rel=1e-15)     # midpoint 0.96875
    assert F.e4m3_boundary_distance(2.0 ** -10) == 0.0                          # 0 | 2^-9
    assert F.e4m3_boundary_distance(432.0) == 0.0                               # 416 | 448
    assert F.e4m3_boundary_distance(440.0) == pytest.approx(8 / 432, rel=1e-15)
    assert F.e4m3_boundary_distance(448.5) == np.inf                            # saturated


def test_e8m0_boundary_distance_hand_values():
    for k in (-130, -20, -1, 0, 1, 7, 100):
        p = 2.0 ** k
        assert P.e8m0_boundary_distance(p) == 0.0
        for nb in (np.nextafter(p, 0.0), np.nextafter(p, np.inf)):
            assert 0.0 < P.e8m0_boundary_distance(nb) < 1e-15
        assert P.e8m0_boundary_distance(p * (1 + 0.9e-5)) <= 1e-5
        assert P.e8m0_boundary_distance(p * (1 - 0.9e-5)) <= 1e-5
        assert P.e8m0_boundary_distance(p * (1 + 1.1e-5)) > 1e-5
        assert P.e8m0_boundary_distance(p * (1 - 1.1e-5)) > 1e-5
    assert P.e8m0_boundary_distance(1.5) == 0.25                                   # |1.5 - 2| / 2
    assert P.e8m0_boundary_distance(1.25) == 0.25                                  # |1.25 - 1| / 1
    assert P.e8m0_boundary_distance(0.0) == np.inf                                   # zero block


def test_checkers_accept_only_boundary_flips():
    ref = np.array([[1, 2, 3, 0, 5]], np.int64)
    value = np.array([[0.5, 1.0, 1.5, 1e-9, 3.0]])
    arg = np.array([[0.5, 1.0, 1.5, 1e-9, 3.0]])
    # one step at a tie argument: accepted
    a2 = arg.copy(); a2[0, 1] = 1.25                                         # noqa: E702
    g = ref.copy(); g[0, 1] = 3                                              # noqa: E702
    assert P.check_e2m1_codes(g, ref, a2, value, 5) == 1
    # the same step away from the midpoint: rejected
    with pytest.raises(AssertionError):
        P.check_e2m1_codes(g, ref, arg, value, 5)
    # two steps at a midpoint: rejected
    g2 = ref.copy(); g2[0, 1] = 4                                            # noqa: E702
    with pytest.raises(AssertionError):
        P.check_e2m1_codes(g2, ref, a2, value, 5)
    # a sign flip of a code rounding to zero from a value ~0 of its block: accepted
    g3 = ref.copy(); g3[0, 3] = 8                                            # noqa: E702
    assert P.check_e2m1_codes(g3, ref, arg, value, 5) == 1
    # a sign flip of a nonzero code: rejected
    g4 = ref.copy(); g4[0, 0] = 9                                            # noqa: E702
    with pytest.raises(AssertionError):
        P.check_e2m1_codes(g4, ref, arg, value, 5)
    # E4M3: one code off at a midpoint only
    sref = np.array([56, 57])
    sarg = np.array([1.0625, 1.2])
    assert P.check_e4m3_scales(np.array([57, 57]), sref, sarg) == 1
    with pytest.raises(AssertionError):
        P.check_e4m3_scales(np.array([56, 58]), sref, sarg)
    # E8M0: one code off at a power of two only, never for a zero block
    eref = np.array([127, 127, 0])
    amax = np.array([4.0, 5.0, 0.0])
    assert P.check_e8m0_scales(np.array([126, 127, 0]), eref, amax) == 1
    with pytest.raises(AssertionError):
        P.check_e8m0_scales(np.array([127, 126, 0]), eref, amax)
    with pytest.raises(AssertionError):
        P.check_e8m0_scales(np.array([127, 127, 1]), eref, amax)
