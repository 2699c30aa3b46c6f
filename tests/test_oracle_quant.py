"""Pins of the oracle's quantizers against an exact rational brute force (tests/exact_ref.py),
closed forms and invariants that fix the method independently of the oracle's code."""
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import arcquant, dualscale, formats as F, gemm, hadamard as H, mxfp4, nvfp4
from tests import exact_ref as X


def _fr_rows(a):
    return [[Fr(float(v)) for v in row] for row in np.asarray(a, dtype=np.float64)]


def _nvfp4_tie_tensor():
    """A tensor whose tensor scale is exactly 2^-8 and whose blocks hit E4M3 values,
    E4M3 midpoints and every E2M1 midpoint exactly (plus their binary32 neighbours)."""
    s_t = 2.0 ** -8
    rows = []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for sb in [1.125, 1.0625, 0.5, 3.0, 2.0 ** -7]:     # E4M3 values and a midpoint (1.0625)
        S = sb * s_t
        blk = []
        for m in mids:
            v = np.float32(m * S)
            blk += [v, np.nextafter(v, np.float32(0)), np.nextafter(v, np.float32(1))]
        blk = blk[:15] + [np.float32(6 * S)]             # block max -> scale argument = sb
        rows.append(blk + [-v for v in blk])
    x = np.array(rows, dtype=np.float32)
    x[0, 0] = np.float32(2688 * s_t)                      # tensor max -> s_t = 2^-8
    return x


@pytest.mark.parametrize("case", ["random", "ties", "wide"])
def test_nvfp4_against_exact_bruteforce(case):
    rng = np.random.default_rng(11)
    if case == "random":
        x = rng.standard_normal((4, 64)).astype(np.float32)
    elif case == "ties":
        x = _nvfp4_tie_tensor()
    else:  # blocks spanning many binades, including subnormal-scale blocks
        x = (rng.standard_normal((4, 64)) * np.exp(rng.uniform(-25, 5, (4, 64)))).astype(np.float32)
        x[1, 16:32] = 0.0
    r = nvfp4.quantize(x)
    s_t, codes, scales = X.nvfp4_tensor(_fr_rows(x))
    assert Fr(float(r["tensor_scale"])) == s_t
    assert r["scales"].tolist() == scales
    assert r["codes"].tolist() == codes
    assert np.array_equal(F.unpack_nibbles(r["packed"]), r["codes"])


def test_nvfp4_tie_tensor_really_has_ties():
    r = nvfp4.quantize(_nvfp4_tie_tensor())
    assert float(r["tensor_scale"]) == 2.0 ** -8
    mids = (F.E2M1_MAGNITUDES[:-1] + F.E2M1_MAGNITUDES[1:]) / 2
    assert np.isin(np.abs(r["elem_arg"]), mids).sum() >= 30
    assert 1.0625 in r["scale_arg"]                       # an E4M3 midpoint -> even code
    assert F.e4m3_decode(r["scales"][1, 0]) == 1.0


def test_nvfp4_given_tensor_scale_and_dequant():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    r = nvfp4.quantize(x, tensor_scale_value=np.float32(0.01))
    s_t, codes, scales = X.nvfp4_tensor(_fr_rows(x), Fr(float(np.float32(0.01))))
    assert r["codes"].tolist() == codes and r["scales"].tolist() == scales
    deq = nvfp4.dequantize(r["packed"], r["scales"], r["tensor_scale"])
    for i in range(4):
        for j in range(64):
            want = X.f32(X.e2m1_value(codes[i][j]) * X.E4M3[scales[i][j // 16]] * s_t)
            assert Fr(float(deq[i, j])) == want


def test_nvfp4_power_of_two_invariance():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    a = nvfp4.quantize(x)
    for k in (-6, 7):
        b = nvfp4.quantize(x * np.float32(2.0 ** k))
        assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])
        assert float(b["tensor_scale"]) == float(a["tensor_scale"]) * 2.0 ** k


def test_nvfp4_idempotent_and_error_bound():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    a = nvfp4.quantize(x)
    xq = nvfp4.dequantize(a["packed"], a["scales"], a["tensor_scale"])
    b = nvfp4.quantize(xq, tensor_scale_value=a["tensor_scale"], block_scales=a["scales"])
    assert np.array_equal(a["codes"], b["codes"])
    S = np.repeat(F.e4m3_decode(a["scales"]) * float(a["tensor_scale"]), 16, axis=1)
    u = np.abs(x) / S
    gap = np.where(u < 2, 0.5, np.where(u < 4, 1.0, 2.0))
    ok = u <= 6
    assert np.all(np.abs(x - xq)[ok] <= (gap * S / 2)[ok] * (1 + 1e-6))


def test_nvfp4_rotated_equals_rotate_then_quantize():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((4, 64))
    a = nvfp4.quantize(x, hadamard=16)
    b = nvfp4.quantize(H.block_rotate(x, 16))
    assert np.array_equal(a["codes"], b["codes"]) and a["tensor_scale"] == b["tensor_scale"]
    deq = nvfp4.dequantize(a["packed"], a["scales"], a["tensor_scale"], inverse_hadamard=16)
    assert np.max(np.abs(deq - x)) < 0.5                  # rotation undone


def test_nvfp4_all_zero_and_signs():
    x = np.zeros((2, 32), np.float32)
    x[1, 3] = -0.0
    r = nvfp4.quantize(x)
    assert float(r["tensor_scale"]) == 0.0 and not r["scales"].any()
    assert r["codes"][1, 3] == 8 and r["codes"].sum() == 8


# ----------------------------------------------------------------------------- MXFP4

def _mx_tie_rows():
    rows = []
    for e in (-3, 0, 2, -20):
        X_ = 2.0 ** e
        blk = [m * X_ for m in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)]
        blk += [np.nextafter(v, 0) for v in blk] + [np.nextafter(v, 10) for v in blk]
        blk += [7.9 * X_, 6.5 * X_, 4 * X_, -5.0 * X_]    # saturation, exact max
        blk += [0.0] * (32 - len(blk))
        rows.append(np.array(blk[:32], dtype=np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("case", ["random", "ties"])
def test_mxfp4_against_exact_bruteforce(case):
    rng = np.random.default_rng(21)
    if case == "random":
        x = (rng.standard_normal((4, 96)) * np.exp(rng.uniform(-8, 8, (4, 96)))).astype(np.float32)
    else:
        x = _mx_tie_rows()
    r = mxfp4.quantize(x)
    for i, row in enumerate(_fr_rows(x)):
        for b in range(0, len(row), 32):
            e, codes = X.mxfp4_block_codes(row[b:b + 32])
            assert r["scales"][i, b // 32] == e
            assert r["codes"][i, b:b + 32].tolist() == codes


def test_mxfp4_power_of_two_invariance_and_exact_dequant():
    rng = np.random.default_rng(22)
    x = rng.standard_normal((8, 128))
    a = mxfp4.quantize(x)
    b = mxfp4.quantize(x * 2.0 ** 9)
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(b["scales"].astype(int), a["scales"].astype(int) + 9)
    deq = mxfp4.dequantize(a["packed"], a["scales"])
    X_ = np.repeat(F.e8m0_decode(a["scales"]), 32, axis=1)
    assert np.all(np.abs(deq) <= 6 * X_)
    assert np.array_equal(deq / X_, F.e2m1_decode(a["codes"]))


def test_mxfp4_rotation_applied_before_quantization():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((4, 64))
    x[:, 5] *= 50                                          # an outlier channel
    a = mxfp4.quantize(x, hadamard=32)
    b = mxfp4.quantize(H.block_rotate(x, 32))
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])
    # the inverse rotation maps the quantization error back unchanged in norm
    err_back = np.linalg.norm(mxfp4.dequantize(a["packed"], a["scales"], 32) - x)
    err_rot = np.linalg.norm(mxfp4.dequantize(a["packed"], a["scales"]) - a["y"])
    assert abs(err_back - err_rot) < 1e-9 * err_rot


def test_two_level_128_rotation_before_nvfp4_and_mxfp4():
    """hadamard=128 quantizes scipy's H_128 of every 128-group (the two-level 16 x 8
    transform equals it), and the inverse rotation on dequantization maps back."""
    import scipy.linalg
    rng = np.random.default_rng(24)
    x = rng.standard_t(4, (3, 384))
    h = scipy.linalg.hadamard(128) / np.sqrt(128.0)
    xr = (x.reshape(3, 3, 128) @ h.T).reshape(3, 384)
    a, b = nvfp4.quantize(x, hadamard=128), nvfp4.quantize(xr)
    assert np.allclose(a["y"], xr, rtol=0, atol=1e-13)
    assert np.array_equal(a["scales"], b["scales"])
    assert np.mean(a["codes"] == b["codes"]) > 0.999          # a few ulp of y may cross a midpoint
    m = mxfp4.quantize(x, hadamard=128)
    back = mxfp4.dequantize(m["packed"], m["scales"], inverse_hadamard=128)
    err_back = np.linalg.norm(back - x)
    err_rot = np.linalg.norm(mxfp4.dequantize(m["packed"], m["scales"]) - m["y"])
    assert abs(err_back - err_rot) < 1e-9 * err_rot
    d = nvfp4.dequantize(a["packed"], a["scales"], a["tensor_scale"], inverse_hadamard=128)
    assert np.allclose(d, (nvfp4.dequantize(a["packed"], a["scales"], a["tensor_scale"]).reshape(3, 3, 128)
                           @ h.T).reshape(3, 384), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- dual scale

def test_dualscale_quantization_against_exact_bruteforce():
    rng = np.random.default_rng(31)
    x = rng.standard_t(4, (2, 256))
    r = dualscale.pack_values(x)
    y = r["y"]
    # pin the rotation independently of the oracle: H_128 by scipy's construction
    import scipy.linalg
    h = scipy.linalg.hadamard(128) / np.sqrt(128)
    assert np.allclose(y, (x.reshape(2, 2, 128) @ h.T).reshape(2, 256), atol=1e-13)
    for i in range(2):
        for g in range(2):
            grp = [Fr(float(v)) for v in y[i, 128 * g:128 * g + 128]]
            s_g = X.f32(max(abs(v) for v in grp) / 2688)
            assert Fr(float(r["group_scales"][i, g])) == s_g
            for m in range(8):
                sb, codes = X.nvfp4_block_codes(grp[16 * m:16 * m + 16], s_g)
                assert r["micro_scales"][i, 8 * g + m] == sb
                assert r["codes"][i, 128 * g + 16 * m:128 * g + 16 * m + 16].tolist() == codes


def test_dualscale_layout_and_roundtrip():
    M, K = 3, 384
    lay = dualscale.layout(M, K)
    assert lay["micro_scales"] % 256 == 0 and lay["group_scales"] % 256 == 0
    assert lay["micro_scales"] >= M * K // 2 and lay["group_scales"] >= lay["micro_scales"] + M * K // 16
    assert lay["total"] >= lay["group_scales"] + 4 * M * K // 128
    rng = np.random.default_rng(32)
    x = rng.standard_t(4, (M, K))
    buf = dualscale.pack(x)
    assert buf.size == lay["total"]
    codes, sm, sg = dualscale.split(buf, M, K)
    r = dualscale.pack_values(x)
    assert np.array_equal(codes, r["codes"]) and np.array_equal(sm, r["micro_scales"])
    assert np.array_equal(sg, r["group_scales"])
    y = dualscale.unpack(buf, M, K)
    # reconstruction error is the rotated quantization error (rotation is orthonormal)
    err_rot = np.linalg.norm(y - x)
    err_q = np.linalg.norm(dualscale.dequantized(codes, sm, sg) - r["y"])
    assert abs(err_rot - err_q) < 1e-9 * max(1.0, err_q)
    assert err_rot / np.linalg.norm(x) < 0.2


# ----------------------------------------------------------------------------- ARCQuant

def _arc_case(seed=41, M=4, K=128, S=32):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    x[:, [7, 90]] *= 30
    x = x.astype(np.float32).astype(np.float64)
    perm = np.argsort(-np.abs(x).max(axis=0), kind="stable")
    return x, perm, S


def test_arcquant_rmsnorm_closed_form():
    rng = np.random.default_rng(40)
    x = rng.standard_normal((5, 64))
    y = arcquant.rmsnorm(x, eps=1e-6)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + 1e-6), rtol=1e-14)
    assert np.allclose(y * np.sqrt(ms + 1e-6)[:, None], x, rtol=1e-14)


def test_arcquant_quantization_against_exact_bruteforce():
    x, perm, S = _arc_case()
    r = arcquant.quantize(x, perm, S)
    z = r["z"]
    assert np.array_equal(z, arcquant.rmsnorm(x)[:, perm])
    s_t, codes, scales = X.nvfp4_tensor(_fr_rows(z))
    assert Fr(float(r["tensor_scale"])) == s_t
    assert r["primary"]["codes"].tolist() == codes and r["primary"]["scales"].tolist() == scales
    for i in range(z.shape[0]):
        res = []
        for j in range(S):
            xhat = X.e2m1_value(codes[i][j]) * X.E4M3[scales[i][j // 16]] * s_t
            res.append(Fr(float(z[i, j])) - xhat)
        # the float64 residual is rounded once; check it, then quantize the exact one
        assert np.allclose(r["residual_value"][i], [float(v) for v in res], rtol=0, atol=1e-15)
        _, rc, rs = X.nvfp4_tensor([res], s_t)
        assert r["residual"]["codes"][i].tolist() == rc[0]
        assert r["residual"]["scales"][i].tolist() == rs[0]
    K = x.shape[1]
    assert r["codes"].shape == (x.shape[0], K + S) and r["scales"].shape == (x.shape[0], (K + S) // 16)


def test_arcquant_residual_reduces_error_elementwise():
    x, perm, S = _arc_case(seed=42, M=16, K=256, S=64)
    r = arcquant.quantize(x, perm, S)
    p, rr = arcquant.dequantize(r["packed"], r["scales"], r["tensor_scale"], 256, S)
    e1 = np.abs(r["z"][:, :S] - p[:, :S])
    e2 = np.abs(r["z"][:, :S] - p[:, :S] - rr)
    assert np.all(e2 <= e1 + 1e-12)
    assert e2.sum() < 0.5 * e1.sum()


def test_arcquant_augmented_gemm_linearity():
    # [P | R] . [W | W_S]^T == P W^T + R W_S^T: the K+S extended reduction
    x, perm, S = _arc_case(seed=43, M=8, K=128, S=32)
    r = arcquant.quantize(x, perm, S)
    p, rr = arcquant.dequantize(r["packed"], r["scales"], r["tensor_scale"], 128, S)
    rng = np.random.default_rng(44)
    w = rng.standard_normal((6, 128))                      # weights in the reordered order
    ext_a = np.concatenate([p, rr], axis=1)
    ext_w = np.concatenate([w, w[:, :S]], axis=1)          # duplicated weight columns
    assert np.allclose(ext_a @ ext_w.T, p @ w.T + rr @ w[:, :S].T, rtol=1e-12, atol=1e-12)
    # and the residual moves the product towards the unquantized one
    exact = r["z"] @ w.T
    assert np.linalg.norm(ext_a @ ext_w.T - exact) < np.linalg.norm(p @ w.T - exact)


def test_arcquant_zero_residual_channels_and_identity_perm():
    x, _, _ = _arc_case(seed=45)
    r0 = arcquant.quantize(x, np.arange(128), 0)
    n = nvfp4.quantize(arcquant.rmsnorm(x))
    assert np.array_equal(r0["codes"], n["codes"]) and np.array_equal(r0["scales"], n["scales"])


def test_arcquant_z_override_is_the_same_steps():
    """Given its own normalized, reordered values, the oracle reproduces its default result
    exactly (both flavours); given other values, those are what the residual is taken
    from (the parity checks condition the residual on the GPU's z this way)."""
    x, perm, S = _arc_case(seed=46, M=6, K=256, S=64)
    g = np.random.default_rng(47).uniform(-1.5, 1.5, 256)
    z = arcquant.rmsnorm(x, g, 1e-6)[:, perm]
    for fn in (arcquant.quantize, arcquant.quantize_mx):
        a = fn(x, perm, S, g, 1e-6)
        b = fn(x, perm, S, g, 1e-6, z=z)
        for key in ("codes", "scales", "z", "residual_value"):
            assert np.array_equal(a[key], b[key]), (fn.__name__, key)
        zp = z * (1 + 2.0 ** -20)
        c = fn(x, perm, S, g, 1e-6, primary_scales=a["primary"]["scales"], primary_codes=a["primary"]["codes"], z=zp)
        assert np.array_equal(c["z"], zp)
        assert not np.array_equal(c["residual_value"], a["residual_value"])


def test_arcquant_mx_against_exact_bruteforce():
    """MXFP4 flavour: E8M0 per 32 on z, residual against the exact primary value."""
    x, perm, S = _arc_case(seed=46, M=3, K=128, S=64)
    r = arcquant.quantize_mx(x, perm, S)
    z = r["z"]
    assert np.array_equal(z, arcquant.rmsnorm(x)[:, perm])
    for i in range(z.shape[0]):
        zr = [Fr(float(v)) for v in z[i]]
        pcodes, pscales = [], []
        for b in range(0, 128, 32):
            e, c = X.mxfp4_block_codes(zr[b:b + 32])
            pscales.append(e)
            pcodes += c
        assert r["primary"]["codes"][i].tolist() == pcodes
        assert r["primary"]["scales"][i].tolist() == pscales
        res = [zr[j] - X.e2m1_value(pcodes[j]) * Fr(2) ** (pscales[j // 32] - 127) for j in range(S)]
        assert np.allclose(r["residual_value"][i], [float(v) for v in res], rtol=0, atol=1e-15)
        rcodes, rscales = [], []
        for b in range(0, S, 32):
            e, c = X.mxfp4_block_codes(res[b:b + 32])
            rscales.append(e)
            rcodes += c
        assert r["residual"]["codes"][i].tolist() == rcodes
        assert r["residual"]["scales"][i].tolist() == rscales
    assert r["codes"].shape == (3, 128 + S) and r["scales"].shape == (3, (128 + S) // 32)


def test_arcquant_mx_residual_reduces_error_and_gemm_linearity():
    x, perm, S = _arc_case(seed=47, M=16, K=256, S=64)
    r = arcquant.quantize_mx(x, perm, S)
    p, rr = arcquant.dequantize_mx(r["packed"], r["scales"], 256, S)
    e1 = np.abs(r["z"][:, :S] - p[:, :S])
    e2 = np.abs(r["z"][:, :S] - p[:, :S] - rr)
    assert np.all(e2 <= e1 + 1e-12)            # 0 is a grid point; saturation stays below |r|
    assert e2.sum() < 0.5 * e1.sum()
    w = np.random.default_rng(48).standard_normal((5, 256))
    ext = np.concatenate([p, rr], axis=1) @ np.concatenate([w, w[:, :S]], axis=1).T
    assert np.allclose(ext, p @ w.T + rr @ w[:, :S].T, rtol=1e-12, atol=1e-12)
    exact = r["z"] @ w.T
    assert np.linalg.norm(ext - exact) < np.linalg.norm(p @ w.T - exact)


def test_arcquant_mx_without_residual_is_plain_mxfp4():
    x, _, _ = _arc_case(seed=49)
    r0 = arcquant.quantize_mx(x, np.arange(128), 0)
    m = mxfp4.quantize(arcquant.rmsnorm(x))
    assert np.array_equal(r0["codes"], m["codes"]) and np.array_equal(r0["scales"], m["scales"])


# ----------------------------------------------------------------------------- GEMM

def test_gemm_against_exact_bruteforce():
    rng = np.random.default_rng(51)
    M, N, K = 3, 4, 64
    a_p = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    b_p = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    a_s = rng.integers(120, 130, (M, K // 32), dtype=np.uint8)
    b_s = rng.integers(120, 130, (N, K // 32), dtype=np.uint8)
    c = gemm.full(a_p, a_s, b_p, b_s)
    for m in range(M):
        for n in range(N):
            acc = Fr(0)
            for k in range(K):
                ca = (a_p[m, k // 2] >> (4 * (k % 2))) & 15
                cb = (b_p[n, k // 2] >> (4 * (k % 2))) & 15
                acc += (X.e2m1_value(ca) * Fr(2) ** (int(a_s[m, k // 32]) - 127)
                        * X.e2m1_value(cb) * Fr(2) ** (int(b_s[n, k // 32]) - 127))
            assert c[m, n] == float(acc)                  # exact: few terms, short values
    t = gemm.tile(a_p, a_s, b_p, b_s, [2, 0], [3, 1])
    assert np.array_equal(t, c[[2, 0]][:, [3, 1]])


def test_rotation_cancels_in_the_product():
    rng = np.random.default_rng(52)
    x = rng.standard_normal((4, 64))
    w = rng.standard_normal((5, 64))
    xr, wr = H.block_rotate(x, 32), H.block_rotate(w, 32)
    assert np.allclose(xr @ wr.T, x @ w.T, rtol=1e-12, atol=1e-12)
