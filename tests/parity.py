"""Comparison rules between the HIP path and the oracle.

Exact paths (no rotation, no normalisation): every code, scale and value bit-identical.

Rotated or normalised paths: the GPU evaluates the rotation / RMSNorm in fp32, the
oracle in float64.  fp32 intermediates must agree to 1e-5 of their block's largest
magnitude.  A discrete decision (E2M1 magnitude, E4M3 or E8M0 scale, sign of a value
that rounds to zero) may differ by one step only where the oracle's real-valued argument
lies within 1e-5 (relative) of that decision's boundary; later decisions are checked
given the GPU's earlier ones (the oracle is re-run with the GPU's scales).
"""
import numpy as np

from oracle import formats as F

TOL = 1e-5


def blockwise_max(ref, block):
    r = np.abs(np.asarray(ref, dtype=np.float64))
    k = r.shape[-1]
    m = r.reshape(r.shape[:-1] + (k // block, block)).max(axis=-1)
    return np.repeat(m, block, axis=-1)


def assert_values_close(gpu, ref, block, tol=TOL, what="values"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = tol * blockwise_max(ref, block)
    bad = np.abs(gpu - ref) > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond {tol} x block max; first at "
                           f"{np.argwhere(bad)[0]}: gpu={gpu[bad][0]!r} ref={ref[bad][0]!r}")


def check_e2m1_codes(gpu, ref, ref_arg, ref_value, block, tol=TOL, what="codes"):
    """Codes may differ by one magnitude step only at a rounding midpoint, and in sign only
    where both round to zero from a value that is ~0 relative to its block."""
    gpu = np.asarray(gpu, dtype=np.int64)
    ref = np.asarray(ref, dtype=np.int64)
    mg, mr = gpu & 7, ref & 7
    near_mid = F.e2m1_boundary_distance(ref_arg) <= tol
    ok_mag = (mg == mr) | ((np.abs(mg - mr) == 1) & near_mid)
    tiny = np.abs(np.asarray(ref_value, dtype=np.float64)) <= tol * blockwise_max(ref_value, block)
    ok_sign = ((gpu & 8) == (ref & 8)) | ((mg == 0) & (mr == 0) & tiny)
    ok = ok_mag & ok_sign
    assert ok.all(), (f"{what}: {np.sum(~ok)} decisions differ away from a boundary; first at "
                      f"{np.argwhere(~ok)[0]}: gpu={gpu[~ok][0]} ref={ref[~ok][0]} "
                      f"arg={np.asarray(ref_arg)[~ok][0]!r}")
    return int(np.sum(gpu != ref))


def check_e4m3_scales(gpu, ref, ref_arg, tol=TOL, what="E4M3 scales"):
    gpu = np.asarray(gpu, dtype=np.int64)
    ref = np.asarray(ref, dtype=np.int64)
    near = F.e4m3_boundary_distance(ref_arg) <= tol
    ok = (gpu == ref) | ((np.abs(gpu - ref) == 1) & near)
    assert ok.all(), (f"{what}: {np.sum(~ok)} differ away from a midpoint; first at "
                      f"{np.argwhere(~ok)[0]}: gpu={gpu[~ok][0]} ref={ref[~ok][0]} "
                      f"arg={np.asarray(ref_arg)[~ok][0]!r}")
    return int(np.sum(gpu != ref))


def e8m0_boundary_distance(amax):
    """Relative distance |amax - 2^k| / 2^k of a block maximum to the nearest power of two:
    the E8M0 code floor(log2 amax) - 2 changes only where amax crosses one.  With
    amax = f 2^E (f in [0.5, 1), exact from frexp) the candidates are 2^(E-1), at 2f - 1,
    and 2^E, at 1 - f; both differences are exact in float64.  An all-zero block
    (amax = 0) has no neighbouring decision: inf."""
    a = np.asarray(amax, dtype=np.float64)
    f, _ = np.frexp(a)
    return np.where(a > 0, np.minimum(2.0 * f - 1.0, 1.0 - f), np.inf)


def check_e8m0_scales(gpu, ref, ref_amax, tol=TOL, what="E8M0 scales"):
    gpu = np.asarray(gpu, dtype=np.int64)
    ref = np.asarray(ref, dtype=np.int64)
    near = e8m0_boundary_distance(ref_amax) <= tol
    ok = (gpu == ref) | ((np.abs(gpu - ref) == 1) & near)
    assert ok.all(), (f"{what}: {np.sum(~ok)} differ away from a power of two; first at "
                      f"{np.argwhere(~ok)[0]}: gpu={gpu[~ok][0]} ref={ref[~ok][0]}")
    return int(np.sum(gpu != ref))


def assert_rel(gpu, ref, tol=TOL, what="scale"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bad = np.abs(gpu - ref) > tol * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} beyond {tol} relative; gpu={gpu[bad][:3]} ref={ref[bad][:3]}"


def assert_bf16_close(gpu_bf16_values, ref, block, tol=TOL, what="bf16 output"):
    """One bf16 rounding (2^-8 relative) of a value within tol x block max of the oracle."""
    g = np.asarray(gpu_bf16_values, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    bound = 2.0 ** -8 * np.abs(r) + tol * blockwise_max(r, block)
    bad = np.abs(g - r) > bound
    assert not bad.any(), (f"{what}: {bad.sum()} beyond one bf16 rounding; first at {np.argwhere(bad)[0]}:"
                           f" gpu={g[bad][0]!r} ref={r[bad][0]!r}")
