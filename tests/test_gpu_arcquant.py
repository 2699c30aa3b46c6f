"""GPU parity of the ARCQuant fused kernel (RMSNorm + reorder + primary / residual NVFP4)."""
import numpy as np
import pytest
import torch

import microscaled_fp4_quantization_block_amd as fp4
from microscaled_fp4_quantization_block_amd import workloads as W
from oracle import arcquant, formats as F
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return t.detach().cpu().numpy()


def _check_arc(xt, perm, S, gamma=None, eps=1e-6, rows=None, given=None):
    M, K = xt.shape
    x = xt.to(DEV)
    dbg = torch.empty((M, K), dtype=torch.float32, device=DEV)
    g = None if gamma is None else torch.from_numpy(gamma.astype(np.float32)).to(DEV)
    ts = None if given is None else torch.tensor([given], dtype=torch.float32, device=DEV)
    codes, scales, ts = fp4.fp4_residual_quantize(
        x, torch.from_numpy(perm.astype(np.int32)).to(DEV), S, gamma=g, eps=eps, tensor_scale=ts,
        mode="compute" if given is None else "given", dbg_normed=dbg)
    rows = np.arange(M) if rows is None else rows
    xv = W.values(xt)
    gam = None if gamma is None else gamma.astype(np.float32).astype(np.float64)
    gst = _np(ts)[0]
    if given is None:
        full = arcquant.rmsnorm(xv, gam, eps)
        P.assert_rel(gst, F.to_f32(np.max(np.abs(full)) / 2688.0), what="tensor scale")
    else:
        assert gst == np.float32(given)
    xr = xv[rows]
    gc = F.unpack_nibbles(_np(codes)[rows])
    gs = _np(scales)[rows]
    nb = K // 16
    base = arcquant.quantize(xr, perm, S, gam, eps, tensor_scale_value=gst)
    P.assert_values_close(_np(dbg)[rows], base["z"], K, what="normalized, reordered values")
    P.check_e4m3_scales(gs[:, :nb], base["primary"]["scales"], base["primary"]["scale_arg"], what="primary scales")
    c1 = arcquant.quantize(xr, perm, S, gam, eps, tensor_scale_value=gst, primary_scales=gs[:, :nb])
    n = P.check_e2m1_codes(gc[:, :K], c1["primary"]["codes"], c1["primary"]["elem_arg"], c1["z"], 16,
                           what="primary codes")
    # The residual z - V s_b s_t is a difference: z's fp32 error (held to 1e-5 of the row
    # maximum above) carries over whole, which can exceed 1e-5 of the residual's own
    # argument where a residual block is small against the row.  Its decisions are
    # therefore checked given the GPU's own z as well as its primary codes and scales.
    zg = _np(dbg)[rows]
    c2 = arcquant.quantize(xr, perm, S, gam, eps, tensor_scale_value=gst, primary_scales=gs[:, :nb],
                           primary_codes=gc[:, :K], z=zg)
    if S:
        P.check_e4m3_scales(gs[:, nb:], c2["residual"]["scales"], c2["residual"]["scale_arg"],
                            what="residual scales")
        c3 = arcquant.quantize(xr, perm, S, gam, eps, tensor_scale_value=gst, primary_scales=gs[:, :nb],
                               primary_codes=gc[:, :K], residual_scales=gs[:, nb:], z=zg)
        n += P.check_e2m1_codes(gc[:, K:], c3["residual"]["codes"], c3["residual"]["elem_arg"],
                                c3["residual_value"], 16, what="residual codes")
    return n


@pytest.mark.parametrize("M,K,S", [(1, 16, 16), (7, 128, 32), (33, 512, 0), (130, 1024, 256)])
def test_arcquant_small(M, K, S):
    print(f"arcquant M={M} K={K} S={S}", flush=True)
    rng = np.random.default_rng(M * 31 + K)
    x = rng.standard_normal((M, K))
    x[:, rng.choice(K, max(1, K // 64), replace=False)] *= 30
    xt = W.to_bf16(x)
    perm = W.calibration_order(xt)
    _check_arc(xt, perm, S)


def test_arcquant_gamma_given_scale_and_random_perm():
    rng = np.random.default_rng(44)
    x = rng.standard_normal((50, 256))
    xt = W.to_bf16(x)
    perm = rng.permutation(256).astype(np.int32)
    gamma = rng.uniform(0.5, 1.5, 256)
    _check_arc(xt, perm, 64, gamma=gamma, eps=1e-5, given=0.0021)


@pytest.mark.parametrize("gam", [False, True])
def test_arcquant_config_full_size(gam):
    """bf16 4096 x 4096 N(0,1), 64 outlier channels x30, S = 256 -> K+S = 4352, every row;
    with a gain vector (uniform in [0.5, 1.5], seed 7) as the timed gain workload has it."""
    print(f"arcquant 4096x4096 seed 4 S=256 gamma={gam}", flush=True)
    xt = W.arcquant_input()
    perm = W.calibration_order(xt)
    n = _check_arc(xt, perm, 256, gamma=W.arcquant_gain(4096) if gam else None)
    print(f"  boundary-tolerated code differences: {n}", flush=True)


@pytest.mark.parametrize("M,K,S,gam", [(9000, 256, 64, False), (40, 8192, 512, False), (37, 12288, 256, True),
                                       (5000, 1024, 128, True)])
def test_arcquant_multi_row_and_long_rows(M, K, S, gam):
    """More rows than resident waves (each wave walks several rows, prefetching the next)
    and rows longer than one 4096-channel chunk (the row streams in several chunks)."""
    print(f"arcquant M={M} K={K} S={S} gamma={gam}", flush=True)
    rng = np.random.default_rng(M + K + S)
    x = rng.standard_normal((M, K))
    x[:, rng.choice(K, max(1, K // 64), replace=False)] *= 30
    xt = W.to_bf16(x)
    perm = W.calibration_order(xt)
    gamma = rng.uniform(0.5, 1.5, K) if gam else None
    rows = np.unique(np.concatenate([W.seeded_rows(M, min(M, 48), 9), [0, M - 1]]))
    _check_arc(xt, perm, S, gamma=gamma, rows=rows)


@pytest.mark.parametrize("M,K,gam", [(1, 256, False), (300, 1024, True), (4099, 512, False), (77, 4096, True),
                                     (5, 8192, False)])
def test_dynamic_scale_matches_quantizing_pass(M, K, gam):
    """The statistics pass and the quantizing pass form the same binary32 z: the computed
    tensor scale is exactly fl32(max |z| / 2688) over the quantizing pass's own normalised
    values (dbg_normed), and the whole result passes the oracle parity checks.  Covers the
    register-resident statistics pass (rows up to 4096 channels, one or two rows per wave
    step, with and without a gain vector) and the chunked pass for longer rows."""
    print(f"arcquant dynamic scale M={M} K={K} gamma={gam}", flush=True)
    rng = np.random.default_rng(M * 7 + K)
    x = rng.standard_normal((M, K))
    x[:, rng.choice(K, max(1, K // 64), replace=False)] *= 30
    xt = W.to_bf16(x)
    perm = rng.permutation(K).astype(np.int32)
    gamma = rng.uniform(0.5, 1.5, K) if gam else None
    g = None if gamma is None else torch.from_numpy(gamma.astype(np.float32)).to(DEV)
    dbg = torch.empty((M, K), dtype=torch.float32, device=DEV)
    _, _, ts = fp4.fp4_residual_quantize(xt.to(DEV), torch.from_numpy(perm).to(DEV), 16, gamma=g,
                                         tensor_scale=torch.zeros(1, dtype=torch.float32, device=DEV),
                                         mode="compute", dbg_normed=dbg)
    zmax = np.float32(np.max(np.abs(_np(dbg))))
    assert _np(ts)[0] == zmax / np.float32(2688.0)
    rows = np.unique(np.concatenate([W.seeded_rows(M, min(M, 24), 3), [0, M - 1]]))
    _check_arc(xt, perm, 16, gamma=gamma, rows=rows)


def _degenerate(K, seed):
    """Rows with nothing to normalise against: all zero, one spike, constant, alternating
    signs, Gaussian, tiny (10^-30, far below the tensor's grid), and one with 2^-120
    elements next to a spike of 300.  The gain has zeros (signed zeros reach the codes) and
    negative entries; the permutation is random."""
    rng = np.random.default_rng(seed)
    x = np.zeros((7, K))
    x[1, 7] = 3.0
    x[2, :] = 0.75
    x[3, :] = np.where(np.arange(K) % 2, 1.5, -1.5)
    x[4, :] = rng.standard_normal(K)
    x[5, :] = 1e-30 * rng.standard_normal(K)
    x[6, :] = 2.0 ** -120
    x[6, K // 2] = 300.0
    gamma = rng.uniform(-1.5, 1.5, K)
    gamma[rng.choice(K, K // 8, replace=False)] = 0.0
    return W.to_bf16(x), gamma, rng.permutation(K).astype(np.int32)


@pytest.mark.parametrize("K,gam", [(512, False), (512, True), (8192, True)])
def test_arcquant_degenerate_rows(K, gam):
    print(f"arcquant degenerate rows K={K} gamma={gam}", flush=True)
    xt, gamma, perm = _degenerate(K, K + 5)
    _check_arc(xt, perm, 64, gamma=gamma if gam else None)


def test_arcquant_all_zero_tensor():
    """max|z| = 0: the computed tensor scale is exactly 0, and every code and scale is 0."""
    xt = W.to_bf16(np.zeros((5, 256)))
    codes, scales, ts = fp4.fp4_residual_quantize(xt.to(DEV), torch.arange(256, dtype=torch.int32, device=DEV), 32)
    assert _np(ts)[0] == 0.0 and not np.signbit(_np(ts)[0])
    assert not _np(codes).any() and not _np(scales).any()
