"""GPU parity of the MXFP4 flavour of the ARCQuant kernel and of the augmented K+S GEMM
it feeds (primary and residual activations against reordered weights whose first S
columns are repeated)."""
import numpy as np
import pytest
import torch

import microscaled_fp4_quantization_block_amd as fp4
from microscaled_fp4_quantization_block_amd import workloads as W
from oracle import arcquant, gemm, formats as F
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return t.detach().cpu().numpy()


def _check_arc_mx(xt, perm, S, gamma=None, eps=1e-6, rows=None):
    M, K = xt.shape
    dbg = torch.empty((M, K), dtype=torch.float32, device=DEV)
    g = None if gamma is None else torch.from_numpy(gamma.astype(np.float32)).to(DEV)
    codes, scales = fp4.fp4_residual_quantize_mx(xt.to(DEV), torch.from_numpy(perm.astype(np.int32)).to(DEV), S,
                                                 gamma=g, eps=eps, dbg_normed=dbg)
    rows = np.arange(M) if rows is None else rows
    xr = W.values(xt)[rows]
    gam = None if gamma is None else gamma.astype(np.float32).astype(np.float64)
    gc = F.unpack_nibbles(_np(codes)[rows])
    gs = _np(scales)[rows]
    nb = K // 32
    base = arcquant.quantize_mx(xr, perm, S, gam, eps)
    P.assert_values_close(_np(dbg)[rows], base["z"], K, what="normalized, reordered values")
    P.check_e8m0_scales(gs[:, :nb], base["primary"]["scales"], base["primary"]["amax"], what="primary scales")
    c1 = arcquant.quantize_mx(xr, perm, S, gam, eps, primary_scales=gs[:, :nb])
    n = P.check_e2m1_codes(gc[:, :K], c1["primary"]["codes"], c1["primary"]["elem_arg"], c1["z"], 32,
                           what="primary codes")
    if S:
        # residual decisions given the GPU's own z (see the NVFP4 check)
        zg = _np(dbg)[rows]
        c2 = arcquant.quantize_mx(xr, perm, S, gam, eps, primary_scales=gs[:, :nb], primary_codes=gc[:, :K], z=zg)
        P.check_e8m0_scales(gs[:, nb:], c2["residual"]["scales"], c2["residual"]["amax"], what="residual scales")
        c3 = arcquant.quantize_mx(xr, perm, S, gam, eps, primary_scales=gs[:, :nb], primary_codes=gc[:, :K],
                                  residual_scales=gs[:, nb:], z=zg)
        n += P.check_e2m1_codes(gc[:, K:], c3["residual"]["codes"], c3["residual"]["elem_arg"],
                                c3["residual_value"], 32, what="residual codes")
    return codes, scales, n


def _input(M, K, seed, outliers):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    x[:, rng.choice(K, outliers, replace=False)] *= 30
    return W.to_bf16(x)


@pytest.mark.parametrize("M,K,S", [(1, 32, 32), (9, 128, 64), (33, 512, 0), (130, 1024, 256), (5000, 256, 96),
                                   (21, 8192, 512)])
def test_arcquant_mx_shapes(M, K, S):
    print(f"arcquant mx M={M} K={K} S={S}", flush=True)
    xt = _input(M, K, M + K, max(1, K // 64))
    perm = W.calibration_order(xt)
    rows = W.seeded_rows(M, 64, 3)
    _check_arc_mx(xt, perm, S, rows=rows)


def test_arcquant_mx_gamma_random_perm():
    rng = np.random.default_rng(61)
    xt = W.to_bf16(rng.standard_normal((40, 256)))
    perm = rng.permutation(256).astype(np.int32)
    _check_arc_mx(xt, perm, 64, gamma=rng.uniform(0.5, 1.5, 256), eps=1e-5)


@pytest.mark.parametrize("gam", [False, True])
def test_arcquant_mx_config_full_size(gam):
    """The ARCQuant configuration (bf16 4096 x 4096, 64 outlier channels x30, S = 256) in
    the MXFP4 flavour, every row; with a gain vector (uniform in [0.5, 1.5], seed 7) too."""
    print(f"arcquant mx 4096x4096 seed 4 S=256 gamma={gam}", flush=True)
    xt = W.arcquant_input()
    perm = W.calibration_order(xt)
    _, _, n = _check_arc_mx(xt, perm, 256, gamma=W.arcquant_gain(4096) if gam else None)
    print(f"  boundary-tolerated code differences: {n}", flush=True)


def test_augmented_gemm_end_to_end():
    """[A_primary | A_residual] x [W_perm | W_perm[:, :S]]^T on scaled MFMA equals the float64
    product of the same operands (T3), and the residual channels move the result towards
    the unquantized y W^T."""
    print("augmented gemm M=256 K=1024 S=128 N=384", flush=True)
    M, K, S, N = 256, 1024, 128, 384
    xt = _input(M, K, 7, 16)
    perm = W.calibration_order(xt)
    codes, scales, _ = _check_arc_mx(xt, perm, S)
    w = W.to_bf16(np.random.default_rng(8).normal(0, 0.02, (N, K))).to(DEV)
    w_perm = w[:, torch.from_numpy(perm.astype(np.int64)).to(DEV)].contiguous()
    w_aug = torch.cat([w_perm, w_perm[:, :S]], dim=1).contiguous()
    bc, bs, _ = fp4.fp4_quantize(w_aug, "mxfp4", 0)
    c = fp4.fp4_gemm(codes, scales, bc, bs, out_dtype=torch.float32)
    ref = gemm.full(_np(codes), _np(scales), _np(bc), _np(bs))
    cg = _np(c).astype(np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    assert np.all(np.abs(cg - ref) <= 1e-3 * np.maximum(np.abs(ref), rms))
    # primary part alone: the first K columns of both operands
    cp = fp4.fp4_gemm(codes[:, :K // 2].contiguous(), scales[:, :K // 32].contiguous(),
                      bc[:, :K // 2].contiguous(), bs[:, :K // 32].contiguous(), out_dtype=torch.float32)
    y = arcquant.rmsnorm(W.values(xt))
    exact = y @ W.values(w.cpu()).T
    e_aug = np.linalg.norm(cg - exact)
    e_plain = np.linalg.norm(_np(cp).astype(np.float64) - exact)
    print(f"  |C - yW^T|: augmented {e_aug:.4g}, primary only {e_plain:.4g}", flush=True)
    assert e_aug < e_plain


@pytest.mark.parametrize("K,gam", [(512, False), (512, True), (8192, True)])
def test_arcquant_mx_degenerate_rows(K, gam):
    """The NVFP4 test's degenerate rows (all zero, spike, constant, alternating, tiny,
    2^-120 beside a spike) with a gain holding zeros and negative entries."""
    from tests.test_gpu_arcquant import _degenerate
    print(f"arcquant mx degenerate rows K={K} gamma={gam}", flush=True)
    xt, gamma, perm = _degenerate(K, K + 9)
    _check_arc_mx(xt, perm, 64, gamma=gamma if gam else None)
