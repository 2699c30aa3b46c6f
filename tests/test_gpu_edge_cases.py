"""Degenerate inputs through the unrotated quantizers (exact paths): all-zero tensors,
negative zeros, a single non-zero element per block, saturating blocks, and binary32
subnormals (which reach the E8M0 clamp at code 0 and subnormal NVFP4 tensor scales).
Every code, scale and dequantized value is compared bit for bit with the oracle."""
import numpy as np
import pytest
import torch

import microscaled_fp4_quantization_block_amd as fp4
from oracle import formats as F, mxfp4, nvfp4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return t.detach().cpu().numpy()


def _cases():
    rng = np.random.default_rng(300)
    zeros = np.zeros((4, 64), np.float32)
    negz = np.full((4, 64), -0.0, np.float32)
    negz[:, ::3] = 0.0
    single = np.zeros((4, 64), np.float32)
    single[np.arange(4), [0, 17, 33, 63]] = [1.5, -3.0e-3, 7.0e5, -2.0 ** -20]
    sat = rng.standard_normal((4, 64)).astype(np.float32)
    sat[:, 5] = 7.9            # block max / scale lands in (6, 8): saturation to 6
    sat[:, 40] = -1e6
    sub = (rng.standard_normal((4, 64)) * 1e-39).astype(np.float32)      # binary32 subnormals
    sub[0, :] = np.float32(2.0 ** -149) * np.arange(64)
    mixed = rng.standard_normal((4, 64)).astype(np.float32) * np.float32(1e-30)
    mixed[:, 7] = 3e20
    return {"zeros": zeros, "negative_zeros": negz, "single": single, "saturating": sat,
            "subnormal": sub, "wide_range": mixed}


@pytest.mark.parametrize("name", list(_cases()))
def test_mxfp4_degenerate_exact(name):
    x = _cases()[name]
    codes, scales, _ = fp4.fp4_quantize(torch.from_numpy(x).to(DEV), "mxfp4", 0)
    ref = mxfp4.quantize(x.astype(np.float64))
    assert np.array_equal(_np(scales), ref["scales"]), name
    assert np.array_equal(_np(codes), ref["packed"]), name
    y = fp4.fp4_dequantize(codes, scales, None, "mxfp4", 0, torch.float32)
    want = mxfp4.dequantize(ref["packed"], ref["scales"]).astype(np.float32)
    assert np.array_equal(_np(y).view(np.uint32), want.view(np.uint32)), name


@pytest.mark.parametrize("name", list(_cases()))
def test_nvfp4_degenerate_exact(name):
    x = _cases()[name]
    codes, scales, ts = fp4.fp4_quantize(torch.from_numpy(x).to(DEV), "nvfp4", 0)
    ref = nvfp4.quantize(x.astype(np.float64))
    assert _np(ts)[0].tobytes() == np.float32(ref["tensor_scale"]).tobytes(), name
    assert np.array_equal(_np(scales), ref["scales"]), name
    assert np.array_equal(_np(codes), ref["packed"]), name
    y = fp4.fp4_dequantize(codes, scales, ts, "nvfp4", 0, torch.float32)
    want = nvfp4.dequantize(ref["packed"], ref["scales"], ref["tensor_scale"]).astype(np.float32)
    assert np.array_equal(_np(y).view(np.uint32), want.view(np.uint32)), name


def test_gemm_zero_and_extreme_scales():
    """All-zero codes give exact zeros; the largest and smallest E8M0 scales that keep the
    products finite in fp32 agree with float64."""
    from oracle import gemm
    M, N, K = 64, 64, 256
    rng = np.random.default_rng(301)
    a = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    b = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    za = np.zeros_like(a)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    g = lambda t: torch.from_numpy(np.ascontiguousarray(t)).to(DEV)
    c0 = fp4.fp4_gemm(g(za), g(sa), g(b), g(sb), out_dtype=torch.float32)
    assert not _np(c0).any()
    for ea, eb in ((127 + 60, 127 + 50), (127 - 60, 127 - 50)):
        sa[:] = ea
        sb[:] = eb
        c = _np(fp4.fp4_gemm(g(a), g(sa), g(b), g(sb), out_dtype=torch.float32)).astype(np.float64)
        ref = gemm.full(a, sa, b, sb)
        rms = np.sqrt(np.mean(ref * ref))
        assert np.all(np.abs(c - ref) <= 1e-3 * np.maximum(np.abs(ref), rms)), (ea, eb)
