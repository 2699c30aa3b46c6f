"""GPU parity of the fused-quantization experiment (libfp4probe.so, fp4probe_gemm_fused_a):
the GEMM that rotates and quantizes its bf16 activations inside every tile must give
exactly what fp4_quantize (MXFP4, H_32) followed by fp4_gemm gives -- same arithmetic, same
MFMA order -- and the oracle's product of the oracle-quantized operands within the GEMM
tolerance."""
import ctypes
import os

import numpy as np
import pytest
import torch

import microscaled_fp4_quantization_block_amd as fp4
from microscaled_fp4_quantization_block_amd import workloads as W
from oracle import gemm, mxfp4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LIB = os.path.join(os.path.dirname(fp4.library_path()), "libfp4probe.so")


def _fused(a, bc, bs, out_dtype):
    L = ctypes.CDLL(LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.fp4probe_gemm_fused_a.argtypes = [vp, vp, vp, i64, i64, i64, vp, ctypes.c_int, vp]
    M, K = a.shape
    N = bc.shape[0]
    c = torch.empty((M, N), dtype=out_dtype, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.fp4probe_gemm_fused_a(vp(a.data_ptr()), vp(bc.data_ptr()), vp(bs.data_ptr()), M, N, K,
                                 vp(c.data_ptr()), int(out_dtype == torch.bfloat16), st)
    assert rc == 0
    return c


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 520, 512), (1, 33, 1024), (777, 392, 2048),
                                   (513, 257, 8192)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_fused_equals_quantize_then_gemm(M, N, K, out):
    print(f"fused gemm M={M} N={N} K={K} {out}", flush=True)
    rng = np.random.default_rng(M * 3 + N + K)
    x = rng.standard_normal((M, K))
    x[:, rng.integers(0, K)] *= 40
    a = W.to_bf16(x).to(DEV)
    w = W.to_bf16(rng.normal(0, 0.02, (N, K))).to(DEV)
    bc, bs, _ = fp4.fp4_quantize(w, "mxfp4", 32)
    ac, asc, _ = fp4.fp4_quantize(a, "mxfp4", 32)
    ref = fp4.fp4_gemm(ac, asc, bc, bs, out_dtype=out)
    got = _fused(a, bc, bs, out)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_fused_against_the_oracle():
    rng = np.random.default_rng(77)
    M, N, K = 200, 300, 1024
    xa = W.to_bf16(rng.standard_normal((M, K)))
    w = W.to_bf16(rng.normal(0, 0.02, (N, K)))
    bc, bs, _ = fp4.fp4_quantize(w.to(DEV), "mxfp4", 32)
    got = W.values(_fused(xa.to(DEV), bc, bs, torch.float32).cpu())
    qa = mxfp4.quantize(W.values(xa), hadamard=32)
    ref = gemm.full(qa["packed"], qa["scales"], bc.cpu().numpy(), bs.cpu().numpy())
    rms = np.sqrt(np.mean(ref * ref))
    # the oracle's codes may differ from the GPU's only at rounding boundaries (T2), which
    # moves a product by one code step of one element: far inside this bound
    assert np.max(np.abs(got - ref)) <= 2e-2 * rms
    assert np.mean(np.abs(got - ref) <= 1e-3 * np.maximum(np.abs(ref), rms)) > 0.999


def test_fused_rejects_ragged_k():
    L = ctypes.CDLL(LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.fp4probe_gemm_fused_a.argtypes = [vp, vp, vp, i64, i64, i64, vp, ctypes.c_int, vp]
    assert L.fp4probe_gemm_fused_a(vp(0x10000), vp(0x10000), vp(0x10000), 4, 4, 384, vp(0x10000), 1, None) == 1
