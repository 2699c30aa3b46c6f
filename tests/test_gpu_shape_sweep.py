"""Seeded sweep of shapes per operation against the oracle, beyond the hand-picked cases:
rows from 1 up to a few hundred (ragged last workgroups and tiles), row lengths across
the rotation and block multiples each call admits, long ARCQuant rows streamed in
chunks, and GEMM shapes with ragged M, N and K.  The shapes come from one seeded
generator, so every run checks the same cases; each is checked with the tolerance rules
of the hand-picked tests (bit-exact where the path is exact)."""
import numpy as np
import pytest
import torch

import microscaled_fp4_quantization_block_amd as fp4
from microscaled_fp4_quantization_block_amd import workloads as W
from oracle import formats as F, gemm, nvfp4
from tests import parity as P
from tests.test_gpu_arcquant import _check_arc
from tests.test_gpu_arcquant_mx import _check_arc_mx
from tests.test_gpu_gemm import _assert_gemm_close, _g
from tests.test_gpu_pack import _check_pack
from tests.test_gpu_quantize import _check_mx_rotated, _nvfp4_exact_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

_rng = np.random.default_rng(20261203)


def _rows():
    return int(_rng.choice([1, 2, 3, 63, 64, 65, 127, 129, 255, 257, 300]))


# (M, K, input dtype) for the exact NVFP4 round trip; K a multiple of 32
NV_EXACT = [(_rows(), 32 * int(_rng.integers(1, 33)), str(_rng.choice(["bf16", "f32"]))) for _ in range(16)]
# (M, K, h) for rotated MXFP4; K a multiple of max(32, h)
MX_ROT = []
for _ in range(18):
    h = int(_rng.choice([16, 32, 128]))
    MX_ROT.append((_rows(), max(32, h) * int(_rng.integers(1, 17 if h == 128 else 33)), h))
# (M, K, h) for rotated NVFP4 with the dynamic tensor scale
NV_ROT = []
for _ in range(12):
    h = int(_rng.choice([16, 32, 128]))
    NV_ROT.append((_rows(), max(32, h) * int(_rng.integers(1, 17 if h == 128 else 33)), h))
# (M, K) for the dual-scale pack; K a multiple of 128
PACK = [(_rows(), 128 * int(_rng.integers(1, 17))) for _ in range(12)]
# (M, K, S, gamma) for ARCQuant NVFP4 (K a multiple of 16) and MXFP4 (of 32); two shapes each with rows past
# one 4096-channel chunk each
ARC_NV = [(_rows(), 16 * int(_rng.integers(1, 257)), None, bool(_rng.integers(0, 2))) for _ in range(12)]
ARC_NV += [(int(_rng.integers(1, 40)), 4096 + 16 * int(_rng.integers(1, 257)), None, bool(_rng.integers(0, 2)))
           for _ in range(2)]
ARC_MX = [(_rows(), 32 * int(_rng.integers(1, 129)), None, bool(_rng.integers(0, 2))) for _ in range(12)]
ARC_MX += [(int(_rng.integers(1, 40)), 4096 + 32 * int(_rng.integers(1, 129)), None, bool(_rng.integers(0, 2)))
           for _ in range(2)]
ARC_NV = [(m, k, 16 * int(_rng.integers(0, k // 16 + 1)), g) for m, k, _, g in ARC_NV]
ARC_MX = [(m, k, 32 * int(_rng.integers(0, k // 32 + 1)), g) for m, k, _, g in ARC_MX]
# (M, N, K) for the GEMM; K a multiple of 128 from 256 up
GEMM = [(int(_rng.integers(1, 700)), int(_rng.integers(1, 700)), 128 * int(_rng.integers(2, 25))) for _ in range(14)]


def _input(M, K, seed, dtype="bf16"):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    x[:, rng.choice(K, max(1, K // 64), replace=False)] *= 30
    if dtype == "f32":
        return torch.from_numpy(x.astype(np.float32))
    return W.to_bf16(x)


@pytest.mark.parametrize("M,K,dt", NV_EXACT)
def test_sweep_nvfp4_roundtrip_exact(M, K, dt):
    print(f"sweep nvfp4 exact M={M} K={K} {dt}", flush=True)
    _nvfp4_exact_case(_input(M, K, M * 7 + K, dt))


@pytest.mark.parametrize("M,K,h", MX_ROT)
def test_sweep_mxfp4_rotated(M, K, h):
    print(f"sweep mxfp4 H{h} M={M} K={K}", flush=True)
    _check_mx_rotated(_input(M, K, M * 11 + K + h), h)


@pytest.mark.parametrize("M,K,h", NV_ROT)
def test_sweep_nvfp4_rotated_dynamic_scale(M, K, h):
    print(f"sweep nvfp4 H{h} M={M} K={K}", flush=True)
    xt = _input(M, K, M * 23 + K + h)
    dbg = torch.empty((M, K), dtype=torch.float32, device=DEV)
    codes, scales, ts = fp4.fp4_quantize(xt.to(DEV), "nvfp4", h, dbg_rotated=dbg)
    xv = W.values(xt)
    ref = nvfp4.quantize(xv, hadamard=h)
    d = dbg.cpu().numpy()
    P.assert_values_close(d, ref["y"], h, what="rotated values")
    gst = ts.cpu().numpy()[0]
    assert gst == np.float32(np.max(np.abs(d))) / np.float32(2688.0)    # of the kernel's own values
    c1 = nvfp4.quantize(xv, hadamard=h, tensor_scale_value=gst)
    P.check_e4m3_scales(scales.cpu().numpy(), c1["scales"], c1["scale_arg"])
    c2 = nvfp4.quantize(xv, hadamard=h, tensor_scale_value=gst, block_scales=scales.cpu().numpy())
    P.check_e2m1_codes(F.unpack_nibbles(codes.cpu().numpy()), c2["codes"], c2["elem_arg"], c2["y"], 16)


@pytest.mark.parametrize("M,K", PACK)
def test_sweep_pack(M, K):
    print(f"sweep pack M={M} K={K}", flush=True)
    _check_pack(_input(M, K, M * 13 + K))


@pytest.mark.parametrize("M,K,S,gam", ARC_NV)
def test_sweep_arcquant(M, K, S, gam):
    print(f"sweep arcquant M={M} K={K} S={S} gamma={gam}", flush=True)
    xt = _input(M, K, M * 17 + K + S)
    rng = np.random.default_rng(K + S)
    _check_arc(xt, rng.permutation(K).astype(np.int32), S, gamma=rng.uniform(0.5, 1.5, K) if gam else None)


@pytest.mark.parametrize("M,K,S,gam", ARC_MX)
def test_sweep_arcquant_mx(M, K, S, gam):
    print(f"sweep arcquant mx M={M} K={K} S={S} gamma={gam}", flush=True)
    xt = _input(M, K, M * 19 + K + S)
    rng = np.random.default_rng(K + S + 1)
    _check_arc_mx(xt, rng.permutation(K).astype(np.int32), S, gamma=rng.uniform(0.5, 1.5, K) if gam else None)


@pytest.mark.parametrize("M,N,K", GEMM)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_sweep_gemm(M, N, K, out):
    print(f"sweep gemm M={M} N={N} K={K} {out}", flush=True)
    a, sa = W.random_mxfp4_operand(M, K, seed=M + 3 * K)
    b, sb = W.random_mxfp4_operand(N, K, seed=N + 5 * K)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    c = fp4.fp4_gemm(_g(a), _g(sa), _g(b), _g(sb), out_dtype=dt)
    _assert_gemm_close(W.values(c.cpu()), gemm.full(a, sa, b, sb), out == "bf16")
