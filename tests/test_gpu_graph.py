"""Every entry point captured into a HIP graph (torch.cuda.graph) replays to the same
bytes as the eager call.

Each graph is replayed three times, with eager work and a synchronization between the
replays, and the outputs are cleared before every replay; every replay must reproduce
the eager output bit for bit (the kernels are deterministic: no atomics decide a value
except an order-independent maximum).
"""
import numpy as np
import pytest
import torch

import microscaled_fp4_quantization_block_amd as fp4
from microscaled_fp4_quantization_block_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _replays_match(run, outs):
    """run() writes into `outs`; compare three graph replays with the eager result."""
    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for o in outs:
            o.fill_(0x5A if o.dtype == torch.uint8 else 0)
        junk = torch.randn(1024, 1024, device=DEV) @ torch.randn(1024, 1024, device=DEV)  # eager work between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del junk
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"replay {rep} differs"


def test_graph_quantize_nvfp4_dynamic_scale():
    print("graph nvfp4 quantize 256x1024 compute-scale", flush=True)
    x = torch.from_numpy(np.random.default_rng(1).standard_normal((256, 1024)).astype(np.float32)).to(DEV)
    codes = torch.empty((256, 512), dtype=torch.uint8, device=DEV)
    scales = torch.empty((256, 64), dtype=torch.uint8, device=DEV)
    ts = torch.zeros(1, dtype=torch.float32, device=DEV)
    y = torch.empty((256, 1024), dtype=torch.float32, device=DEV)

    def run():
        fp4.fp4_quantize(x, "nvfp4", 0, codes=codes, scales=scales, tensor_scale=ts)
        fp4.fp4_dequantize(codes, scales, ts, "nvfp4", 0, y=y)
    _replays_match(run, [codes, scales, ts, y])


def test_graph_quantize_mxfp4_h32_and_gemm():
    print("graph mxfp4 h32 quantize + gemm 512x1024 @ 768x1024", flush=True)
    rng = np.random.default_rng(2)
    a = W.to_bf16(rng.standard_normal((512, 1024))).to(DEV)
    w = W.to_bf16(rng.normal(0, 0.02, (768, 1024))).to(DEV)
    bc, bs, _ = fp4.fp4_quantize(w, "mxfp4", 32)
    ac = torch.empty((512, 512), dtype=torch.uint8, device=DEV)
    asc = torch.empty((512, 32), dtype=torch.uint8, device=DEV)
    c = torch.empty((512, 768), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((512, 1024), dtype=torch.bfloat16, device=DEV)

    def run():
        fp4.fp4_quantize(a, "mxfp4", 32, codes=ac, scales=asc)
        fp4.fp4_gemm(ac, asc, bc, bs, c=c)
        fp4.fp4_dequantize(ac, asc, None, "mxfp4", 32, y=y)
    _replays_match(run, [ac, asc, c, y])


def test_graph_residual_quantize_dynamic_scale():
    print("graph arcquant 256x1024 S=128 compute-scale", flush=True)
    x_cpu = W.to_bf16(np.random.default_rng(4).standard_normal((256, 1024)))
    perm = torch.from_numpy(W.calibration_order(x_cpu)).to(DEV)
    x = x_cpu.to(DEV)
    codes = torch.empty((256, (1024 + 128) // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((256, (1024 + 128) // 16), dtype=torch.uint8, device=DEV)
    ts = torch.zeros(1, dtype=torch.float32, device=DEV)

    def run():
        fp4.fp4_residual_quantize(x, perm, 128, codes=codes, scales=scales, tensor_scale=ts)
    _replays_match(run, [codes, scales, ts])


def test_graph_residual_quantize_gamma_nvfp4_and_mxfp4():
    """Both residual flavours with a gain vector (one 16-wave workgroup per CU, gamma in
    LDS) and a given NVFP4 tensor scale."""
    print("graph arcquant gamma 300x4096 S=256, nvfp4 given scale + mxfp4", flush=True)
    rng = np.random.default_rng(6)
    x = W.to_bf16(rng.standard_normal((300, 4096))).to(DEV)
    perm = torch.from_numpy(rng.permutation(4096).astype(np.int32)).to(DEV)
    gamma = torch.from_numpy(rng.uniform(0.5, 1.5, 4096).astype(np.float32)).to(DEV)
    ts = torch.tensor([0.004], dtype=torch.float32, device=DEV)
    c_nv = torch.empty((300, (4096 + 256) // 2), dtype=torch.uint8, device=DEV)
    s_nv = torch.empty((300, (4096 + 256) // 16), dtype=torch.uint8, device=DEV)
    c_mx = torch.empty((300, (4096 + 256) // 2), dtype=torch.uint8, device=DEV)
    s_mx = torch.empty((300, (4096 + 256) // 32), dtype=torch.uint8, device=DEV)

    def run():
        fp4.fp4_residual_quantize(x, perm, 256, gamma=gamma, codes=c_nv, scales=s_nv, tensor_scale=ts, mode="given")
        fp4.fp4_residual_quantize_mx(x, perm, 256, gamma=gamma, codes=c_mx, scales=s_mx)
    _replays_match(run, [c_nv, s_nv, c_mx, s_mx])


def test_graph_pack_unpack():
    print("graph pack/unpack 256x1024", flush=True)
    x = W.to_bf16(np.random.default_rng(3).standard_t(4, (256, 1024))).to(DEV)
    packed = torch.empty(fp4.fp4_pack_bytes(256, 1024), dtype=torch.uint8, device=DEV)
    y = torch.empty((256, 1024), dtype=torch.bfloat16, device=DEV)

    def run():
        fp4.fp4_pack(x, packed=packed)
        fp4.fp4_unpack(packed, 256, 1024, y=y)
    _replays_match(run, [packed, y])
