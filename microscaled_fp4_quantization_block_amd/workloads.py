"""Seeded synthetic inputs shaped like the LLM activations and weights the pages quantize.

This module holds input generation only (random draws, dtype casts, a calibration-style
channel ordering); none of the quantization arithmetic lives here.  It is shared by the
tests (which hand the same bytes to the HIP library and to the CPU oracle) and by the
benchmark.

The pages measure on trained LLMs (Qwen-7B for FP4Quant; LLaMA-3.1 and Qwen2.5 7B-70B
for ARCQuant; LLM layers on B200 / RTX 5090 for MR-GPTQ).  No weights or datasets are
used: the stand-ins below draw Gaussian / Student-t values with planted outlier channels
at the hidden sizes of those model classes (4096 for 8B-class, 8192 x 28672 for a
70B-class MLP projection).

Draws: NumPy PCG64 `default_rng(seed)` in float64, rounded to binary32 (nearest-even)
and, for bfloat16 inputs, to bfloat16 by torch (nearest-even).
"""
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    shape: tuple
    seed: int
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "nvfp4_roundtrip": Workload(
        "nvfp4_roundtrip",
        "NVFP4 quantize + dequantize, no rotation: fp32 256x1024 N(0,1), block 16, "
        "E4M3 block scales + FP32 tensor scale",
        (256, 1024), 1),
    "mxfp4_h32": Workload(
        "mxfp4_h32",
        "MXFP4 quantize with block Hadamard 32: bf16 4096x4096 N(0,1), 41 outlier "
        "channels x50, E8M0 per 32, packed output + dequant",
        (4096, 4096), 2, dict(outliers=41, outlier_gain=50.0)),
    "nvfp4_h16": Workload(
        "nvfp4_h16",
        "NVFP4 quantize with block Hadamard 16 and a calibrated (static) FP32 tensor scale: the "
        "MXFP4 workload's input (bf16 4096x4096 N(0,1), 41 outlier channels x50), E4M3 scales "
        "per 16, packed output + dequant with the inverse rotation",
        (4096, 4096), 2, dict(outliers=41, outlier_gain=50.0)),
    "dualscale_pack": Workload(
        "dualscale_pack",
        "dual-scale micro-grouped FP4 pack/unpack, two-level FWHT 16x8: bf16 8192x8192 "
        "Student-t df=4",
        (8192, 8192), 3, dict(df=4)),
    "arcquant": Workload(
        "arcquant",
        "fused RMSNorm + absmax channel reorder + NVFP4 primary + residual of top 256 "
        "channels: bf16 4096x4096 N(0,1), 64 outlier channels x30, K+S = 4352",
        (4096, 4096), 4, dict(outliers=64, outlier_gain=30.0, S=256, eps=1e-6)),
    "arcquant_gamma": Workload(
        "arcquant_gamma",
        "the arcquant workload with a gain vector: gamma[K] uniform in [0.5, 1.5] (seed 7), "
        "NVFP4 primary + residual of top 256 channels, K+S = 4352",
        (4096, 4096), 4, dict(outliers=64, outlier_gain=30.0, S=256, eps=1e-6, gamma_seed=7)),
    "arcquant_mx": Workload(
        "arcquant_mx",
        "the arcquant workload in the MXFP4 flavour: RMSNorm + reorder + MXFP4 primary + "
        "residual of top 256 channels, E8M0 per 32, K+S = 4352",
        (4096, 4096), 4, dict(outliers=64, outlier_gain=30.0, S=256, eps=1e-6)),
    "arcquant_gemm": Workload(
        "arcquant_gemm",
        "ARCQuant augmented GEMM (MXFP4 flavour): bf16 4096x4096 activations N(0,1) with 64 "
        "outlier channels x30, RMSNorm + reorder + MXFP4 primary + residual of the top 256 "
        "channels, then the K+S = 4352 GEMM against 14336 reordered MXFP4 weight rows (first "
        "256 reordered columns repeated) from N(0,0.02); compared with the same path at S = 0",
        (4096, 4096), 4, dict(outliers=64, outlier_gain=30.0, S=256, eps=1e-6, N=14336, weight_seed=51,
                              weight_std=0.02)),
    "w4a4_gemm": Workload(
        "w4a4_gemm",
        "W4A4 MXFP4 GEMM, Hadamard-32 activation quant on the fly: A bf16 8192x8192 "
        "N(0,1), B = Hadamard-rotated MXFP4 weights 28672x8192 from N(0,0.02)",
        (8192, 8192), 5, dict(N=28672, weight_seed=50, weight_std=0.02, tile_seed=500,
                              tiles=64, tile=128)),
    "w4a4_shard": Workload(
        "w4a4_shard",
        "the W4A4 step at one GPU's column shard of eight: Hadamard-32 MXFP4 quantization of "
        "A bf16 8192x8192 N(0,1), GEMM against the first 3584 of the 28672 rotated MXFP4 "
        "weight rows (N(0,0.02), the same draw)",
        (8192, 8192), 5, dict(N=3584, shards=8, weight_seed=50, weight_std=0.02, tile_seed=500,
                              tiles=64, tile=128)),
}


def to_bf16(a):
    """float64 array -> torch bfloat16 tensor (via binary32, both nearest-even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64).astype(np.float32)).to(torch.bfloat16)


def values(t):
    """Exact float64 numpy values of a CPU tensor of any float dtype."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def gaussian_with_outliers(shape, seed, outliers=0, gain=1.0):
    """N(0,1) draws; `outliers` distinct columns (seeded choice) multiplied by `gain`."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    if outliers:
        cols = rng.choice(shape[1], outliers, replace=False)
        x[:, cols] *= gain
    return x


def nvfp4_roundtrip_input(shape=(256, 1024), seed=1):
    """fp32 tensor of N(0,1) draws."""
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32))


def mxfp4_h32_input(shape=(4096, 4096), seed=2, outliers=41, gain=50.0):
    return to_bf16(gaussian_with_outliers(shape, seed, outliers, gain))


def student_t_input(shape=(8192, 8192), seed=3, df=4):
    rng = np.random.default_rng(seed)
    return to_bf16(rng.standard_t(df, shape))


def arcquant_input(shape=(4096, 4096), seed=4, outliers=64, gain=30.0):
    return to_bf16(gaussian_with_outliers(shape, seed, outliers, gain))


def arcquant_gain(k, seed=7):
    """A seeded RMSNorm gain vector, float32 [k], uniform in [0.5, 1.5]."""
    return np.random.default_rng(seed).uniform(0.5, 1.5, k).astype(np.float32)


def calibration_order(x):
    """Channel order by descending column absolute maximum, ties to the lower index.

    Stand-in for ARCQuant's calibration step (channels reordered by their absolute
    maxima, measured on calibration data): the activations themselves serve as the
    calibration set.  Returns int32 [K].
    """
    colmax = np.max(np.abs(values(x) if isinstance(x, torch.Tensor) else np.asarray(x)), axis=0)
    return np.argsort(-colmax, kind="stable").astype(np.int32)


def gemm_activations(shape=(8192, 8192), seed=5):
    rng = np.random.default_rng(seed)
    return to_bf16(rng.standard_normal(shape))


def gemm_weights(n=28672, k=8192, seed=50, std=0.02):
    """Weight matrix [N, K] (one row per output column), N(0, std) in bf16."""
    rng = np.random.default_rng(seed)
    return to_bf16(rng.normal(0.0, std, (n, k)))


def gemm_tiles(m, n, tile=128, count=64, seed=500):
    """`count` distinct (row0, col0) output tiles of size tile x tile, seeded."""
    rng = np.random.default_rng(seed)
    tm, tn = m // tile, n // tile
    picks = rng.choice(tm * tn, min(count, tm * tn), replace=False)
    return [(int(p // tn) * tile, int(p % tn) * tile) for p in picks]


def random_mxfp4_operand(rows, k, seed, exp_lo=120, exp_hi=128):
    """Random packed E2M1 codes [rows, k/2] and E8M0 codes [rows, k/32] in [exp_lo, exp_hi).

    Uniform code bytes cover every element value and sign; the scale range mimics the
    block scales of unit-variance (around 2^-2) and small-weight (around 2^-8) tensors.
    """
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    scales = rng.integers(exp_lo, exp_hi, (rows, k // 32), dtype=np.uint8)
    return packed, scales


def seeded_rows(m, count, seed):
    """Sorted distinct row indices including the first and the last row."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(m, min(count, m), replace=False).tolist()) | {0, m - 1}
    return np.array(sorted(rows))
