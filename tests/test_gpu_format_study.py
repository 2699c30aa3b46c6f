"""The format-error figures reported by `bench.py --workload format_study` agree with the
oracle: on sampled rows, the library's quantize + dequantize round trip has the same
relative squared error as the float64 oracle (rotated formats within fp32 rounding of
the rotation, unrotated ones exactly)."""
import numpy as np
import pytest
import torch

import bench
from microscaled_fp4_quantization_block_amd import workloads as W
from oracle import dualscale, mxfp4, nvfp4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _rel(xhat, x):
    return float(np.sum((xhat - x) ** 2) / np.sum(x * x))


@pytest.mark.parametrize("dist", ["outliers", "student_t"])
def test_format_errors_match_oracle(dist):
    print(f"format study {dist}", flush=True)
    rng = np.random.default_rng(70)
    if dist == "outliers":
        x = W.gaussian_with_outliers((256, 1024), 71, 10, 50.0)
    else:
        x = rng.standard_t(4, (256, 1024))
    xt = W.to_bf16(x)
    xv = W.values(xt)
    gpu = bench.format_errors(xt.to(DEV))
    ref = {}
    for h in (0, 16, 32):
        q = nvfp4.quantize(xv, hadamard=h)
        ref["nvfp4" + (f"+H{h}" if h else "")] = _rel(nvfp4.dequantize(q["packed"], q["scales"], q["tensor_scale"], h), xv)
        q = mxfp4.quantize(xv, hadamard=h)
        ref["mxfp4" + (f"+H{h}" if h else "")] = _rel(mxfp4.dequantize(q["packed"], q["scales"], h), xv)
    m = dualscale.pack(xv)
    ref["dualscale+H128(16x8)"] = _rel(dualscale.unpack(m, 256, 1024), xv)
    for k, v in ref.items():
        tol = 1e-9 if k in ("nvfp4", "mxfp4") else 2e-3
        assert abs(gpu[k] - v) <= tol * v, (k, gpu[k], v)
