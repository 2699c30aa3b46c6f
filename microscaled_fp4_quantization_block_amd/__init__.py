"""Micro-scaled FP4 quantization on AMD Instinct MI355X (gfx950).

The compute lives in libfp4.so (hand-written HIP kernels behind a C ABI, see
include/fp4.h); `binding` exposes the same entry points for torch tensors and
`workloads` generates the seeded synthetic inputs.  Importing the package does not load
the library; the first call does, and fails loudly if it has not been built.
"""
from .binding import (  # noqa: F401
    Fp4Error, fp4_dequantize, fp4_gemm, fp4_pack, fp4_pack_bytes, fp4_quantize,
    fp4_residual_quantize, fp4_residual_quantize_mx, fp4_unpack, lib, library_path,
)
