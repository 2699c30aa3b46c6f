"""W4A4 MXFP4 GEMM on dequantized operands, float64 accumulation.

TEST INFRASTRUCTURE: part of the CPU oracle (see oracle/__init__.py).

MR-GPTQ abstract (hyper.ai, Résumé): FP4 GPU kernels with the rotation fused into the
weights and the activations rotated and quantized on the fly; ARCQuant summary
(gist.science, Méthodologie items 3-4): one GEMM over the (extended) reduction
dimension whose high-precision accumulator sums every product.

C[m, n] = sum_k A[m, k] * B[n, k] where A and B are the real values of their MXFP4
codes and E8M0 scales (both operands K-contiguous, B holds one weight row per output
column).  Evaluated on selected rows and columns only; the matrix product of the
dequantized float64 operands is the definition itself.
"""
import numpy as np

from . import mxfp4


def dequantize_rows(packed, scales, rows):
    """Real values of selected rows of an MXFP4 operand (float64)."""
    rows = np.asarray(rows)
    return mxfp4.dequantize(np.asarray(packed)[rows], np.asarray(scales)[rows])


def tile(a_packed, a_scales, b_packed, b_scales, rows, cols):
    """C[rows][:, cols] in float64."""
    a = dequantize_rows(a_packed, a_scales, rows)
    b = dequantize_rows(b_packed, b_scales, cols)
    return a @ b.T


def full(a_packed, a_scales, b_packed, b_scales):
    """The whole product (small shapes only)."""
    a = mxfp4.dequantize(a_packed, a_scales)
    b = mxfp4.dequantize(b_packed, b_scales)
    return a @ b.T
