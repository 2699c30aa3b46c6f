"""MXFP4 quantization and dequantization, in float64.

TEST INFRASTRUCTURE: part of the CPU oracle (see oracle/__init__.py).

What the pages fix: MXFP4 uses power-of-two scales, which the MR-GPTQ abstract
(hyper.ai, Résumé, finding (2)) blames for a high induced error; the same abstract
applies block Hadamard rotations before quantization, fused into the weights offline
and computed on the fly for activations.  The ARCQuant summary (Énoncé du Problème)
notes that the higher-precision micro-scaled formats use blocks of 32.

Reading taken where the pages are silent (OCP MX v1.0): one E8M0 scale per 32
contiguous elements along the last axis, X = 2^(floor(log2 amax_b) - 2), element code
E2M1_RNE(y / X).  Values in (6 X, 8 X) therefore saturate to 6 X.  Division by a power
of two is exact in float64, so the codes are exact.
"""
import numpy as np

from . import formats as F
from .hadamard import rotate

BLOCK = 32


def quantize(x, hadamard=0, block_scales=None):
    """MXFP4 of a 2-D tensor [M, K] after an optional block Hadamard rotation (0/16/32, or
    128 for the two-level 16 x 8 transform).

    Returns `packed` [M, K/2] u8, `codes` [M, K], `scales` [M, K/32] u8 (E8M0 codes),
    the rotated values `y`, the block maxima `amax` and the element arguments
    `elem_arg` (y / X).  `block_scales` overrides the computed E8M0 codes.
    """
    y = rotate(np.asarray(x, dtype=np.float64), hadamard)
    k = y.shape[-1]
    assert k % BLOCK == 0
    blocks = y.reshape(y.shape[:-1] + (k // BLOCK, BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    if block_scales is None:
        e = F.e8m0_from_amax(amax)
    else:
        e = np.asarray(block_scales, dtype=np.uint8).reshape(amax.shape)
    q = blocks / F.e8m0_decode(e)[..., None]
    codes = F.e2m1_rne(q).reshape(y.shape)
    return dict(packed=F.pack_nibbles(codes), codes=codes, scales=e.astype(np.uint8),
                y=y, amax=amax, elem_arg=q.reshape(y.shape))


def dequantize_exact(codes, scales):
    """V(c) * 2^(e - 127) of unpacked codes, float64 (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    k = codes.shape[-1]
    v = F.e2m1_decode(codes).reshape(codes.shape[:-1] + (k // BLOCK, BLOCK))
    return (v * F.e8m0_decode(scales)[..., None]).reshape(codes.shape)


def dequantize(packed, scales, inverse_hadamard=0):
    """Dequantized values (float64), with the optional inverse rotation applied after."""
    return rotate(dequantize_exact(F.unpack_nibbles(packed), scales), inverse_hadamard)
