"""NVFP4 quantization and dequantization, in float64.

TEST INFRASTRUCTURE: part of the CPU oracle (see oracle/__init__.py).

What the pages fix: NVFP4 is a fine-grained micro-scaled format with blocks of 16
(ARCQuant summary, gist.science, Énoncé du Problème, second bullet) and E2M1 elements
(Méthodologie, item 1); standard NVFP4 practice uses a per-tensor scale next to the
block scales (nGPT abstract on thelatestinai.com, which names per-tensor scaling and
random Hadamard transforms as the usual NVFP4 interventions).  ARCQuant's primary
stage is "standard block NVFP4 quantization" (Méthodologie, item 2).

Reading taken where the pages are silent (bit-level formats in oracle/formats.py):
* tensor scale   s_t = fl32(amax(x) / (6 * 448)), one correctly rounded fp32 division
                 (a decode scale: the largest block scale 448 times the largest
                 element 6 maps to amax), or a caller-given value;
* block scale    s_b = E4M3_RNE(amax_b / (6 s_t)) of the exact quotient; s_b = 0 when
                 s_t = 0 or amax_b = 0;
* element code   c_i = E2M1_RNE(x_i / (s_b s_t)) of the exact quotient; when
                 s_b s_t = 0 the code keeps only the sign bit;
* dequantized    fl32(V(c) * s_b * s_t) (V(c) * s_b is exact, so one rounding).

Exactness of the float64 evaluation: every operand is a binary32 (or shorter) value,
s_b has 4 significant bits and the grid midpoints 5, so a real quotient that is not a
midpoint sits at least 2^-33 (relative) away from every midpoint, far above the 2^-53
error of one float64 division; an exact midpoint divides exactly.  The float64
quotients therefore take the same decisions as the exact real ones.
"""
import numpy as np

from . import formats as F
from .hadamard import rotate

BLOCK = 16
#: largest E4M3 block scale times largest E2M1 magnitude
TENSOR_SCALE_DIVISOR = F.E4M3_MAX * F.E2M1_MAX      # 2688


def tensor_scale(x):
    """s_t = fl32(amax / 2688).  The float64 quotient rounded once more to binary32 is
    the correctly rounded binary32 quotient (53 >= 2*24 + 2, so double rounding is
    innocuous for division)."""
    amax = float(np.max(np.abs(np.asarray(x, dtype=np.float64)))) if np.size(x) else 0.0
    return np.float32(amax / TENSOR_SCALE_DIVISOR)


def quantize_blocks(y, s_t, block_scales=None):
    """Block NVFP4 of values y (float64, last axis a multiple of 16) under tensor scale s_t.

    Returns codes (one per element, uint8 0..15), E4M3 scale codes (one per block) and
    the real arguments of both decisions (for boundary-aware comparisons).  If
    `block_scales` is given, those E4M3 codes are used instead of being computed.
    """
    y = np.asarray(y, dtype=np.float64)
    k = y.shape[-1]
    assert k % BLOCK == 0
    s_t = float(np.float32(s_t))
    blocks = y.reshape(y.shape[:-1] + (k // BLOCK, BLOCK))
    amax_b = np.max(np.abs(blocks), axis=-1)
    if s_t > 0:
        scale_arg = amax_b / (6.0 * s_t)
    else:
        scale_arg = np.zeros_like(amax_b)
    if block_scales is None:
        sb = F.e4m3_rne(scale_arg)
    else:
        sb = np.asarray(block_scales, dtype=np.uint8).reshape(amax_b.shape)
    S = F.e4m3_decode(sb) * s_t                       # exact in float64
    safe = np.where(S > 0, S, 1.0)[..., None]
    q = np.where(S[..., None] > 0, blocks / safe, np.copysign(0.0, blocks))
    codes = F.e2m1_rne(q).reshape(y.shape)
    return codes, sb.astype(np.uint8), scale_arg, q.reshape(y.shape)


def quantize(x, hadamard=0, tensor_scale_value=None, block_scales=None):
    """NVFP4 of a 2-D tensor [M, K] with an optional block Hadamard rotation first.

    Returns a dict with `packed` [M, K/2] u8, `codes` [M, K] u8, `scales` [M, K/16] u8
    (E4M3 bits), `tensor_scale` (np.float32), the rotated values `y` and the decision
    arguments `scale_arg` (amax_b / 6 s_t) and `elem_arg` (y / (s_b s_t)).
    """
    y = rotate(np.asarray(x, dtype=np.float64), hadamard)
    s_t = tensor_scale(y) if tensor_scale_value is None else np.float32(tensor_scale_value)
    codes, sb, scale_arg, q = quantize_blocks(y, s_t, block_scales)
    return dict(packed=F.pack_nibbles(codes), codes=codes, scales=sb,
                tensor_scale=np.float32(s_t), y=y, scale_arg=scale_arg, elem_arg=q)


def dequantize_exact(codes, scales, s_t):
    """Real value V(c) * s_b * s_t of unpacked codes (float64, exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    k = codes.shape[-1]
    sb = F.e4m3_decode(np.asarray(scales, dtype=np.uint8))
    v = F.e2m1_decode(codes).reshape(codes.shape[:-1] + (k // BLOCK, BLOCK))
    return (v * sb[..., None] * float(np.float32(s_t))).reshape(codes.shape)


def dequantize(packed, scales, s_t, inverse_hadamard=0):
    """fl32(V * s_b * s_t) per element, then the optional inverse rotation (float64).

    Returns float64 values: the binary32 dequantized values when inverse_hadamard = 0,
    else H applied (in float64) to those binary32 values.
    """
    codes = F.unpack_nibbles(packed)
    xq = F.to_f32(dequantize_exact(codes, scales, s_t)).astype(np.float64)
    return rotate(xq, inverse_hadamard)
