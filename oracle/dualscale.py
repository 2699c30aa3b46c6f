"""FP4Quant-style micro-grouped dual-scale FP4 pack / unpack, in float64.

TEST INFRASTRUCTURE: part of the CPU oracle (see oracle/__init__.py).

The FP4Quant abstract (paperdot.bitmofang.com) names three parts: a micro-grouped
dual-scale FP4 quantization that keeps local distribution characteristics, a packed
sub-byte representation, and a hybrid two-level FWHT that lowers quantization error.
It gives no formats or layouts.  Reading taken here:

* rotation       two-level FWHT of every 128-group: H_16 in each micro-group of 16,
                 then H_8 across the 8 micro-groups (oracle/hadamard.py);
* coarse scale   one binary32 scale per 128-group, s_g = fl32(amax_g / 2688);
* fine scale     one E4M3 scale per 16-element micro-group,
                 s_m = E4M3_RNE(amax_m / (6 s_g)), 0 when s_g = 0 or amax_m = 0;
* codes          E2M1_RNE(y / (s_m s_g)), sign only when s_m s_g = 0;
* message        planar bytes: [codes, M*K/2][s_m, M*K/16][s_g, 4*M*K/128 LE binary32],
                 each section starting at a multiple of 256 bytes, 4.75 bits/element;
* unpack         y_hat = fl32(V * s_m * s_g), then the same two-level FWHT (its own
                 inverse), then the output type.

This is NVFP4's two-level scaling with the tensor scale moved down to the 128-group;
the decision arguments are evaluated in float64 exactly as in oracle/nvfp4.py.
"""
import numpy as np

from . import formats as F
from .hadamard import two_level_128
from .nvfp4 import TENSOR_SCALE_DIVISOR

GROUP = 128
MICRO = 16
SECTION_ALIGN = 256


def _align(n):
    return (n + SECTION_ALIGN - 1) // SECTION_ALIGN * SECTION_ALIGN


def layout(M, K):
    """Byte offsets of the three sections and the total size of the packed message."""
    codes = M * K // 2
    off_sm = _align(codes)
    off_sg = _align(off_sm + M * K // MICRO)
    total = _align(off_sg + 4 * (M * K // GROUP))
    return dict(codes=0, micro_scales=off_sm, group_scales=off_sg, total=total)


def pack_values(x, group_scales=None, micro_scales=None):
    """Quantize [M, K] (K a multiple of 128); returns codes, scales and decision arguments.

    `group_scales` ([M, K/128] binary32) and `micro_scales` ([M, K/16] E4M3 codes)
    override the computed values, so that later decisions can be checked given the
    earlier ones.
    """
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    assert K % GROUP == 0
    y = two_level_128(x)
    g = y.reshape(M, K // GROUP, GROUP)
    amax_g = np.max(np.abs(g), axis=-1)
    if group_scales is None:
        s_g = F.to_f32(amax_g / TENSOR_SCALE_DIVISOR)
    else:
        s_g = np.asarray(group_scales, dtype=np.float32).reshape(M, K // GROUP)
    s_g64 = s_g.astype(np.float64)
    m = g.reshape(M, K // GROUP, GROUP // MICRO, MICRO)
    amax_m = np.max(np.abs(m), axis=-1)
    sg_b = s_g64[..., None]
    scale_arg = np.where(sg_b > 0, amax_m / (6.0 * np.where(sg_b > 0, sg_b, 1.0)), 0.0)
    if micro_scales is None:
        s_m = F.e4m3_rne(scale_arg)
    else:
        s_m = np.asarray(micro_scales, dtype=np.uint8).reshape(amax_m.shape)
    S = F.e4m3_decode(s_m) * sg_b                              # exact
    q = np.where(S[..., None] > 0, m / np.where(S > 0, S, 1.0)[..., None],
                 np.copysign(0.0, m))
    codes = F.e2m1_rne(q).reshape(M, K)
    return dict(codes=codes, micro_scales=s_m.reshape(M, K // MICRO).astype(np.uint8),
                group_scales=s_g.reshape(M, K // GROUP), y=y, amax_g=amax_g,
                scale_arg=scale_arg.reshape(M, K // MICRO), elem_arg=q.reshape(M, K))


def pack(x):
    """The packed message (uint8 array of layout(M, K)['total'] bytes) for [M, K]."""
    M, K = np.shape(x)
    r = pack_values(x)
    lay = layout(M, K)
    buf = np.zeros(lay["total"], dtype=np.uint8)
    codes = F.pack_nibbles(r["codes"]).reshape(-1)
    buf[:codes.size] = codes
    sm = r["micro_scales"].reshape(-1)
    buf[lay["micro_scales"]:lay["micro_scales"] + sm.size] = sm
    sg = r["group_scales"].astype("<f4").reshape(-1).view(np.uint8)
    buf[lay["group_scales"]:lay["group_scales"] + sg.size] = sg
    return buf


def split(buf, M, K):
    """Codes [M, K] (unpacked), micro scales [M, K/16] and group scales [M, K/128]."""
    buf = np.asarray(buf, dtype=np.uint8)
    lay = layout(M, K)
    codes = F.unpack_nibbles(buf[:M * K // 2].reshape(M, K // 2))
    sm = buf[lay["micro_scales"]:lay["micro_scales"] + M * K // MICRO].reshape(M, K // MICRO)
    sg = buf[lay["group_scales"]:lay["group_scales"] + 4 * (M * K // GROUP)].copy()
    return codes, sm, sg.view("<f4").reshape(M, K // GROUP)


def dequantized(codes, micro_scales, group_scales):
    """y_hat = fl32(V * s_m * s_g) per element (V * s_m is exact), as float64."""
    M, K = codes.shape
    v = F.e2m1_decode(codes).reshape(M, K // MICRO, MICRO)
    sm = F.e4m3_decode(micro_scales).reshape(M, K // MICRO)
    sg = np.repeat(np.asarray(group_scales, dtype=np.float64), GROUP // MICRO, axis=1)
    return F.to_f32(v * (sm * sg)[..., None]).astype(np.float64).reshape(M, K)


def unpack(buf, M, K):
    """Reconstruction (float64) before the output-type rounding: FWHT of y_hat."""
    codes, sm, sg = split(buf, M, K)
    return two_level_128(dequantized(codes, sm, sg))
