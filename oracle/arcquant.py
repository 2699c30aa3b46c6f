"""ARCQuant activation path: RMSNorm, channel reorder, primary NVFP4 and residual NVFP4.

TEST INFRASTRUCTURE: part of the CPU oracle (see oracle/__init__.py).

Follows the ARCQuant technical summary (gist.science/fr/paper/2601.07475), Méthodologie:
* item 1: channels are reordered by their absolute maxima (the order comes from
  calibration data and reaches this function as the permutation `perm`; the subset S
  is the first S channels of that order);
* item 2, primary stage: the reordered activations are quantized with standard block
  NVFP4;  residual stage: for the outlier channels the residual (original value minus
  the primary quantized value) is quantized separately into a second set of NVFP4
  channels;
* item 3: the residual channels are concatenated to the primary ones along the
  reduction dimension K;
* item 5: one fused kernel does the reorder, the RMSNorm, the primary and the residual
  quantization and emits the GEMM-ready layout.

Readings where the summary is silent: RMSNorm y = x / sqrt(mean(x^2) + eps) * gamma,
applied before the reorder (z[:, c] = y[:, perm[c]]); one tensor scale s_t shared by
the primary and residual channels (so the extended GEMM has a single global factor),
computed from max|z| like oracle/nvfp4.tensor_scale or given; the residual is taken
against the exact real value of the primary quantization; output rows are the plain
concatenation [K primary | S residual] for codes and for scales.
"""
import numpy as np

from . import mxfp4, nvfp4
from . import formats as F

BLOCK = nvfp4.BLOCK


def rmsnorm(x, gamma=None, eps=1e-6):
    """y = x / sqrt(mean(x^2) + eps) * gamma, per row, float64."""
    x = np.asarray(x, dtype=np.float64)
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x / rms
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    return y


def quantize(x, perm, S, gamma=None, eps=1e-6, tensor_scale_value=None,
             primary_scales=None, primary_codes=None, residual_scales=None, z=None):
    """Fused ARCQuant activation quantization of [M, K] into the [K | S] layout.

    The optional overrides replace a decision by a given one (E4M3 codes for the
    scales, unpacked codes for the primary elements), so that each later decision can
    be checked against the oracle given the earlier ones; `z` replaces the normalized,
    reordered values [M, K] (the steps from the tensor scale on are unchanged).

    Returns `packed` [M, (K+S)/2], `scales` [M, (K+S)/16] (E4M3), `tensor_scale`, the
    normalized-and-reordered values `z`, and per stage the codes and decision
    arguments: `primary` and `residual` dicts as from nvfp4.quantize_blocks.
    """
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    perm = np.asarray(perm, dtype=np.int64)
    assert sorted(perm.tolist()) == list(range(K)), "perm must be a permutation of 0..K-1"
    assert S % BLOCK == 0 and 0 <= S <= K and K % BLOCK == 0
    z = rmsnorm(x, gamma, eps)[:, perm] if z is None else np.asarray(z, dtype=np.float64).reshape(M, K)
    s_t = nvfp4.tensor_scale(z) if tensor_scale_value is None else np.float32(tensor_scale_value)
    pc, psb, parg, pq = nvfp4.quantize_blocks(z, s_t, primary_scales)
    if primary_codes is not None:
        pc = np.asarray(primary_codes, dtype=np.uint8).reshape(M, K)
    xhat = nvfp4.dequantize_exact(pc, psb, s_t)
    r = z[:, :S] - xhat[:, :S]
    if S > 0:
        rc, rsb, rarg, rq = nvfp4.quantize_blocks(r, s_t, residual_scales)
    else:
        rc = np.zeros((M, 0), np.uint8)
        rsb = np.zeros((M, 0), np.uint8)
        rarg = rq = np.zeros((M, 0))
    codes = np.concatenate([pc, rc], axis=1)
    scales = np.concatenate([psb, rsb], axis=1)
    return dict(packed=F.pack_nibbles(codes), codes=codes, scales=scales.astype(np.uint8),
                tensor_scale=np.float32(s_t), z=z, residual_value=r,
                primary=dict(codes=pc, scales=psb, scale_arg=parg, elem_arg=pq),
                residual=dict(codes=rc, scales=rsb, scale_arg=rarg, elem_arg=rq))


def dequantize(packed, scales, s_t, K, S):
    """Real values of the primary [M, K] and residual [M, S] parts (float64, exact)."""
    codes = F.unpack_nibbles(packed)
    p = nvfp4.dequantize_exact(codes[:, :K], scales[:, :K // BLOCK], s_t)
    r = nvfp4.dequantize_exact(codes[:, K:K + S], scales[:, K // BLOCK:], s_t)
    return p, r


def quantize_mx(x, perm, S, gamma=None, eps=1e-6, primary_scales=None, primary_codes=None,
                residual_scales=None, z=None):
    """MXFP4 flavour of the fused activation quantization, [K | S] layout.

    The ARCQuant summary (Résultats Expérimentaux, Généralisabilité) reports that the
    augmented-residual scheme extends to MXFP4; its Méthodologie items 2-3 give the two
    stages.  Same steps as quantize() with MXFP4 in place of NVFP4: primary = MXFP4 (E8M0
    per 32, oracle/mxfp4.py) of the reordered normalized z; residual = z - the exact value
    of the primary quantization on the first S channels, quantized with its own E8M0
    block scales.  There is no tensor scale.  S and K are multiples of 32.

    Overrides replace decisions (and `z` the normalized, reordered values) by given ones,
    as in quantize().  Returns `packed`
    [M, (K+S)/2], `scales` [M, (K+S)/32] (E8M0), `z`, `residual_value`, and `primary` /
    `residual` dicts with codes, scales, block maxima `amax` and element arguments.
    """
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    perm = np.asarray(perm, dtype=np.int64)
    assert sorted(perm.tolist()) == list(range(K)), "perm must be a permutation of 0..K-1"
    B = mxfp4.BLOCK
    assert S % B == 0 and 0 <= S <= K and K % B == 0
    z = rmsnorm(x, gamma, eps)[:, perm] if z is None else np.asarray(z, dtype=np.float64).reshape(M, K)
    p = mxfp4.quantize(z, 0, primary_scales)
    pc = p["codes"] if primary_codes is None else np.asarray(primary_codes, dtype=np.uint8).reshape(M, K)
    xhat = mxfp4.dequantize_exact(pc, p["scales"])
    r = z[:, :S] - xhat[:, :S]
    if S > 0:
        q = mxfp4.quantize(r, 0, residual_scales)
        rc, rs, ramax, rarg = q["codes"], q["scales"], q["amax"], q["elem_arg"]
    else:
        rc = np.zeros((M, 0), np.uint8)
        rs = np.zeros((M, 0), np.uint8)
        ramax = rarg = np.zeros((M, 0))
    codes = np.concatenate([pc, rc], axis=1)
    scales = np.concatenate([p["scales"], rs], axis=1)
    return dict(packed=F.pack_nibbles(codes), codes=codes, scales=scales.astype(np.uint8), z=z,
                residual_value=r,
                primary=dict(codes=pc, scales=p["scales"], amax=p["amax"], elem_arg=p["elem_arg"]),
                residual=dict(codes=rc, scales=rs, amax=ramax, elem_arg=rarg))


def dequantize_mx(packed, scales, K, S):
    """Real values of the MXFP4 primary [M, K] and residual [M, S] parts (float64, exact)."""
    codes = F.unpack_nibbles(packed)
    B = mxfp4.BLOCK
    p = mxfp4.dequantize_exact(codes[:, :K], scales[:, :K // B])
    r = mxfp4.dequantize_exact(codes[:, K:K + S], scales[:, K // B:])
    return p, r
