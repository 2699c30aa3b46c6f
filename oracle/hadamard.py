"""Block Hadamard rotations, in float64.

TEST INFRASTRUCTURE: part of the CPU oracle (see oracle/__init__.py).

* Block Hadamard transforms applied before FP4 quantization: MR-GPTQ abstract
  (hyper.ai, Résumé: "transformations de Hadamard par blocs", rotation fused into the
  weights offline and applied online to the activations).
* Hybrid two-level FWHT: FP4Quant abstract (paperdot.bitmofang.com), which names a
  two-level fast Walsh-Hadamard pipeline ahead of micro-grouped FP4 quantization.  The
  split used here is 16 within a micro-group, then 8 across the micro-groups of one
  128-element group.

The pages give neither the ordering, the normalisation nor sign randomisation.  Read
here: Sylvester ordering (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]), scaled by
1/sqrt(n) so that H H^T = I, no random signs, blocks contiguous along the last axis
starting at index 0.  H is symmetric and orthogonal, so it is its own inverse.
"""
import numpy as np


def sylvester(n):
    """Orthonormal Sylvester-Hadamard matrix of order n (a power of two), float64."""
    assert n >= 1 and (n & (n - 1)) == 0, "order must be a power of two"
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(n)


def block_rotate(x, n):
    """y = H_n x on every contiguous n-block of the last axis (n = 0 or 1: identity)."""
    x = np.asarray(x, dtype=np.float64)
    if n in (0, 1):
        return x.copy()
    k = x.shape[-1]
    assert k % n == 0, "last axis must be a multiple of the block"
    blocks = x.reshape(x.shape[:-1] + (k // n, n))
    h = sylvester(n)
    return (blocks @ h.T).reshape(x.shape)


def two_level_128(x):
    """Two-level FWHT of every 128-group: H_16 inside each of the 8 micro-groups of 16,
    then H_8 across the 8 micro-groups at each fixed in-group position.

    Element j of micro-group g sits at index 16 g + j of the group.  Each level is
    orthonormal, so the whole is orthonormal (it equals H_8 (x) H_16 = H_128).
    """
    x = np.asarray(x, dtype=np.float64)
    k = x.shape[-1]
    assert k % 128 == 0, "last axis must be a multiple of 128"
    g = x.reshape(x.shape[:-1] + (k // 128, 8, 16))
    level1 = g @ sylvester(16).T                                   # within micro-groups
    level2 = np.swapaxes(np.swapaxes(level1, -1, -2) @ sylvester(8).T, -1, -2)  # across
    return level2.reshape(x.shape)


def rotate(x, hadamard):
    """Dispatch on the rotation kind used by the quantizers: 0 (none), 16, 32, or 128
    (the two-level 16 x 8 transform)."""
    if hadamard == 128:
        return two_level_128(x)
    return block_rotate(x, hadamard)
