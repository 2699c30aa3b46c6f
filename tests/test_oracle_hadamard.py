"""Pins of the oracle's Hadamard rotations: scipy's Sylvester construction, closed forms
of single entries, orthogonality, energy, involution and the Kronecker identity of the
two-level 16 x 8 transform."""
import numpy as np
import pytest
import scipy.linalg

from oracle import hadamard as H


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_sylvester_matches_scipy_and_is_orthonormal(n):
    h = H.sylvester(n)
    assert np.allclose(h, scipy.linalg.hadamard(n) / np.sqrt(n), atol=0, rtol=1e-15)
    assert np.allclose(h @ h.T, np.eye(n), atol=1e-14)


@pytest.mark.parametrize("n", [16, 32, 128])
def test_sylvester_entry_closed_form(n):
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    popc = np.vectorize(lambda v: bin(v).count("1"))(i & j)
    assert np.array_equal(H.sylvester(n) * np.sqrt(n), (-1.0) ** popc)


@pytest.mark.parametrize("n", [16, 32])
def test_block_rotate_closed_forms(n):
    k = 4 * n
    # a delta at index b*n + j maps to column j of H inside block b only
    x = np.zeros((1, k))
    x[0, 2 * n + 3] = 1.0
    y = H.block_rotate(x, n)
    expect = np.zeros(k)
    expect[2 * n:3 * n] = H.sylvester(n)[:, 3]
    assert np.allclose(y[0], expect, atol=1e-15)
    # a constant block c maps to (sqrt(n) c, 0, ..., 0)
    y = H.block_rotate(np.full((1, k), 2.5), n)
    for b in range(4):
        assert abs(y[0, b * n] - np.sqrt(n) * 2.5) < 1e-12
        assert np.allclose(y[0, b * n + 1:(b + 1) * n], 0, atol=1e-12)


@pytest.mark.parametrize("n", [16, 32, 128])
def test_energy_and_involution(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((8, 4 * 128))
    y = H.rotate(x, n)
    blocks_x = x.reshape(8, -1, n)
    blocks_y = y.reshape(8, -1, n)
    assert np.allclose(np.linalg.norm(blocks_x, axis=-1), np.linalg.norm(blocks_y, axis=-1), rtol=1e-13)
    assert np.allclose(H.rotate(y, n), x, atol=1e-12)


def test_two_level_equals_kronecker_and_h128():
    assert np.allclose(np.kron(H.sylvester(8), H.sylvester(16)), H.sylvester(128), atol=1e-15)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 256))
    assert np.allclose(H.two_level_128(x), H.block_rotate(x, 128), atol=1e-13)
    # level 1 alone is H16 per micro-group: check on an input that level 2 leaves alone
    # (only micro-group 0 non-zero -> level 2 spreads it with +1/sqrt(8) to all groups)
    x = np.zeros((1, 128))
    x[0, :16] = rng.standard_normal(16)
    y = H.two_level_128(x)
    h16 = H.block_rotate(x[:, :16], 16)[0]
    for g in range(8):
        assert np.allclose(y[0, 16 * g:16 * g + 16], h16 / np.sqrt(8), atol=1e-14)


def test_identity_rotation():
    x = np.arange(64.0).reshape(2, 32)
    assert np.array_equal(H.rotate(x, 0), x)
