"""Pins of the oracle's 128-point rotation (CPU only)."""

import numpy as np
import pytest
import scipy.linalg

from oracle import hadamard


def test_matches_scipy_sylvester():
    ref = scipy.linalg.hadamard(128).astype(np.float64) / np.sqrt(128)
    assert np.allclose(hadamard.hadamard_matrix(), ref, rtol=0, atol=1e-15)


def test_involution_and_orthonormal():
    H = hadamard.hadamard_matrix()
    assert np.allclose(H @ H, np.eye(128), atol=1e-13)
    v = np.random.default_rng(0).standard_normal((5, 384))
    assert np.allclose(hadamard.rotate_blocks(hadamard.rotate_blocks(v)), v,
                       atol=1e-12)
    assert np.allclose(np.linalg.norm(hadamard.rotate_blocks(v), axis=1),
                       np.linalg.norm(v, axis=1), rtol=1e-13)


def test_blocks_are_independent_and_contiguous():
    # a unit vector in block b maps to a row of H inside block b only
    ref = scipy.linalg.hadamard(128) / np.sqrt(128)
    for b, j in ((0, 0), (1, 5), (2, 127)):
        v = np.zeros(384)
        v[128 * b + j] = 1.0
        out = hadamard.rotate_blocks(v)
        expect = np.zeros(384)
        expect[128 * b:128 * b + 128] = ref[j]
        assert np.allclose(out, expect, atol=1e-15)


def test_constant_block_maps_to_dc():
    out = hadamard.rotate_blocks(np.full(128, 3.0))
    assert out[0] == pytest.approx(3.0 * np.sqrt(128))
    assert np.all(np.abs(out[1:]) < 1e-13)


def test_rejects_ragged_dimension():
    with pytest.raises(ValueError):
        hadamard.rotate_blocks(np.zeros(200))
