"""Pins for oracle.mse (MSE-only keys, norm correction, randomized Hadamard)."""

from __future__ import annotations

import numpy as np
import pytest
from scipy.linalg import hadamard

import synth
from oracle import mse as om
from oracle.codebook import codebook_fp32


@pytest.mark.parametrize("n", [1, 2, 4, 8, 32, 64, 128, 256])
def test_fwht_is_the_orthonormal_sylvester_hadamard(n):
    x = np.random.default_rng(n).standard_normal((5, n))
    np.testing.assert_allclose(om.fwht(x), x @ (hadamard(n) / np.sqrt(n)).T, rtol=0, atol=1e-12)


def test_fwht_small_cases_and_involution():
    a, b = 3.0, -1.5
    np.testing.assert_allclose(om.fwht(np.array([a, b])), [(a + b) / np.sqrt(2), (a - b) / np.sqrt(2)], atol=1e-15)
    # H_4 e_0 is the all-ones column over 2; H_4 e_3 alternates as +,-,-,+
    np.testing.assert_allclose(om.fwht(np.eye(4)[0]), [0.5, 0.5, 0.5, 0.5], atol=1e-15)
    np.testing.assert_allclose(om.fwht(np.eye(4)[3]), [0.5, -0.5, -0.5, 0.5], atol=1e-15)
    x = np.random.default_rng(1).standard_normal((3, 64))
    np.testing.assert_allclose(om.fwht(om.fwht(x)), x, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(om.fwht(x), axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    with pytest.raises(ValueError):
        om.fwht(np.ones(12))


def test_randomized_hadamard_round_trip_and_dense_form():
    rng = np.random.default_rng(2)
    D = 128
    signs = rng.choice([-1.0, 1.0], D)
    x = rng.standard_normal((7, D))
    y = om.hadamard_forward(x, signs)
    np.testing.assert_allclose(om.hadamard_inverse(y, signs), x, atol=1e-12)
    R = om.hadamard_rotation(signs)
    np.testing.assert_allclose(R, (hadamard(D) / np.sqrt(D)) @ np.diag(signs), atol=1e-14)
    np.testing.assert_allclose(R @ R.T, np.eye(D), atol=1e-13)
    np.testing.assert_allclose(x @ R.T, y, atol=1e-12)
    np.testing.assert_allclose(om.query_transform_hadamard(x, signs), y, atol=0)


def test_hand_example_d2():
    # Pi = H D with signs (1, -1): R = [[1, -1], [1, 1]] / sqrt(2). Key stored as
    # idx (1, 0), rho 2, codebook (-0.5, 0.5): c = (0.5, -0.5), k_hat = 2 R^T c
    # = 2 [[1, 1], [-1, 1]] (0.5, -0.5) / sqrt(2) = (0, -sqrt(2)). Query (3, 1):
    # score -sqrt(2); A = R q = (2, 4) / sqrt(2) and rho (A . c) = 2 (1 - 2) / sqrt(2).
    signs = np.array([1.0, -1.0])
    R = om.hadamard_rotation(signs)
    np.testing.assert_allclose(R, np.array([[1, -1], [1, 1]]) / np.sqrt(2), atol=1e-15)
    idx = np.array([[1, 0]], np.uint8)
    rho = np.array([2.0])
    cb = np.array([-0.5, 0.5])
    q = np.array([[3.0, 1.0]])
    np.testing.assert_allclose(om.dequantize_mse_keys(idx, rho, R, cb), [[0.0, -np.sqrt(2)]], atol=1e-15)
    np.testing.assert_allclose(om.scores_mse_by_reconstruction(q, idx, rho, R, cb), [[-np.sqrt(2)]], atol=1e-14)
    A = om.query_transform_hadamard(q, signs)
    np.testing.assert_allclose(A, [[np.sqrt(2), 2 * np.sqrt(2)]], atol=1e-14)
    np.testing.assert_allclose(om.scores_mse_from_transformed(A, idx, rho, cb), [[-np.sqrt(2)]], atol=1e-14)


@pytest.mark.parametrize("nc", [False, True])
def test_compress_mse_nearest_centroid_and_norms(nc):
    rng = np.random.default_rng(3)
    D, C = 64, 8
    signs = rng.choice([-1.0, 1.0], D)
    R = om.hadamard_rotation(signs)
    cb = codebook_fp32(D, C).astype(np.float64)
    k = rng.standard_normal((50, D)) * rng.uniform(0.1, 4.0, (50, 1))
    k[7] = 0.0
    idx, rho = om.compress_mse(k, R, cb, norm_correction=nc)
    norm = np.linalg.norm(k, axis=1)
    unit = k / np.where(norm > 0, norm, 1.0)[:, None]
    y = om.hadamard_forward(unit, signs)
    np.testing.assert_array_equal(idx, np.argmin(np.abs(y[..., None] - cb), axis=-1))
    k_hat = om.dequantize_mse_keys(idx, rho, R, cb)
    if nc:
        # the corrected codeword is back on the sphere: k_hat has the key's length
        np.testing.assert_allclose(np.linalg.norm(k_hat, axis=1), norm, rtol=1e-13, atol=1e-15)
    else:
        np.testing.assert_allclose(rho, norm, rtol=1e-15)
        c = cb[idx.astype(np.intp)]
        np.testing.assert_allclose(np.linalg.norm(k_hat, axis=1), norm * np.linalg.norm(c, axis=1), rtol=1e-13)


def test_transformed_scores_equal_reconstruction():
    rng = np.random.default_rng(4)
    D, C = 128, 4
    for rot in ("hadamard", "haar"):
        signs = rng.choice([-1.0, 1.0], D)
        Pi = om.hadamard_rotation(signs) if rot == "hadamard" else synth.haar_rotation(rng, D).astype(np.float64)
        cb = codebook_fp32(D, C).astype(np.float64)
        k = synth.unit_keys(rng, 40, D, "outlier") * rng.uniform(0.5, 2.0, (40, 1))
        idx, rho = om.compress_mse(k, Pi, cb, norm_correction=True)
        q = rng.standard_normal((6, D))
        A = q @ Pi.T if rot == "haar" else om.query_transform_hadamard(q, signs)
        np.testing.assert_allclose(om.scores_mse_from_transformed(A, idx, rho, cb),
                                   om.scores_mse_by_reconstruction(q, idx, rho, Pi, cb), rtol=0, atol=1e-12)


def test_norm_correction_removes_the_radial_shrinkage():
    """MSE codewords sit inside the sphere, so <k, k_hat> / ||k||^2 is below one
    (about 0.88 at 2 bits, section 6); the corrected reconstruction is longer and
    its slope is closer to one."""
    rng = np.random.default_rng(5)
    D, C = 128, 4
    signs = rng.choice([-1.0, 1.0], D)
    R = om.hadamard_rotation(signs)
    cb = codebook_fp32(D, C).astype(np.float64)
    k = synth.unit_keys(rng, 4000, D, "uniform")
    slopes = []
    for nc in (False, True):
        idx, rho = om.compress_mse(k, R, cb, norm_correction=nc)
        slopes.append(np.mean(np.sum(k * om.dequantize_mse_keys(idx, rho, R, cb), axis=1)))
    assert 0.86 < slopes[0] < 0.90
    assert slopes[0] < slopes[1] < 1.0
