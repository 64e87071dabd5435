"""Pins for oracle.attend (decode output over compressed values)."""

from __future__ import annotations

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import synth
from oracle import attend as oa
from oracle.codebook import codebook_fp32


def random_case(seed, B=3, S=50, D=16, C=4):
    rng = np.random.default_rng(seed)
    Pi_v = synth.haar_rotation(rng, D).astype(np.float64)
    cb = np.sort(rng.standard_normal(C)) / np.sqrt(D)
    idx = rng.integers(0, C, (S, D)).astype(np.uint8)
    norm = rng.uniform(0.5, 3.0, S)
    scores = rng.standard_normal((B, S)) * 3
    return scores, idx, norm, Pi_v, cb


def test_hand_example():
    # D = 2, Pi_v = I, codebook [-0.5, 0.5]; value 1: idx [1, 0], norm 2 -> [1, -1];
    # value 2: idx [1, 1], norm 4 -> [2, 2]; scores [0, ln 3] give weights [1/4, 3/4]
    scores = np.array([[0.0, np.log(3.0)]])
    idx = np.array([[1, 0], [1, 1]], np.uint8)
    norm = np.array([2.0, 4.0])
    cb = np.array([-0.5, 0.5])
    for f in (oa.attend_explicit, oa.attend_rotated):
        np.testing.assert_allclose(f(scores, idx, norm, np.eye(2), cb, 1.0), [[1.75, 1.25]], rtol=0, atol=1e-14)


def test_rotated_domain_equals_explicit():
    for seed in range(5):
        scores, idx, norm, Pi_v, cb = random_case(seed)
        a = oa.attend_explicit(scores, idx, norm, Pi_v, cb, 0.7)
        b = oa.attend_rotated(scores, idx, norm, Pi_v, cb, 0.7)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_uniform_scores_and_zero_scale_give_the_mean():
    scores, idx, norm, Pi_v, cb = random_case(1)
    v_hat = oa.dequantize_values(idx, norm, Pi_v, cb)
    mean = v_hat.mean(axis=0)
    flat = np.full_like(scores, 2.5)
    for s, scale in ((flat, 1.0), (scores, 0.0)):
        out = oa.attend_rotated(s, idx, norm, Pi_v, cb, scale)
        np.testing.assert_allclose(out, np.broadcast_to(mean, out.shape), rtol=0, atol=1e-13)


def test_dominant_score_selects_its_value():
    scores, idx, norm, Pi_v, cb = random_case(2)
    scores[:, 17] = 1e3
    v_hat = oa.dequantize_values(idx, norm, Pi_v, cb)
    out = oa.attend_rotated(scores, idx, norm, Pi_v, cb, 1.0)
    np.testing.assert_allclose(out, np.broadcast_to(v_hat[17], out.shape), rtol=0, atol=1e-12)


def test_shift_invariance_and_weights():
    scores, idx, norm, Pi_v, cb = random_case(3)
    a = oa.attend_rotated(scores, idx, norm, Pi_v, cb, 0.9)
    b = oa.attend_rotated(scores + 123.0, idx, norm, Pi_v, cb, 0.9)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    p = oa.softmax_weights(scores, 0.9)
    np.testing.assert_allclose(p, scipy_softmax(0.9 * scores, axis=-1), rtol=1e-13, atol=0)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("cuts", [(10, 20), (1, 49), (25,), (5, 6, 30, 44)])
def test_split_ranges_combine_to_the_full_softmax(cuts):
    scores, idx, norm, Pi_v, cb = random_case(4)
    edges = (0,) + tuple(cuts) + (scores.shape[1],)
    parts = [oa.partial_state(scores[:, a:b], idx[a:b], norm[a:b], cb, 1.3) for a, b in zip(edges, edges[1:])]
    np.testing.assert_allclose(oa.combine_partials(parts, Pi_v), oa.attend_rotated(scores, idx, norm, Pi_v, cb, 1.3),
                               rtol=0, atol=1e-13)


def test_compress_values_norm_and_nearest_centroid():
    rng = np.random.default_rng(5)
    D, C = 16, 4
    Pi_v = np.linalg.qr(rng.standard_normal((D, D)))[0]    # orthogonal in float64 (no fp32 rounding)
    cb = codebook_fp32(D, C).astype(np.float64)
    v = rng.standard_normal((40, D)) * rng.uniform(0.1, 5.0, (40, 1))
    v[3] = 0.0
    idx, norm = oa.compress_values(v, Pi_v, cb)
    np.testing.assert_allclose(norm, np.linalg.norm(v, axis=1), rtol=1e-15, atol=0)
    unit = v / np.where(norm > 0, norm, 1.0)[:, None]
    y = unit @ Pi_v.T
    brute = np.argmin(np.abs(y[..., None] - cb[None, None, :]), axis=-1)   # ties cannot occur here
    np.testing.assert_array_equal(idx, brute)
    # the dequantized vector keeps the stored norm's scale: ||v_hat|| = norm * ||c[idx]||
    v_hat = oa.dequantize_values(idx, norm, Pi_v, cb)
    np.testing.assert_allclose(np.linalg.norm(v_hat, axis=1), norm * np.linalg.norm(cb[idx], axis=1), rtol=1e-13)
