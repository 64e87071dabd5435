"""The seeded generators: determinism, shapes and the stated distributions."""

import numpy as np

import synth


def test_deterministic_and_independent_streams():
    a = synth.head_matrices(5, 2, 16)
    b = synth.head_matrices(5, 2, 16)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    assert not np.array_equal(a[0][0], a[0][1])
    k0 = synth.unit_keys(synth.keys_rng(5, 0), 10, 16, "outlier")
    k1 = synth.unit_keys(synth.keys_rng(5, 1), 10, 16, "outlier")
    assert not np.array_equal(k0, k1)


def test_haar_rotation_is_orthogonal():
    Pi = synth.haar_rotation(np.random.default_rng(0), 128).astype(np.float64)
    np.testing.assert_allclose(Pi @ Pi.T, np.eye(128), atol=2e-6)


def test_unit_keys_and_outliers():
    k = synth.unit_keys(np.random.default_rng(1), 4000, 128, "outlier")
    np.testing.assert_allclose(np.linalg.norm(k, axis=1), 1.0, atol=1e-12)
    e = np.mean(k ** 2, axis=0)
    hot = list(synth.OUTLIER_CHANNELS)
    cold = [c for c in range(128) if c not in hot]
    # before normalising the four hot channels hold 4*225/(4*225+124) = 88% of the
    # expected energy; normalisation per key pulls the average share down a little
    assert 0.75 < e[hot].sum() < 0.9
    assert e[hot].min() > 100 * e[cold].mean()


def test_workload_table():
    w = synth.workload("decode")
    assert (w.B, w.S, w.D, w.C, w.layout) == (32, 32768, 128, 4, "unpacked")
    assert w.algorithmic_bytes() == 32768 * 260 + 32 * 32768 * 4 + 2 * 32 * 128 * 4 + 4 * 4
    g = synth.workload("gqa")
    assert g.P == 128 and g.H == 8 and g.B == 4 and g.key_bytes() == 128 * 32768 * 66


def test_timing_streams_are_valid_codes():
    idx, sign, gamma = synth.timing_code_streams(0, 2, 64, 32, 4, "unpacked", 2)
    assert idx.max() < 4 and set(np.unique(sign)) == {-1, 1} and gamma.dtype == np.float32
    idx, sign, gamma = synth.timing_code_streams(0, 1, 64, 128, 8, "packed", 3)
    assert idx.shape == (1, 64, 48) and sign.shape == (1, 64, 16) and gamma.dtype == np.float16
