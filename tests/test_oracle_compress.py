"""Pins for the oracle's TurboQuant_prod compressor (CPU only).

Nearest-centroid assignment against brute force; MSE distortion against the
model, the paper's bounds and the page's Haar round-trip numbers; the 1-bit
shrinkage closed form; and unbiasedness of the full (MSE + QJL) inner-product
estimate over random projections, with its closed-form variance. The last test
also shows the check has power: without the QJL term the estimate is biased.
"""

import math

import numpy as np
import pytest
from scipy.special import gammaln

import synth
from oracle import codebook as ocb
from oracle import compress as ocp
from oracle import score as osc


def test_nearest_indices_brute_force():
    rng = np.random.default_rng(20)
    cb = ocb.codebook_fp32(128, 8).astype(np.float64)
    y = rng.standard_normal((500, 128)) / math.sqrt(128)
    got = ocp.nearest_indices(y, cb)
    brute = np.argmin(np.abs(y[..., None] - cb[None, None, :]), axis=-1)
    np.testing.assert_array_equal(got, brute)


def test_tie_takes_lower_index():
    cb = np.array([-1.0, -0.25, 0.5, 2.0])
    y = np.array([[-0.625, 0.125, 1.25, 5.0, -7.0]])
    np.testing.assert_array_equal(ocp.nearest_indices(y, cb), [[0, 1, 2, 3, 0]])


def test_signs_are_plus_minus_one_and_gamma_is_residual_length():
    rng = np.random.default_rng(21)
    D = 32
    Pi = synth.haar_rotation(rng, D)
    S_mat = synth.gaussian_projection(rng, D)
    cb = ocb.codebook_fp32(D, 4)
    k = synth.unit_keys(rng, 200, D, "uniform")
    idx, sign, gamma = ocp.quantize_prod_unit(k, Pi, S_mat, cb)
    assert set(np.unique(sign)) <= {-1, 1}
    # gamma^2 = ||k||^2 - 2<k, x_mse> + ||x_mse||^2, expanded without forming r
    xm = cb.astype(np.float64)[idx] @ Pi.astype(np.float64)
    g2 = 1.0 - 2 * np.einsum("sd,sd->s", k, xm) + np.einsum("sd,sd->s", xm, xm)
    np.testing.assert_allclose(gamma ** 2, g2, atol=1e-12)
    # sign agrees with the projection of the residual row by row
    for s in range(0, 200, 37):
        r = k[s] - xm[s]
        for i in range(0, D, 5):
            pr = float(np.dot(S_mat[i].astype(np.float64), r))
            assert sign[s, i] == (1 if pr >= 0 else -1)


@pytest.mark.slow
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_distortion_model_and_bounds(golden, bits):
    g = golden("lloyd_sphere_d128.json")
    d = 128
    rng = np.random.default_rng(22 + bits)
    Pi = synth.haar_rotation(rng, d)
    c, _, model = ocb.lloyd_max(d, bits, "sphere")
    u = synth.unit_keys(rng, 8000, d, "uniform")
    idx = ocp.quantize_mse_unit(u, Pi, c)
    err = np.mean(np.sum((u - ocp.dequantize_mse(idx, Pi, c)) ** 2, axis=1))
    assert g["lower_bound"][str(bits)] < err < g["upper_bound"][str(bits)]
    assert err == pytest.approx(model, rel=0.02)
    if str(bits) in g["haar_roundtrip_isotropic"]:
        assert err == pytest.approx(g["haar_roundtrip_isotropic"][str(bits)], rel=0.01)


@pytest.mark.slow
def test_one_bit_shrinkage_closed_form():
    """1-bit MSE quantization over Haar rotations scales <x_hat, x> by d (E|y_1|)^2 ~ 2/pi,
    with E|y_1| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)) for a coordinate of a unit vector."""
    d = 64
    e_abs = math.exp(gammaln(d / 2) - gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    c, _, _ = ocb.lloyd_max(d, 1, "sphere")
    assert c[1] == pytest.approx(e_abs, rel=3e-5)       # grid resolution
    rng = np.random.default_rng(23)
    x = synth.unit_keys(rng, 1, d, "uniform")
    vals = []
    for _ in range(1500):
        Pi = synth.haar_rotation(rng, d).astype(np.float64)
        xh = ocp.dequantize_mse(ocp.quantize_mse_unit(x, Pi, c), Pi, c)
        vals.append(float(xh[0] @ x[0]))
    slope = float(np.mean(vals))
    assert slope == pytest.approx(d * e_abs ** 2, rel=2e-3)
    assert slope == pytest.approx(2 / math.pi, rel=0.01)


def _qjl_trials(q, k, Pi, cb, rng, M, D, with_qjl=True):
    est = np.empty(M)
    for m in range(M):
        S_mat = rng.standard_normal((D, D))
        idx, sign, gamma = ocp.quantize_prod_unit(k[None], Pi, S_mat, cb)
        g = gamma if with_qjl else np.zeros(1)
        est[m] = osc.scores_by_reconstruction(q[None], idx, sign, g, Pi, S_mat, cb)[0, 0]
    return est, idx, gamma


@pytest.mark.slow
def test_inner_product_unbiased_over_projections():
    """E_S <q, k_hat> = <q, k>, Var = [(pi/2) gamma^2 |q|^2 - <q, r>^2] / D (D projection rows)."""
    D, M = 32, 20000
    rng = np.random.default_rng(24)
    Pi = synth.haar_rotation(rng, D).astype(np.float64)
    cb = ocb.codebook_fp32(D, 4).astype(np.float64)
    k = synth.unit_keys(rng, 1, D, "uniform")[0]
    r = k - ocp.dequantize_mse(ocp.quantize_mse_unit(k[None], Pi, cb), Pi, cb)[0]
    gamma = float(np.linalg.norm(r))
    q = 3.0 * r / gamma + 0.5 * k
    true = float(q @ k)
    var = ((math.pi / 2) * gamma ** 2 * float(q @ q) - float(q @ r) ** 2) / D
    est, _, _ = _qjl_trials(q, k, Pi, cb, rng, M, D)
    z = (est.mean() - true) / math.sqrt(var / M)
    assert abs(z) < 5.0
    assert est.var() == pytest.approx(var, rel=0.06)
    # the MSE stage alone is biased for this pair: the test can tell
    est0, _, _ = _qjl_trials(q, k, Pi, cb, rng, 200, D, with_qjl=False)
    assert abs(est0.mean() - true) > 50 * math.sqrt(var / M)


def test_normalise_then_compress():
    """quantize_prod divides by the length first: unit keys give quantize_prod_unit's
    codes and norm 1; a key scaled by any a > 0 gives the same codes and a times the
    norm; a zero key is the zero vector (indices of 0, gamma = 0) with norm 0."""
    rng = np.random.default_rng(31)
    D = 64
    Pi = synth.haar_rotation(rng, D)
    S_mat = synth.gaussian_projection(rng, D)
    cb = ocb.codebook_fp32(D, 4)
    k = synth.unit_keys(rng, 50, D, "outlier")
    i0, s0, g0 = ocp.quantize_prod_unit(k, Pi, S_mat, cb)
    i1, s1, g1, n1 = ocp.quantize_prod(k, Pi, S_mat, cb)
    np.testing.assert_array_equal(i1, i0)
    np.testing.assert_array_equal(s1, s0)
    np.testing.assert_allclose(g1, g0, rtol=1e-14)
    np.testing.assert_allclose(n1, 1.0, rtol=1e-14)
    scale = rng.uniform(0.01, 100.0, size=50)
    i2, s2, g2, n2 = ocp.quantize_prod(k * scale[:, None], Pi, S_mat, cb)
    np.testing.assert_array_equal(i2, i0)
    np.testing.assert_array_equal(s2, s0)
    np.testing.assert_allclose(g2, g0, rtol=1e-12)
    np.testing.assert_allclose(n2, scale, rtol=1e-14)
    iz, sz, gz, nz = ocp.quantize_prod(np.zeros((1, D)), Pi, S_mat, cb)
    np.testing.assert_array_equal(iz, ocp.nearest_indices(np.zeros((1, D)), cb))
    assert nz[0] == 0.0
    # the residual of the zero vector is minus the centroid rebuild
    np.testing.assert_allclose(gz[0], np.linalg.norm(ocp.dequantize_mse(iz, Pi, cb)[0]), rtol=1e-14)
