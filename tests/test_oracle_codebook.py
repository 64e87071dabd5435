"""Pins for the oracle's Lloyd-Max codebooks (CPU only).

Against the table the codebook page prints, the paper's bounds, the closed
1-bit centroid, and the Lloyd fixed-point conditions evaluated with scipy's
exact normal distribution and numerical quadrature (independent of the grid).
"""

import math

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import codebook as ocb


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_sphere_table_from_page(golden, bits):
    g = golden("lloyd_sphere_d128.json")
    d = g["d"]
    c, edges, mse = ocb.lloyd_max(d, bits, "sphere")
    assert round(mse, g["d_mse_decimals"]) == pytest.approx(g["d_mse"][str(bits)], abs=1e-12)
    if str(bits) in g["centroids_times_sqrt_d"]:
        np.testing.assert_array_equal(np.round(c * math.sqrt(d), g["centroid_decimals"]),
                                      g["centroids_times_sqrt_d"][str(bits)])
    assert g["lower_bound"][str(bits)] < mse < g["upper_bound"][str(bits)]
    assert mse == pytest.approx(g["paper_expected"][str(bits)], rel=0.15)
    np.testing.assert_allclose(edges, 0.5 * (c[1:] + c[:-1]), rtol=0, atol=0)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_bounds_formula(golden, bits):
    g = golden("lloyd_sphere_d128.json")
    assert round(4.0 ** -bits, 4) == g["lower_bound"][str(bits)]
    assert round(math.sqrt(3) * math.pi / 2 * 4.0 ** -bits, 4) == g["upper_bound"][str(bits)]


@pytest.mark.parametrize("d", [32, 128])
def test_gaussian_one_bit_closed_form(d):
    c, _, mse = ocb.lloyd_max(d, 1, "gaussian")
    # the 400,001-point grid resolves centroids to about 1e-5 relative
    np.testing.assert_allclose(c, [-math.sqrt(2 / math.pi / d), math.sqrt(2 / math.pi / d)], rtol=3e-5)
    assert mse == pytest.approx(1 - 2 / math.pi, rel=1e-5)


@pytest.mark.parametrize("d,bits", [(32, 2), (128, 2), (128, 3), (32, 3)])
def test_gaussian_lloyd_fixed_point(d, bits):
    """Each centroid is the exact conditional mean of N(0, 1/d) on its cell."""
    c, edges, mse = ocb.lloyd_max(d, bits, "gaussian")
    sd = 1 / math.sqrt(d)
    lo = np.concatenate([[-np.inf], edges]) / sd
    hi = np.concatenate([edges, [np.inf]]) / sd
    mass = stats.norm.cdf(hi) - stats.norm.cdf(lo)
    cond_mean = sd * (stats.norm.pdf(lo) - stats.norm.pdf(hi)) / mass
    # 300 fixed iterations leave a ~3e-5 relative residual at 8 levels; a wrong
    # density or cell rule moves centroids by more than 1e-3
    np.testing.assert_allclose(c, cond_mean, rtol=8e-5, atol=1e-8)
    # model MSE against the exact integral of the squared error
    exact = 0.0
    for k in range(len(c)):
        f = lambda x, ck=c[k]: (x - ck) ** 2 * stats.norm.pdf(x, scale=sd)
        a = -np.inf if k == 0 else edges[k - 1]
        b = np.inf if k == len(c) - 1 else edges[k]
        exact += integrate.quad(f, a, b)[0]
    assert mse == pytest.approx(d * exact, rel=1e-4)


def test_gaussian_two_and_three_bit_textbook_levels():
    """Max's Gaussian quantizer levels (unit variance): 4 levels +-0.4528, +-1.510;
    8 levels +-0.2451, +-0.7560, +-1.344, +-2.152; MSE 0.1175 and 0.03455."""
    c2, _, m2 = ocb.lloyd_max(128, 2, "gaussian")
    c3, _, m3 = ocb.lloyd_max(128, 3, "gaussian")
    s = math.sqrt(128)
    np.testing.assert_allclose(np.abs(c2 * s), [1.510, 0.4528, 0.4528, 1.510], atol=1.5e-3)
    np.testing.assert_allclose(np.abs(c3 * s), [2.152, 1.344, 0.7560, 0.2451, 0.2451, 0.7560, 1.344, 2.152],
                               atol=1.5e-3)
    assert m2 == pytest.approx(0.1175, abs=2e-4)
    assert m3 == pytest.approx(0.03455, abs=1e-4)


def test_sphere_lloyd_fixed_point_quadrature():
    d, bits = 128, 2
    c, edges, _ = ocb.lloyd_max(d, bits, "sphere")
    f = lambda x: (1 - x * x) ** ((d - 3) / 2)
    bounds = np.concatenate([[-1.0], edges, [1.0]])
    for k in range(len(c)):
        m0 = integrate.quad(f, bounds[k], bounds[k + 1], epsabs=0, epsrel=1e-12)[0]
        m1 = integrate.quad(lambda x: x * f(x), bounds[k], bounds[k + 1], epsabs=0, epsrel=1e-12)[0]
        assert c[k] == pytest.approx(m1 / m0, rel=2e-5)


def test_codebook_fp32_is_float32_sorted():
    cb = ocb.codebook_fp32(128, 8)
    assert cb.dtype == np.float32 and cb.shape == (8,)
    assert np.all(np.diff(cb) > 0)
    with pytest.raises(ValueError):
        ocb.codebook_fp32(128, 6)
