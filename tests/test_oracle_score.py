"""Pins for the oracle's query transform and scorers (CPU only).

Each check ties the oracle to something other than itself: the numbers the
worked example prints, closed forms that special inputs reduce to, a scalar
brute force over every code of a tiny key, and algebraic invariants.
"""

import itertools
import math

import numpy as np
import pytest
from scipy.linalg import hadamard

from oracle import query_transform as oqt
from oracle import score as osc

COEF = math.sqrt(math.pi / 2.0)


def _ex(golden):
    g = golden("worked_example.json")
    arr = {k: np.array(v) for k, v in g.items() if isinstance(v, list)}
    return g, arr


def test_worked_example_query_transform(golden):
    g, a = _ex(golden)
    A, T = oqt.transform_one(a["q"], a["Pi"], a["S_mat"])
    np.testing.assert_array_equal(A, a["A"])
    np.testing.assert_array_equal(T, a["T"])


@pytest.mark.parametrize("route", ["reconstruction", "transformed"])
def test_worked_example_scores(golden, route):
    g, a = _ex(golden)
    if route == "reconstruction":
        s = osc.scores_by_reconstruction(a["q"], a["K_idx"], a["qjl_signs"], a["gamma"],
                                         a["Pi"], a["S_mat"], a["codebook"])
    else:
        A, T = oqt.transform_one(a["q"], a["Pi"], a["S_mat"])
        s = osc.scores_from_transformed(A, T, a["K_idx"], a["qjl_signs"], a["gamma"], a["codebook"])
    np.testing.assert_array_equal(np.round(s, g["decimals"]), a["scores"])


def test_worked_example_partial_terms(golden):
    """The page's intermediate terms: centroid scores, residual dots, token-0 correction."""
    g, a = _ex(golden)
    A, T = oqt.transform_one(a["q"], a["Pi"], a["S_mat"])
    zero_gamma = np.zeros(2)
    mse = osc.scores_from_transformed(A, T, a["K_idx"], a["qjl_signs"], zero_gamma, a["codebook"])
    np.testing.assert_allclose(mse[0], a["centroid_scores"], atol=1e-15)
    # with a zero codebook and gamma = D / sqrt(pi/2) the score is the bare residual dot
    unit_gamma = np.full(2, g["D"] / COEF)
    res = osc.scores_from_transformed(A, T, a["K_idx"], a["qjl_signs"], unit_gamma, np.zeros(4))
    np.testing.assert_allclose(res[0], a["residual_dots"], atol=1e-12)
    full = osc.scores_from_transformed(A, T, a["K_idx"], a["qjl_signs"], a["gamma"], a["codebook"])
    assert round(full[0, 0] - mse[0, 0], 6) == g["correction_token0"]


def test_gamma_example(golden):
    g = golden("gamma_example.json")
    assert round(float(np.linalg.norm(g["residual"])), g["decimals"]) == g["gamma"]


def _random_problem(rng, B, S, D, C):
    q = rng.standard_normal((B, D))
    Pi = np.linalg.qr(rng.standard_normal((D, D)))[0]
    S_mat = rng.standard_normal((D, D))
    cb = np.sort(rng.standard_normal(C)) / np.sqrt(D)
    idx = rng.integers(0, C, size=(S, D))
    sign = np.where(rng.integers(0, 2, size=(S, D)) == 1, 1, -1)
    gamma = rng.uniform(0.0, 1.0, size=S)
    return q, Pi, S_mat, cb, idx, sign, gamma


@pytest.mark.parametrize("B,S,D,C", [(1, 5, 2, 4), (3, 40, 7, 4), (5, 300, 32, 8), (4, 100, 128, 16)])
def test_query_side_identity(B, S, D, C):
    """Transforming the query gives the same scores as reconstructing every key."""
    rng = np.random.default_rng(100 + D)
    q, Pi, S_mat, cb, idx, sign, gamma = _random_problem(rng, B, S, D, C)
    ref = osc.scores_by_reconstruction(q, idx, sign, gamma, Pi, S_mat, cb, key_chunk=37)
    A, T = oqt.transform_one(q, Pi, S_mat)
    got = osc.scores_from_transformed(A, T, idx, sign, gamma, cb, key_chunk=53)
    assert np.max(np.abs(got - ref) / (1 + np.abs(ref))) < 1e-12


def test_identity_rotation_zero_gamma_is_gather_matmul():
    rng = np.random.default_rng(7)
    q, _, S_mat, cb, idx, sign, _ = _random_problem(rng, 3, 50, 16, 8)
    expect = q @ cb[idx].T
    for route in ("r", "t"):
        if route == "r":
            got = osc.scores_by_reconstruction(q, idx, sign, np.zeros(50), np.eye(16), S_mat, cb)
        else:
            A, T = oqt.transform_one(q, np.eye(16), S_mat)
            got = osc.scores_from_transformed(A, T, idx, sign, np.zeros(50), cb)
        np.testing.assert_allclose(got, expect, rtol=0, atol=1e-13)


def test_permutation_rotation():
    """Pi[d, perm[d]] = 1 makes A[b, d] = q[b, perm[d]]."""
    rng = np.random.default_rng(8)
    D = 12
    q, _, S_mat, cb, idx, sign, _ = _random_problem(rng, 2, 30, D, 4)
    perm = rng.permutation(D)
    Pi = np.zeros((D, D))
    Pi[np.arange(D), perm] = 1.0
    expect = q[:, perm] @ cb[idx].T
    got = osc.scores_by_reconstruction(q, idx, sign, np.zeros(30), Pi, S_mat, cb)
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-13)


@pytest.mark.parametrize("D", [4, 32, 128])
def test_hadamard_projection_closed_form(D):
    """Zero codebook, S_mat = Sylvester Hadamard H, sigma_s = row r_s of H:
    the key reconstructs to sqrt(pi/2) gamma_s e_{r_s}, so score = sqrt(pi/2) gamma_s q[b, r_s]."""
    rng = np.random.default_rng(9)
    H = hadamard(D).astype(np.float64)
    rows = rng.integers(0, D, size=20)
    sign = H[rows].astype(np.int64)
    gamma = rng.uniform(0.1, 1.0, size=20)
    q = rng.standard_normal((3, D))
    idx = rng.integers(0, 4, size=(20, D))
    Pi = np.linalg.qr(rng.standard_normal((D, D)))[0]
    expect = COEF * gamma[None, :] * q[:, rows]
    got = osc.scores_by_reconstruction(q, idx, sign, gamma, Pi, H, np.zeros(4))
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-12)
    A, T = oqt.transform_one(q, Pi, H)
    got2 = osc.scores_from_transformed(A, T, idx, sign, gamma, np.zeros(4))
    np.testing.assert_allclose(got2, expect, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("D", [2, 3])
def test_brute_force_every_code(D):
    """Every index and sign pattern of a tiny key, scored by scalar loops."""
    rng = np.random.default_rng(10 + D)
    C = 4
    q = rng.standard_normal((2, D))
    Pi = np.linalg.qr(rng.standard_normal((D, D)))[0]
    S_mat = rng.standard_normal((D, D))
    cb = np.array([-0.9, -0.2, 0.3, 1.1])
    codes = list(itertools.product(range(C), repeat=D))
    signs = list(itertools.product((-1, 1), repeat=D))
    keys = [(c, s) for c in codes for s in signs]
    idx = np.array([k[0] for k in keys])
    sign = np.array([k[1] for k in keys])
    gamma = np.linspace(0.05, 0.95, len(keys))
    expect = np.zeros((2, len(keys)))
    for j, (code, sg) in enumerate(keys):
        k_hat = [0.0] * D
        for i in range(D):
            acc = 0.0
            for d in range(D):
                acc += Pi[d][i] * cb[code[d]]
                acc += COEF / D * gamma[j] * S_mat[d][i] * sg[d]
            k_hat[i] = acc
        for b in range(2):
            expect[b, j] = sum(q[b][i] * k_hat[i] for i in range(D))
    got = osc.scores_by_reconstruction(q, idx, sign, gamma, Pi, S_mat, cb)
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-13)
    A, T = oqt.transform_one(q, Pi, S_mat)
    np.testing.assert_allclose(osc.scores_from_transformed(A, T, idx, sign, gamma, cb),
                               expect, rtol=1e-12, atol=1e-13)


def test_invariants():
    rng = np.random.default_rng(11)
    q, Pi, S_mat, cb, idx, sign, gamma = _random_problem(rng, 4, 60, 24, 8)
    f = lambda qq, cc=cb, ss=sign, gg=gamma: osc.scores_by_reconstruction(qq, idx, ss, gg, Pi, S_mat, cc)
    q2 = rng.standard_normal(q.shape)
    # linear in the query
    np.testing.assert_allclose(f(2.0 * q - 3.0 * q2), 2.0 * f(q) - 3.0 * f(q2), atol=1e-12)
    # negating the codebook and the signs negates the score
    np.testing.assert_allclose(f(q, -cb, -sign), -f(q), atol=1e-13)
    # affine in gamma: s(2g) = 2 s(g) - s(0)
    np.testing.assert_allclose(f(q, gg=2 * gamma), 2 * f(q) - f(q, gg=0 * gamma), atol=1e-12)


def test_batched_query_transform_uses_head_p_mod_H():
    rng = np.random.default_rng(12)
    P, H, B, D = 6, 3, 2, 8
    q = rng.standard_normal((P, B, D))
    Pi = rng.standard_normal((H, D, D))
    S_mat = rng.standard_normal((H, D, D))
    A, T = oqt.query_transform(q, Pi, S_mat)
    for p in range(P):
        for b in range(B):
            for d in range(D):
                assert abs(A[p, b, d] - sum(Pi[p % H, d, j] * q[p, b, j] for j in range(D))) < 1e-12
                assert abs(T[p, b, d] - sum(S_mat[p % H, d, j] * q[p, b, j] for j in range(D))) < 1e-12
