"""Seeded random shapes for the scoring path: the query transform and tq_score
(the automatic choice and every kernel family the shape admits) against the
oracle, over shapes drawn from the ranges the kernels handle (problem and head
counts, ragged query and key counts, every supported D, both key layouts and
codebook sizes). Each case prints its draw before it runs; the seed of the
draw is the case's index, so any case can be rerun alone.

Bars: scores within 1e-4 * (1 + |exact|) of the oracle's float64 value from
the A, T the GPU computed; A and T within the fp32 dot-product bound."""

import numpy as np
import pytest
import torch

import compressed_attention_scoring_amd as tq
import synth
from oracle import query_transform as oqt
from tests.gpu_util import (SCORE_TOL, keys_to_gpu, oracle_scores_transformed, random_codes, rel_err,
                            say, t)

pytestmark = pytest.mark.gpu

N_CASES = 48
FAMILIES = ["auto", "valu", "mfma_lds", "mfma_reg", "mfma16", "mfma_shared"]


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw(i):
    rng = np.random.default_rng([2024, i])
    layout = "packed" if rng.random() < 0.6 else "unpacked"
    if layout == "packed":
        bits = int(rng.choice([2, 3]))
        C = 1 << bits
        D = int(rng.choice([64, 128, 256]))
    else:
        bits = 0
        C = int(rng.choice([2, 4, 8, 16]))
        D = int(rng.choice([32, 64, 128, 256, 40]))
    H = int(rng.choice([1, 2, 3]))
    P = H * int(rng.integers(1, 3))
    B = int(rng.choice([1, 2, 3, 4, 5, 16, 31, 32, 33, 64, 97, 129, 140]))
    S = int(rng.choice([1, 2, 17, 31, 32, 33, 100, 511, 1000, 2049, 4097]))
    return layout, bits, C, D, P, H, B, S


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    layout, bits, C, D, P, H, B, S = draw(i)
    say(f"random shape {i}: {layout} bits={bits} C={C} D={D} P={P} H={H} B={B} S={S}")
    rng = np.random.default_rng([7, i])
    q = rng.standard_normal((P, B, D)).astype(np.float32)
    Pi = np.stack([synth.haar_rotation(rng, D) for _ in range(H)])
    Sm = rng.standard_normal((H, D, D)).astype(np.float32)
    A_g, T_g = tq.tq_query_transform(t(q), t(Pi), t(Sm))
    A, T = A_g.cpu().numpy(), T_g.cpu().numpy()
    rA, rT = oqt.query_transform(q, Pi, Sm)
    for got, ref, W in ((A, rA, Pi), (T, rT, Sm)):
        bound = np.stack([np.abs(q[p].astype(np.float64)) @ np.abs(W[p % H].astype(np.float64)).T
                          for p in range(P)]) * D * 2.0 ** -24 * 1.01 + 1e-30
        assert np.all(np.abs(got - ref) <= bound)
    cb = np.sort(rng.standard_normal(C) / np.sqrt(D)).astype(np.float32)
    idx_u, sign_u, gamma_k, idx, sign = random_codes(rng, P, S, D, C, layout, bits)
    keys = keys_to_gpu(layout, bits, idx, sign, gamma_k)
    ref = oracle_scores_transformed(A, T, idx_u, sign_u, gamma_k, cb)
    ran = 0
    for fam in FAMILIES:
        name = tq.tq_score_kernel_name(layout, bits, C, P, B, S, D, fam)
        if name is None:
            continue
        say(f"random shape {i}: kernel {fam} ({name})")
        got = tq.tq_score_with_kernel(A_g, T_g, keys, t(cb), fam).cpu().numpy()
        err = rel_err(got, ref)
        assert err <= SCORE_TOL, f"{fam} ({name}): max rel err {err:.3e}"
        ran += 1
    assert ran >= 2     # the automatic choice and at least the vector family
