"""The integer four-query scorer (packed keys with signs, B <= 4 per workgroup
row: kernel names mfma16i8_*): A and T enter as four int8 limbs below their
row's largest coordinate, the codebook as three below its largest entry; the
products are exact in int32. On random ragged shapes these tests hold it to
1e-5 * (1 + |exact|), ten times inside tq_score's bar; on rows whose
magnitudes span nine decades (each row's scale follows its largest
coordinate) to that bar and to the split-f16 kernels' own error on the same
inputs; and on values where rounding to a limb ties (half-integers of the
scaled grid) to tq_score's bar."""

import math
import zlib

import numpy as np
import pytest
import torch

import compressed_attention_scoring_amd as tq
from tests.gpu_util import SCORE_TOL, keys_to_gpu, oracle_scores_transformed, random_codes, rel_err, say, t

pytestmark = pytest.mark.gpu

I8_TOL = 1e-5


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_case(bits, C, D, P, B, S, rng, A=None, T=None, cb=None, kernel="mfma16"):
    if kernel == "mfma16":
        name = tq.tq_score_kernel_name("packed", bits, C, P, B, S, D, kernel)
        assert name == f"mfma16i8_packed{bits}", name
    if A is None:
        A = rng.standard_normal((P, B, D)).astype(np.float32)
    if T is None:
        T = (rng.standard_normal((P, B, D)) * math.sqrt(D)).astype(np.float32)
    if cb is None:
        cb = np.sort(rng.standard_normal(C) / math.sqrt(D)).astype(np.float32)
    idx_u, sign_u, gamma_k, idx, sign = random_codes(rng, P, S, D, C, "packed", bits)
    keys = keys_to_gpu("packed", bits, idx, sign, gamma_k)
    got = tq.tq_score_with_kernel(t(A), t(T), keys, t(cb), kernel).cpu().numpy()
    assert np.all(np.isfinite(got))
    ref = oracle_scores_transformed(A, T, idx_u, sign_u, gamma_k, cb)
    return rel_err(got, ref)


CASES = [(bits, C, D, P, B, S)
         for bits, C in ((2, 4), (3, 8))
         for D in (128, 256)
         for P, B, S in ((1, 1, 1), (2, 3, 37), (1, 4, 300), (3, 5, 129), (1, 8, 64), (2, 2, 1 << 12))]


@pytest.mark.parametrize("bits,C,D,P,B,S", CASES)
def test_i8_random(bits, C, D, P, B, S):
    say(f"i8 score bits={bits} C={C} D={D} P={P} B={B} S={S}")
    rng = np.random.default_rng(zlib.crc32(repr((bits, C, D, P, B, S)).encode()))
    err = run_case(bits, C, D, P, B, S, rng)
    say(f"i8 score: max rel err {err:.2e}")
    assert err <= I8_TOL


@pytest.mark.parametrize("D", [128, 256])
def test_i8_wide_dynamic_range(D):
    """Rows whose coordinates span 1e-6 .. 1e3 (and a T row a thousand times
    larger than its A row), with a codebook spanning four decades: within
    tq_score's 1e-4 bar and no worse than the split-f16 kernels on the same
    inputs (both carry about 21-22 bits of each operand, so a coordinate of 1e3
    against the largest codebook entry already costs ~5e-5)."""
    say(f"i8 score wide dynamic range D={D}")
    P, B, S, C = 2, 4, 257, 8

    def inputs():
        rng = np.random.default_rng(5 + D)
        mag = 10.0 ** rng.uniform(-6, 3, size=(P, B, D))
        A = (rng.choice([-1.0, 1.0], size=(P, B, D)) * mag).astype(np.float32)
        T = (rng.standard_normal((P, B, D)) * 1e3).astype(np.float32)
        return rng, A, T

    cb = np.array([-3.1, -0.7, -0.05, 1e-4, 0.02, 0.33, 0.9, 2.6], np.float32) / np.float32(math.sqrt(D))
    rng, A, T = inputs()
    err = run_case(3, C, D, P, B, S, rng, A, T, cb)
    rng, A, T = inputs()
    err_f16 = run_case(3, C, D, P, B, S, rng, A, T, cb, kernel="mfma_lds")
    say(f"i8 wide range: max rel err {err:.2e} (split-f16 LDS kernel {err_f16:.2e})")
    assert err <= SCORE_TOL
    assert err <= 2.0 * err_f16 + 1e-6


def test_i8_limb_rounding_ties():
    """Coordinates that scale to exact half-integers at the first and second
    limb (x = k + 1/2 and k + (j + 1/2)/128 after scaling by 127 / max, with
    the row maximum 127 so the scale is exactly 1), against a codebook whose
    largest entry is 127 and whose entries sit on or halfway between integers:
    every limb is then exact, a limb rounded out of int8 range would cost about
    2^-7 of a score, and the integer sums leave only the epilogue's fp32
    rounding."""
    say("i8 score limb rounding ties")
    rng = np.random.default_rng(77)
    P, B, S, D, C = 1, 4, 96, 128, 8
    k = rng.integers(-126, 126, size=(P, B, D)).astype(np.float64)
    j = rng.integers(-63, 63, size=(P, B, D)).astype(np.float64)
    x = np.where(rng.integers(0, 2, size=(P, B, D)) == 1, k + 0.5, k + (j + 0.5) / 128.0)
    x[..., 0] = 127.0
    A = x.astype(np.float32)
    T = x[:, ::-1].astype(np.float32).copy()
    cb = np.array([-127.0, -90.5, -50.0, -0.5, 0.5, 33.5, 80.0, 127.0], np.float32)
    err = run_case(3, C, D, P, B, S, rng, A, T, cb)
    say(f"i8 ties: max rel err {err:.2e}")
    assert err <= I8_TOL


@pytest.mark.parametrize("bits,C,D", [(2, 4, 128), (3, 8, 128), (2, 4, 256), (3, 8, 256)])
def test_i8_mse_only(bits, C, D):
    """MSE-only keys (tq_score_mse: no signs, the stored norm scales M) on the
    four-query shape, which takes the integer form for packed keys: every score
    of a million-key launch within 1e-5 * (1 + |exact|)."""
    from oracle import mse as om
    from oracle import pack as opk
    from oracle.codebook import codebook_fp32

    say(f"i8 score_mse bits={bits} C={C} D={D}")
    P, B, S = 8, 3, 131075
    rng = np.random.default_rng([D, bits, 21])
    idx = rng.integers(0, C, size=(P, S, D), dtype=np.uint8)
    r = opk.gamma_to_half(rng.uniform(0.5, 2.0, size=(P, S)))
    cb = codebook_fp32(D, C)
    keys = tq.Values("packed", t(opk.pack_indices(idx, bits)), t(r), bits)
    A = (rng.standard_normal((P, B, D)) * 3.0).astype(np.float32)
    got = tq.tq_score_mse(t(A), keys, t(cb)).cpu().numpy()
    err = max(rel_err(got[p], om.scores_mse_from_transformed(A[p].astype(np.float64), idx[p],
                                                               r[p].astype(np.float64), cb)) for p in range(P))
    say(f"i8 score_mse: max rel err {err:.2e}")
    assert err <= I8_TOL
