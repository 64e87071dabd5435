"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Scores must be within 1e-4 * (1 + |exact|) of the oracle's float64 value;
unpacking (tq_decode_debug) must be bit-exact. Every kernel family is checked on
every shape it supports, over ragged key counts (tails shorter than a 32-key
tile), ragged query counts (partial 32-query tiles), several D, both layouts,
multi-problem batches with per-head matrices, extreme operand magnitudes and
empty inputs.
"""

import math
import zlib

import numpy as np
import pytest
import torch

import compressed_attention_scoring_amd as tq
import synth
from oracle import codebook as ocb
from oracle import pack as opk
from oracle import query_transform as oqt
from oracle import score as osc
from tests.gpu_util import (SCORE_TOL, dev, keys_to_gpu, oracle_scores_transformed,
                            random_codes, rel_err, say, t)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ---------------------------------------------------------------------------
# the worked example
# ---------------------------------------------------------------------------

def test_worked_example(golden):
    g = golden("worked_example.json")
    say("worked example B=1 S=2 D=2")
    q = t(np.array(g["q"], np.float32))
    Pi = t(np.array(g["Pi"], np.float32))
    Sm = t(np.array(g["S_mat"], np.float32))
    A, T = tq.tq_query_transform(q, Pi, Sm)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(A.cpu().numpy(), g["A"])
    np.testing.assert_array_equal(T.cpu().numpy(), g["T"])
    keys = keys_to_gpu("unpacked", 0, np.array(g["K_idx"], np.uint8),
                       np.array(g["qjl_signs"], np.int8), np.array(g["gamma"], np.float32))
    s = tq.tq_score(A, T, keys, t(np.array(g["codebook"], np.float32))).cpu().numpy()
    np.testing.assert_array_equal(np.round(s.astype(np.float64), g["decimals"]), g["scores"])


# ---------------------------------------------------------------------------
# query transform
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("P,H,B,D", [(1, 1, 1, 2), (1, 1, 2, 32), (1, 1, 32, 128), (3, 3, 5, 64),
                                     (16, 8, 4, 128), (1, 1, 128, 128), (2, 1, 7, 256),
                                     (1, 1, 3, 1000), (2, 2, 17, 33),
                                     # problems of one head share 32-row tiles (rows span problems)
                                     (128, 8, 4, 128), (6, 2, 33, 64), (12, 3, 1, 96),
                                     # every D of the matrix-core form; 16-row tiles cut across problems
                                     (2, 2, 17, 160), (1, 1, 16, 192), (3, 1, 15, 224), (4, 2, 9, 32),
                                     (5, 1, 3, 128)])
def test_query_transform_parity(P, H, B, D):
    say(f"query_transform P={P} H={H} B={B} D={D}")
    rng = np.random.default_rng(P * 1000 + D)
    q = rng.standard_normal((P, B, D)).astype(np.float32)
    Pi = np.stack([synth.haar_rotation(rng, D) for _ in range(H)])
    Sm = rng.standard_normal((H, D, D)).astype(np.float32)
    A, T = tq.tq_query_transform(t(q), t(Pi), t(Sm))
    A, T = A.cpu().numpy(), T.cpu().numpy()
    rA, rT = oqt.query_transform(q, Pi, Sm)
    # fp32 dot product of length D: |err| <= D * 2^-24 * sum |terms|
    for got, ref, W in ((A, rA, Pi), (T, rT, Sm)):
        bound = np.stack([np.abs(q[p].astype(np.float64)) @ np.abs(W[p % H].astype(np.float64)).T
                          for p in range(P)]) * D * 2.0 ** -24 * 1.01 + 1e-30
        assert np.all(np.abs(got - ref) <= bound)


# ---------------------------------------------------------------------------
# tq_score on random valid codes: every kernel family, layout, D and ragged shape
# ---------------------------------------------------------------------------

SCORE_CASES = []
for layout, bits, C in (("unpacked", 0, 4), ("unpacked", 0, 8), ("packed", 2, 4), ("packed", 3, 8)):
    for D in ((32, 64, 128, 256) if layout == "unpacked" else (64, 128, 256)):
        for B, S in ((1, 1), (2, 31), (4, 33), (5, 257), (32, 300), (33, 64), (64, 100), (96, 70), (128, 95),
                     (161, 40)):
            SCORE_CASES.append((layout, bits, C, D, B, S))


@pytest.mark.parametrize("kernel", ["valu", "mfma_lds", "mfma_reg", "mfma16", "mfma_shared"])
@pytest.mark.parametrize("layout,bits,C,D,B,S", SCORE_CASES)
def test_score_random_codes(kernel, layout, bits, C, D, B, S):
    if tq.tq_score_kernel_name(layout, bits, C, 2, B, S, D, kernel) is None:
        pytest.skip("kernel does not cover this shape")
    say(f"score kernel={kernel} {layout} bits={bits} C={C} D={D} B={B} S={S}")
    rng = np.random.default_rng(zlib.crc32(repr((layout, bits, C, D, B, S)).encode()))
    P = 2
    A = rng.standard_normal((P, B, D)).astype(np.float32)
    T = (rng.standard_normal((P, B, D)) * math.sqrt(D)).astype(np.float32)
    cb = np.sort(rng.standard_normal(C) / math.sqrt(D)).astype(np.float32)
    idx_u, sign_u, gamma_k, idx, sign = random_codes(rng, P, S, D, C, layout, bits)
    keys = keys_to_gpu(layout, bits, idx, sign, gamma_k)
    got = tq.tq_score_with_kernel(t(A), t(T), keys, t(cb), kernel).cpu().numpy()
    ref = oracle_scores_transformed(A, T, idx_u, sign_u, gamma_k, cb)
    assert got.shape == (P, B, S)
    assert rel_err(got, ref) <= SCORE_TOL


@pytest.mark.parametrize("D", [2, 3, 24, 40, 1024])
def test_score_valu_odd_dims(D):
    say(f"score valu unpacked odd D={D}")
    rng = np.random.default_rng(D)
    P, B, S, C = 1, 3, 77, 16
    A = rng.standard_normal((P, B, D)).astype(np.float32)
    T = rng.standard_normal((P, B, D)).astype(np.float32)
    cb = rng.standard_normal(C).astype(np.float32)
    idx_u, sign_u, gamma_k, idx, sign = random_codes(rng, P, S, D, C, "unpacked", 0)
    got = tq.tq_score(t(A), t(T), keys_to_gpu("unpacked", 0, idx, sign, gamma_k), t(cb)).cpu().numpy()
    assert rel_err(got, oracle_scores_transformed(A, T, idx_u, sign_u, gamma_k, cb)) <= SCORE_TOL


@pytest.mark.parametrize("kernel", ["valu", "mfma_lds", "mfma_reg", "mfma16", "mfma_shared"])
@pytest.mark.parametrize("B", [3, 32, 100])
@pytest.mark.parametrize("scale", [1e-6, 1e4, 3e5])
def test_score_extreme_magnitudes(kernel, B, scale):
    """Large and tiny A, T (and a large codebook) stay accurate: the matrix-core
    path rescales its f16 operands by powers of two."""
    say(f"score extreme magnitudes kernel={kernel} B={B} scale={scale}")
    rng = np.random.default_rng(7)
    P, S, D, C = 1, 64, 128, 8
    A = (rng.standard_normal((P, B, D)) * scale).astype(np.float32)
    T = (rng.standard_normal((P, B, D)) * scale * 10).astype(np.float32)
    cb = (np.sort(rng.standard_normal(C)) * scale).astype(np.float32)
    idx_u, sign_u, gamma_k, idx, sign = random_codes(rng, P, S, D, C, "packed", 3)
    got = tq.tq_score_with_kernel(t(A), t(T), keys_to_gpu("packed", 3, idx, sign, gamma_k), t(cb),
                                  kernel).cpu().numpy()
    ref = oracle_scores_transformed(A, T, idx_u, sign_u, gamma_k, cb)
    # With operands this large the scores cancel; an fp32 dot product of length
    # D carries an error up to D * 2^-24 * sum |terms| (the terms' absolute sum is
    # the same formula on |A|, |T|, |codebook| and all-positive signs).
    terms = oracle_scores_transformed(np.abs(A), np.abs(T), idx_u, np.ones_like(sign_u), gamma_k, np.abs(cb))
    bound = SCORE_TOL * (1.0 + np.abs(ref)) + D * 2.0 ** -24 * terms
    assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("kernel", ["valu", "mfma_lds", "mfma_reg", "mfma16", "mfma_shared"])
@pytest.mark.parametrize("B", [3, 32])
@pytest.mark.parametrize("case", ["tiny", "zero_rows", "tiny_codebook", "zero_codebook"])
def test_score_tiny_and_zero_operands(kernel, B, case):
    """Rows and codebooks near the bottom of the fp32 range, and all-zero ones,
    give finite scores within the tolerance: the power-of-two operand scale is
    clamped, so it never overflows to inf (inf * 0 would be NaN)."""
    say(f"score tiny/zero operands kernel={kernel} B={B} case={case}")
    rng = np.random.default_rng(11)
    P, S, D, C = 1, 64, 128, 8
    A = rng.standard_normal((P, B, D)).astype(np.float32)
    T = (rng.standard_normal((P, B, D)) * 10).astype(np.float32)
    cb = np.sort(rng.standard_normal(C)).astype(np.float32)
    if case == "tiny":
        A *= np.float32(1e-36)
        T *= np.float32(1e-36)
    elif case == "zero_rows":
        A[:, ::2] = 0.0
        T[:, ::2] = 0.0
        A[:, 1] *= np.float32(1e-37)
    elif case == "tiny_codebook":
        cb *= np.float32(1e-37)
    else:
        cb[:] = 0.0
    idx_u, sign_u, gamma_k, idx, sign = random_codes(rng, P, S, D, C, "packed", 3)
    got = tq.tq_score_with_kernel(t(A), t(T), keys_to_gpu("packed", 3, idx, sign, gamma_k), t(cb),
                                  kernel).cpu().numpy()
    assert np.all(np.isfinite(got))
    ref = oracle_scores_transformed(A, T, idx_u, sign_u, gamma_k, cb)
    assert np.all(np.abs(got - ref) <= SCORE_TOL * (1.0 + np.abs(ref)))


def test_empty_inputs():
    say("empty inputs")
    D = 128
    A = torch.zeros((1, 4, D), device=dev())
    cb = torch.zeros(4, device=dev())
    keys = tq.Keys("unpacked", torch.zeros((1, 0, D), dtype=torch.uint8, device=dev()),
                   torch.zeros((1, 0, D), dtype=torch.int8, device=dev()),
                   torch.zeros((1, 0), dtype=torch.float32, device=dev()))
    out = tq.tq_score(A, A, keys, cb)
    assert out.shape == (1, 4, 0)
    q0 = torch.zeros((1, 0, D), device=dev())
    A0, T0 = tq.tq_query_transform(q0, torch.eye(D, device=dev()), torch.eye(D, device=dev()))
    assert A0.shape == (1, 0, D)


def test_misaligned_buffer_is_rejected():
    say("misaligned buffer")
    D, S = 128, 8
    raw = torch.zeros(S * D + 1, dtype=torch.uint8, device=dev())
    keys = tq.Keys("unpacked", raw[1:].view(1, S, D), torch.ones((1, S, D), dtype=torch.int8, device=dev()),
                   torch.zeros((1, S), device=dev()))
    A = torch.zeros((1, 2, D), device=dev())
    with pytest.raises(tq.TqError, match="aligned"):
        tq.tq_score(A, A, keys, torch.zeros(4, device=dev()))


# ---------------------------------------------------------------------------
# debug decode: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout,bits,D", [("unpacked", 0, 2), ("unpacked", 0, 128), ("packed", 2, 8),
                                           ("packed", 2, 128), ("packed", 3, 8), ("packed", 3, 128),
                                           ("packed", 3, 256), ("packed", 2, 96)])
def test_decode_bit_exact(layout, bits, D):
    say(f"decode {layout} bits={bits} D={D}")
    rng = np.random.default_rng(D + bits)
    P, S = 3, 123
    C = 2 ** bits if bits else 4
    idx_u, sign_u, gamma_k, idx, sign = random_codes(rng, P, S, D, C, layout, bits)
    i, s, g = tq.tq_decode_debug(keys_to_gpu(layout, bits, idx, sign, gamma_k), D)
    np.testing.assert_array_equal(i.cpu().numpy(), idx_u)
    np.testing.assert_array_equal(s.cpu().numpy(), sign_u)
    np.testing.assert_array_equal(g.cpu().numpy(), gamma_k.astype(np.float32))
    # the oracle's unpacker reads the same bytes back identically
    if layout == "packed":
        np.testing.assert_array_equal(opk.unpack_indices(idx, bits, D), idx_u)
        np.testing.assert_array_equal(opk.unpack_signs(sign, D), sign_u)
