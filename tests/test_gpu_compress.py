"""tq_compress_keys against the oracle compressor (oracle.compress.quantize_prod,
which normalises each key first, then oracle.pack): indices and signs
bit-exact, gamma and the key lengths equal after their single rounding
(float32 unpacked, binary16 packed). Both sides take the index and
sign decisions in float64, so they agree except within rounding distance of a
midpoint or of a zero projection (probability about 1e-15 per coordinate).
Then compress-then-score on the GPU against the oracle's reconstruction."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import compressed_attention_scoring_amd as tq
import synth
from oracle import compress as oc
from oracle import pack as opk
from oracle import score as osc
from oracle.codebook import codebook_fp32
from tests.gpu_util import SCORE_TOL, rel_err, say, t

pytestmark = pytest.mark.gpu


def make_case(seed: int, P: int, H: int, S: int, D: int, C: int, family: str = "outlier"):
    Pi, S_mat = synth.head_matrices(seed, H, D)
    keys = np.stack([synth.unit_keys(synth.keys_rng(seed, p), S, D, family) for p in range(P)]).astype(np.float32)
    return keys, Pi, S_mat, codebook_fp32(D, C)


def oracle_compress(keys32, Pi, S_mat, cb, H, with_norm=False):
    """The oracle on the float32 keys the GPU sees (widened to float64)."""
    out = [oc.quantize_prod(keys32[p].astype(np.float64), Pi[p % H], S_mat[p % H], cb)
           for p in range(keys32.shape[0])]
    res = tuple(np.stack([o[i] for o in out]) for i in range(4))
    return res if with_norm else res[:3]


def check_equal(kg: tq.Keys, idx_u, sign_u, gamma, layout, bits, norm=None):
    gi, gs, gg = kg.idx.cpu().numpy(), kg.sign.cpu().numpy(), kg.gamma.cpu().numpy()
    gn = kg.norm.cpu().numpy()
    if layout == "unpacked":
        np.testing.assert_array_equal(gi, idx_u)
        np.testing.assert_array_equal(gs, sign_u)
        np.testing.assert_array_equal(gg, gamma.astype(np.float32))
        if norm is not None:
            np.testing.assert_array_equal(gn, norm.astype(np.float32))
    else:
        np.testing.assert_array_equal(gi, opk.pack_indices(idx_u, bits))
        np.testing.assert_array_equal(gs, opk.pack_signs(sign_u))
        np.testing.assert_array_equal(gg.view(np.uint16), opk.gamma_to_half(gamma).view(np.uint16))
        if norm is not None:
            np.testing.assert_array_equal(gn.view(np.uint16), opk.gamma_to_half(norm).view(np.uint16))


CASES = [
    # layout, bits, C, D, P, H, S
    ("unpacked", 0, 4, 128, 1, 1, 1),
    ("unpacked", 0, 4, 128, 1, 1, 17),
    ("unpacked", 0, 4, 128, 2, 1, 1000),
    ("unpacked", 0, 8, 64, 3, 3, 65),
    ("unpacked", 0, 16, 128, 1, 1, 300),
    ("unpacked", 0, 2, 64, 1, 1, 40),
    ("packed", 2, 4, 128, 1, 1, 257),
    ("packed", 2, 4, 64, 2, 2, 100),
    ("packed", 3, 8, 128, 4, 2, 100),
    ("packed", 3, 8, 64, 1, 1, 63),
]


@pytest.mark.parametrize("layout,bits,C,D,P,H,S", CASES)
def test_compress_matches_oracle(layout, bits, C, D, P, H, S):
    say(f"compress {layout} bits={bits} C={C} D={D} P={P} H={H} S={S}")
    keys, Pi, S_mat, cb = make_case(11 + S + D, P, H, S, D, C)
    kg = tq.tq_compress_keys(t(keys), t(Pi), t(S_mat), t(cb), layout, bits)
    torch.cuda.synchronize()
    idx_u, sign_u, gamma = oracle_compress(keys, Pi, S_mat, cb, H)
    check_equal(kg, idx_u, sign_u, gamma, layout, bits)


@pytest.mark.parametrize("name,P", [("decode", 1), ("packed", 1), ("gqa", 8), ("long", 1)])
def test_compress_workload_sizes(name, P):
    """Each workload's key set at full S (GQA: one sequence, its 8 heads, of the 128 problems)."""
    w = synth.workload(name)
    say(f"compress workload {name}: P={P} S={w.S} D={w.D} C={w.C} {w.layout}")
    keys, Pi, S_mat, cb = make_case(w.seed, P, w.H, w.S, w.D, w.C, w.keys)
    kg = tq.tq_compress_keys(t(keys), t(Pi), t(S_mat), t(cb), w.layout, w.bits)
    torch.cuda.synchronize()
    idx_u, sign_u, gamma = oracle_compress(keys, Pi, S_mat, cb, w.H)
    check_equal(kg, idx_u, sign_u, gamma, w.layout, w.bits)


def test_compress_then_score():
    """Keys compressed on the GPU, scored on the GPU, against the oracle's
    explicit reconstruction from the oracle's own compression."""
    say("compress then score, packed 3-bit D=128")
    P, H, B, S, D, C = 2, 2, 5, 333, 128, 8
    keys, Pi, S_mat, cb = make_case(5, P, H, S, D, C)
    q = synth.queries(5, P, B, D)
    kg = tq.tq_compress_keys(t(keys), t(Pi), t(S_mat), t(cb), "packed", 3)
    A, T = tq.tq_query_transform(t(q), t(Pi), t(S_mat))
    got = tq.tq_score(A, T, kg, t(cb)).cpu().numpy()
    idx_u, sign_u, gamma = oracle_compress(keys, Pi, S_mat, cb, H)
    g16 = opk.gamma_to_half(gamma).astype(np.float64)
    for p in range(P):
        ref = osc.scores_by_reconstruction(q[p], idx_u[p], sign_u[p], g16[p], Pi[p % H], S_mat[p % H], cb)
        assert rel_err(got[p], ref) <= SCORE_TOL


def test_compress_empty_and_tail():
    say("compress empty and single-key tail")
    keys, Pi, S_mat, cb = make_case(3, 1, 1, 16 * 4 * 2 + 1, 128, 4)
    kg = tq.tq_compress_keys(t(keys), t(Pi), t(S_mat), t(cb), "unpacked")
    idx_u, sign_u, gamma = oracle_compress(keys, Pi, S_mat, cb, 1)
    check_equal(kg, idx_u, sign_u, gamma, "unpacked", 0)
    empty = tq.tq_compress_keys(t(keys[:, :0]), t(Pi), t(S_mat), t(cb), "packed", 2)
    assert empty.idx.shape == (1, 0, 32)


@pytest.mark.parametrize("layout,bits,C,D", [("unpacked", 0, 4, 128), ("packed", 2, 4, 128), ("packed", 3, 8, 64)])
def test_compress_normalises_keys_of_any_length(layout, bits, C, D):
    """Keys of lengths from 1e-3 to 1e3 and an all-zero key: the codes are those of
    the unit keys (the oracle normalises first), the stored norm is the length."""
    say(f"compress non-unit keys {layout} bits={bits} C={C} D={D}")
    rng = np.random.default_rng([41, D, C])
    P, H, S = 2, 1, 150
    Pi, S_mat = synth.head_matrices(41, H, D)
    cb = codebook_fp32(D, C)
    keys = rng.standard_normal((P, S, D)) * np.exp(rng.uniform(np.log(1e-3), np.log(1e3), size=(P, S, 1)))
    keys[0, 7] = 0.0
    keys = keys.astype(np.float32)
    kg = tq.tq_compress_keys(t(keys), t(Pi), t(S_mat), t(cb), layout, bits)
    torch.cuda.synchronize()
    idx_u, sign_u, gamma, norm = oracle_compress(keys, Pi, S_mat, cb, H, with_norm=True)
    assert norm[0, 7] == 0.0
    check_equal(kg, idx_u, sign_u, gamma, layout, bits, norm)
    # the unit-length keys compress to the same codes
    unit = (keys.astype(np.float64) / np.maximum(norm, 1e-300)[..., None]).astype(np.float32)
    kg1 = tq.tq_compress_keys(t(unit), t(Pi), t(S_mat), t(cb), layout, bits)
    same = (kg1.idx.cpu().numpy() == kg.idx.cpu().numpy()).mean()
    assert same > 0.999, same
