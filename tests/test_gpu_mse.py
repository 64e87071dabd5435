"""The MSE-only variant against the oracle (oracle.mse): the randomized
Hadamard query transform, and scores against MSE-only keys (stored norm,
with and without norm correction), on ragged shapes, several problems and
heads, and each workload's full size. Keys are compressed by the oracle; the
oracle scores the exact fp32 A (or fp16 norms) the GPU is given, widened to
float64. Bar: max |gpu - exact| / (1 + |exact|) <= 1e-4."""

from __future__ import annotations

import numpy as np
import pytest

import compressed_attention_scoring_amd as tq
import synth
from oracle import mse as om
from oracle import pack as opk
from oracle.codebook import codebook_fp32
from tests.gpu_util import SCORE_TOL, rel_err, say, t

pytestmark = pytest.mark.gpu


def head_signs(seed: int, H: int, D: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 11])
    return np.where(rng.integers(0, 2, size=(H, D)) == 1, 1.0, -1.0).astype(np.float32)


@pytest.mark.parametrize("D", [1, 2, 16, 32, 64, 128, 256, 1024])
@pytest.mark.parametrize("P,H,B", [(1, 1, 1), (1, 1, 37), (6, 3, 5)])
def test_hadamard_transform(D, P, H, B):
    say(f"hadamard transform D={D} P={P} H={H} B={B}")
    signs = head_signs(D, H, D)
    q = synth.queries(D + B, P, B, D)
    got = tq.tq_query_transform_hadamard(t(q), t(signs)).cpu().numpy()
    ref = np.stack([om.query_transform_hadamard(q[p].astype(np.float64), signs[p % H].astype(np.float64))
                    for p in range(P)])
    assert rel_err(got, ref) <= 1e-5


def mse_case(seed, P, H, S, D, C, layout, bits, nc):
    """MSE-only keys compressed by the oracle with each head's Hadamard rotation.
    Returns (GPU keys, idx [P,S,D], stored norms as the GPU sees them, signs, codebook)."""
    signs = head_signs(seed, H, D)
    cb = codebook_fp32(D, C)
    rng = np.random.default_rng([seed, 12])
    idx = np.empty((P, S, D), np.uint8)
    rho = np.empty((P, S))
    for p in range(P):
        k = synth.unit_keys(rng, S, D, "outlier") * rng.uniform(0.3, 3.0, (S, 1))
        R = om.hadamard_rotation(signs[p % H].astype(np.float64))
        idx[p], rho[p] = om.compress_mse(k, R, cb.astype(np.float64), norm_correction=nc)
    if layout == "unpacked":
        r32 = rho.astype(np.float32)
        return tq.Values("unpacked", t(idx), t(r32)), idx, r32.astype(np.float64), signs, cb
    r16 = opk.gamma_to_half(rho)
    return tq.Values("packed", t(opk.pack_indices(idx, bits)), t(r16), bits), idx, r16.astype(np.float64), signs, cb


CASES = [
    # layout, bits, C, D, P, H, B, S, norm correction
    ("unpacked", 0, 4, 128, 1, 1, 1, 1, False),
    ("unpacked", 0, 4, 128, 1, 1, 32, 100, True),
    ("unpacked", 0, 8, 128, 1, 1, 33, 1000, False),
    ("unpacked", 0, 4, 32, 2, 1, 70, 333, True),
    ("unpacked", 0, 8, 64, 3, 3, 5, 257, True),
    ("unpacked", 0, 2, 256, 1, 1, 128, 200, False),
    ("packed", 2, 4, 128, 1, 1, 32, 4097, True),
    ("packed", 2, 4, 64, 4, 2, 161, 300, False),
    ("packed", 3, 8, 128, 4, 2, 4, 2000, True),
    ("packed", 3, 8, 256, 1, 1, 40, 65, True),
    ("packed", 3, 8, 64, 1, 1, 96, 31, False),
    # more than 96 queries: the shared-decode form
    ("packed", 3, 8, 128, 2, 1, 128, 1000, True),
    ("unpacked", 0, 4, 128, 1, 1, 200, 333, False),
    ("packed", 2, 4, 128, 3, 3, 97, 65, False),
]


@pytest.mark.parametrize("layout,bits,C,D,P,H,B,S,nc", CASES)
def test_score_mse_matches_oracle(layout, bits, C, D, P, H, B, S, nc):
    say(f"score_mse {layout} bits={bits} C={C} D={D} P={P} H={H} B={B} S={S} nc={nc}")
    keys, idx, rho, signs, cb = mse_case(S + B + D, P, H, S, D, C, layout, bits, nc)
    A = synth.queries(S + 1, P, B, D) * 2.0
    got = tq.tq_score_mse(t(A), keys, t(cb)).cpu().numpy()
    ref = np.stack([om.scores_mse_from_transformed(A[p].astype(np.float64), idx[p], rho[p], cb) for p in range(P)])
    assert rel_err(got, ref) <= SCORE_TOL


@pytest.mark.parametrize("layout,bits,C", [("unpacked", 0, 4), ("packed", 3, 8)])
def test_hadamard_then_score_mse_equals_reconstruction(layout, bits, C):
    """GPU transform then GPU scores against the oracle's explicit reconstruction
    of every key (norm-corrected codes)."""
    say(f"hadamard then score_mse {layout}")
    P, H, B, S, D = 2, 2, 9, 700, 128
    keys, idx, rho, signs, cb = mse_case(31, P, H, S, D, C, layout, bits, True)
    q = synth.queries(31, P, B, D)
    A = tq.tq_query_transform_hadamard(t(q), t(signs))
    got = tq.tq_score_mse(A, keys, t(cb)).cpu().numpy()
    ref = np.stack([om.scores_mse_by_reconstruction(q[p].astype(np.float64), idx[p], rho[p],
                                                    om.hadamard_rotation(signs[p % H].astype(np.float64)), cb)
                    for p in range(P)])
    assert rel_err(got, ref) <= SCORE_TOL


def test_score_mse_norm_extremes():
    """Norms from 1e-30 to 1e30 and zero: the per-key scale is applied in fp32."""
    say("score_mse norm extremes")
    P, B, S, D, C = 1, 8, 64, 128, 4
    rng = np.random.default_rng(7)
    idx = rng.integers(0, C, size=(P, S, D)).astype(np.uint8)
    rho = np.geomspace(1e-30, 1e30, S).astype(np.float32)[None, :]
    rho[0, 5] = 0.0
    cb = codebook_fp32(D, C)
    A = synth.queries(7, P, B, D)
    got = tq.tq_score_mse(t(A), tq.Values("unpacked", t(idx), t(rho)), t(cb)).cpu().numpy()
    ref = om.scores_mse_from_transformed(A[0].astype(np.float64), idx[0], rho[0].astype(np.float64), cb)
    # relative to each key's own scale
    scale = 1.0 + np.abs(ref)
    assert np.max(np.abs(got[0] - ref) / np.maximum(scale, rho[0].astype(np.float64)[None, :])) <= SCORE_TOL


@pytest.mark.parametrize("layout,bits,C,D", [("unpacked", 0, 4, 128), ("packed", 2, 4, 128),
                                              ("packed", 3, 8, 128), ("unpacked", 0, 8, 256)])
@pytest.mark.parametrize("B", [1, 3, 4])
def test_score_mse_small_batch_many_keys(layout, bits, C, D, B):
    """Up to four queries over a million keys or more (the 16x16-tile form):
    random codes and norms, a ragged key count, every score checked."""
    say(f"score_mse 16x16 tiles {layout} bits={bits} C={C} D={D} B={B}")
    P, S = 8, 131075
    rng = np.random.default_rng([D, B, C, 14])
    idx = rng.integers(0, C, size=(P, S, D), dtype=np.uint8)
    rho = rng.uniform(0.5, 2.0, size=(P, S))
    cb = codebook_fp32(D, C)
    if layout == "unpacked":
        r = rho.astype(np.float32)
        keys = tq.Values("unpacked", t(idx), t(r))
    else:
        r = opk.gamma_to_half(rho)
        keys = tq.Values("packed", t(opk.pack_indices(idx, bits)), t(r), bits)
    A = synth.queries(B + D, P, B, D) * 3.0
    got = tq.tq_score_mse(t(A), keys, t(cb)).cpu().numpy()
    for p in range(P):
        ref = om.scores_mse_from_transformed(A[p].astype(np.float64), idx[p], r[p].astype(np.float64), cb)
        assert rel_err(got[p], ref) <= SCORE_TOL


@pytest.mark.parametrize("name", ["decode", "packed", "gqa", "long"])
def test_score_mse_workload_sizes(name):
    """Each workload's shape with MSE-only keys in its layout: full scores for the
    first and last problem's queries, a sample of keys."""
    w = synth.workload(name)
    say(f"score_mse workload {name}: P={w.P} B={w.B} S={w.S}")
    rng = np.random.default_rng([w.seed, 13])
    bits = w.bits if w.layout == "packed" else 0
    idx = rng.integers(0, w.C, size=(w.P, w.S, w.D), dtype=np.uint8)
    rho = rng.uniform(0.5, 2.0, size=(w.P, w.S))
    cb = codebook_fp32(w.D, w.C)
    if w.layout == "unpacked":
        r = rho.astype(np.float32)
        keys = tq.Values("unpacked", t(idx), t(r))
    else:
        r = opk.gamma_to_half(rho)
        keys = tq.Values("packed", t(opk.pack_indices(idx, bits)), t(r), bits)
    A = synth.queries(w.seed, w.P, w.B, w.D)
    got = tq.tq_score_mse(t(A), keys, t(cb)).cpu().numpy()
    sample = np.unique(np.concatenate([np.arange(0, w.S, max(1, w.S // 997)), [w.S - 1]]))
    for p in sorted({0, w.P - 1}):
        ref = om.scores_mse_from_transformed(A[p].astype(np.float64), idx[p][sample], r[p][sample].astype(np.float64), cb)
        assert rel_err(got[p][:, sample], ref) <= SCORE_TOL
