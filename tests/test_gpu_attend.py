"""tq_attend against the oracle (oracle.attend): softmax over scaled scores
times the dequantized values, for both value layouts, ragged key counts and
query blocks, several problems and heads, and each workload's full size.
Inputs are seeded and synthetic; the oracle sees the exact fp32 (or fp16)
numbers the GPU is given, widened to float64. Bar: max |gpu - exact| /
(1 + |exact|) <= 1e-4 over every output element."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import compressed_attention_scoring_amd as tq
import synth
from oracle import attend as oa
from oracle import pack as opk
from oracle import score as osc
from oracle.codebook import codebook_fp32
from tests.gpu_util import SCORE_TOL, rel_err, say, t

pytestmark = pytest.mark.gpu


def value_case(seed: int, P: int, H: int, S: int, D: int, C: int, layout: str, bits: int):
    """Gaussian value vectors compressed by the oracle's value quantizer.

    Returns (GPU Values, unpacked idx [P,S,D], norms as the GPU sees them
    (float64 of the stored fp32/fp16), Pi_v [H,D,D] fp32, codebook fp32)."""
    rng = np.random.default_rng([seed, 7])
    Pi_v = np.stack([synth.haar_rotation(rng, D) for _ in range(H)])
    cb = codebook_fp32(D, C)
    idx = np.empty((P, S, D), np.uint8)
    norm = np.empty((P, S), np.float64)
    for p in range(P):
        v = rng.standard_normal((S, D)) * rng.uniform(0.2, 3.0, (S, 1))
        i, n = oa.compress_values(v, Pi_v[p % H].astype(np.float64), cb.astype(np.float64))
        idx[p], norm[p] = i, n
    if layout == "unpacked":
        n32 = norm.astype(np.float32)
        vals = tq.Values("unpacked", t(idx), t(n32))
        return vals, idx, n32.astype(np.float64), Pi_v, cb
    n16 = opk.gamma_to_half(norm)
    vals = tq.Values("packed", t(opk.pack_indices(idx, bits)), t(n16), bits)
    return vals, idx, n16.astype(np.float64), Pi_v, cb


def oracle_out(scores, idx, norm, Pi_v, cb, scale, H):
    P = scores.shape[0]
    return np.stack([oa.attend_rotated(scores[p].astype(np.float64), idx[p], norm[p],
                                       Pi_v[p % H].astype(np.float64), cb.astype(np.float64), scale)
                     for p in range(P)])


def run_case(seed, P, H, B, S, D, C, layout, bits, scale, spread=3.0):
    vals, idx, norm, Pi_v, cb = value_case(seed, P, H, S, D, C, layout, bits)
    rng = np.random.default_rng([seed, 8])
    scores = (rng.standard_normal((P, B, S)) * spread).astype(np.float32)
    got = tq.tq_attend(t(scores), vals, t(cb), t(Pi_v), scale).cpu().numpy()
    ref = oracle_out(scores, idx, norm, Pi_v, cb, scale, H)
    err = rel_err(got, ref)
    assert err <= SCORE_TOL, f"max rel err {err:.3e}"
    return scores, vals, idx, norm, Pi_v, cb


CASES = [
    # layout, bits, C, D, P, H, B, S
    ("unpacked", 0, 4, 128, 1, 1, 1, 1),
    ("unpacked", 0, 4, 128, 1, 1, 2, 31),
    ("unpacked", 0, 4, 128, 1, 1, 32, 32),
    ("unpacked", 0, 4, 128, 1, 1, 33, 33),
    ("unpacked", 0, 4, 128, 1, 1, 5, 5000),
    ("unpacked", 0, 8, 64, 3, 3, 7, 1000),
    ("unpacked", 0, 2, 64, 1, 1, 64, 129),
    ("unpacked", 0, 1, 128, 1, 1, 4, 77),
    ("packed", 2, 4, 128, 1, 1, 32, 2049),
    ("packed", 2, 4, 64, 4, 2, 3, 300),
    ("packed", 3, 8, 128, 4, 2, 70, 1500),
    ("packed", 3, 8, 64, 1, 1, 1, 100),
    ("packed", 3, 8, 128, 2, 1, 96, 40000),
    ("unpacked", 0, 4, 128, 1, 1, 8, 3000),
    ("packed", 3, 8, 128, 1, 1, 9, 700),
    ("packed", 2, 4, 64, 1, 1, 161, 2500),
    ("unpacked", 0, 8, 128, 2, 2, 128, 5000),
]


@pytest.mark.parametrize("layout,bits,C,D,P,H,B,S", CASES)
def test_attend_matches_oracle(layout, bits, C, D, P, H, B, S):
    say(f"attend {layout} bits={bits} C={C} D={D} P={P} H={H} B={B} S={S}")
    run_case(100 + S + B, P, H, B, S, D, C, layout, bits, 1.0)


@pytest.mark.parametrize("scale", [0.0, 1.0 / np.sqrt(128), 4.0, -2.0])
def test_attend_scales(scale):
    """Zero scale is the mean of the values; a large scale a near-one-hot softmax."""
    say(f"attend scale={scale}")
    run_case(9, 1, 1, 8, 700, 128, 4, "unpacked", 0, float(scale))


def test_attend_dominant_key():
    say("attend dominant key")
    vals, idx, norm, Pi_v, cb = value_case(4, 1, 1, 300, 128, 8, "packed", 3)
    scores = np.random.default_rng(1).standard_normal((1, 3, 300)).astype(np.float32)
    scores[0, :, 123] = 80.0
    got = tq.tq_attend(t(scores), vals, t(cb), t(Pi_v), 1.0).cpu().numpy()
    ref = oracle_out(scores, idx, norm, Pi_v, cb, 1.0, 1)
    assert rel_err(got, ref) <= SCORE_TOL
    v123 = oa.dequantize_values(idx[0, 123:124], norm[0, 123:124], Pi_v[0].astype(np.float64), cb.astype(np.float64))
    assert rel_err(got[0], np.broadcast_to(v123, (3, 128))) <= SCORE_TOL


def test_attend_empty_and_workspace_reuse():
    say("attend empty calls and workspace reuse")
    vals, idx, norm, Pi_v, cb = value_case(5, 1, 1, 90, 64, 4, "unpacked", 0)
    empty = tq.tq_attend(t(np.zeros((1, 0, 90), np.float32)), vals, t(cb), t(Pi_v))
    assert empty.shape == (1, 0, 64)
    ws = torch.empty(tq.tq_attend_workspace_bytes(1, 40, 90, 64), dtype=torch.uint8, device="cuda")
    out = torch.empty((1, 40, 64), dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(2)
    for _ in range(3):
        scores = rng.standard_normal((1, 40, 90)).astype(np.float32)
        tq.tq_attend(t(scores), vals, t(cb), t(Pi_v), 0.5, out=out, workspace=ws)
        assert rel_err(out.cpu().numpy(), oracle_out(scores, idx, norm, Pi_v, cb, 0.5, 1)) <= SCORE_TOL


def test_attend_rejects_small_workspace():
    say("attend small workspace")
    vals, _, _, Pi_v, cb = value_case(6, 1, 1, 90, 64, 4, "unpacked", 0)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(tq.TqError):
        tq.tq_attend(t(np.zeros((1, 4, 90), np.float32)), vals, t(cb), t(Pi_v), workspace=ws)


@pytest.mark.parametrize("name", ["decode", "packed", "gqa", "long"])
def test_attend_workload_sizes(name):
    """Each workload's full shape: its B, S, D and P problems, values in the
    workload's key layout and codebook size."""
    w = synth.workload(name)
    say(f"attend workload {name}: P={w.P} B={w.B} S={w.S} D={w.D} C={w.C} {w.layout}")
    rng = np.random.default_rng([w.seed, 9])
    Pi_v = np.stack([synth.haar_rotation(rng, w.D) for _ in range(w.H)])
    cb = codebook_fp32(w.D, w.C)
    idx = rng.integers(0, w.C, size=(w.P, w.S, w.D), dtype=np.uint8)
    norm = rng.uniform(0.5, 2.0, size=(w.P, w.S)) * np.sqrt(w.D)
    if w.layout == "unpacked":
        n = norm.astype(np.float32)
        vals = tq.Values("unpacked", t(idx), t(n))
    else:
        n = opk.gamma_to_half(norm)
        vals = tq.Values("packed", t(opk.pack_indices(idx, w.bits)), t(n), w.bits)
    scores = rng.standard_normal((w.P, w.B, w.S)).astype(np.float32) * 4.0
    scale = 1.0 / np.sqrt(w.D)
    got = tq.tq_attend(t(scores), vals, t(cb), t(Pi_v), scale).cpu().numpy()
    ref = oracle_out(scores, idx, n.astype(np.float64), Pi_v, cb, scale, w.H)
    assert rel_err(got, ref) <= SCORE_TOL


def test_score_then_attend():
    """Keys scored on the GPU then attended on the GPU, against the oracle's
    own scores of the same compressed keys."""
    say("score then attend, packed 3-bit D=128")
    P, H, B, S, D, C = 2, 2, 6, 1234, 128, 8
    Pi, S_mat = synth.head_matrices(21, H, D)
    q = synth.queries(21, P, B, D)
    rng = np.random.default_rng(3)
    idx_k = rng.integers(0, C, size=(P, S, D)).astype(np.uint8)
    sign_k = np.where(rng.integers(0, 2, size=(P, S, D)) == 1, 1, -1).astype(np.int8)
    gamma = opk.gamma_to_half(rng.uniform(0.05, 0.6, size=(P, S)))
    cb = codebook_fp32(D, C)
    keys = tq.Keys("packed", t(opk.pack_indices(idx_k, 3)), t(opk.pack_signs(sign_k)), t(gamma), 3)
    vals, idx_v, norm, Pi_v, cbv = value_case(22, P, H, S, D, C, "packed", 3)
    A, T = tq.tq_query_transform(t(q), t(Pi), t(S_mat))
    scores = tq.tq_score(A, T, keys, t(cb))
    got = tq.tq_attend(scores, vals, t(cbv), t(Pi_v), 1.0 / np.sqrt(D)).cpu().numpy()
    ref_scores = np.stack([osc.scores_by_reconstruction(q[p], idx_k[p], sign_k[p], gamma[p].astype(np.float64),
                                                        Pi[p % H], S_mat[p % H], cb) for p in range(P)])
    ref = oracle_out(ref_scores, idx_v, norm, Pi_v, cbv, 1.0 / np.sqrt(D), H)
    assert rel_err(got, ref) <= SCORE_TOL


@pytest.mark.parametrize("B", [3, 40])
def test_attend_rescales(B):
    """Scores rising along the keys (the running maximum moves many times), norms
    growing over six decades with zero norms between (the norm scale moves)."""
    say(f"attend rescales B={B}")
    P, H, S, D, C = 1, 1, 4000, 128, 8
    vals, idx, _, Pi_v, cb = value_case(12, P, H, S, D, C, "unpacked", 0)
    norm = np.geomspace(1e-3, 1e3, S).astype(np.float32)[None, :]
    norm[0, ::7] = 0.0
    vals = tq.Values("unpacked", vals.idx, t(norm))
    rng = np.random.default_rng(13)
    ramp = np.linspace(-50.0, 50.0, S)[None, None, :]
    scores = (ramp + rng.standard_normal((P, B, S)) * 2.0).astype(np.float32)
    got = tq.tq_attend(t(scores), vals, t(cb), t(Pi_v), 0.3).cpu().numpy()
    ref = oracle_out(scores, idx, norm.astype(np.float64), Pi_v, cb, 0.3, H)
    assert rel_err(got, ref) <= SCORE_TOL
