"""tq_score_attend (the fused decode step), in both its forms and the automatic
choice, against the oracle chain: oracle
scores from the fp32 A, T the GPU is given (oracle.score), then the oracle's
softmax and value sum (oracle.attend). Key and value layouts, ragged query
and key counts, several problems and heads, and each workload's full size.
Bar: max |gpu - exact| / (1 + |exact|) <= 1e-4."""

from __future__ import annotations

import numpy as np
import pytest

import compressed_attention_scoring_amd as tq
import synth
from oracle import attend as oa
from oracle import pack as opk
from oracle.codebook import codebook_fp32
from tests.gpu_util import SCORE_TOL, keys_to_gpu, oracle_scores_transformed, random_codes, rel_err, say, t

pytestmark = pytest.mark.gpu

D = 128


def values_case(rng, P, H, S, C, layout, bits):
    Pi_v = np.stack([synth.haar_rotation(rng, D) for _ in range(H)])
    cb = codebook_fp32(D, C)
    idx = rng.integers(0, C, size=(P, S, D)).astype(np.uint8)
    norm = rng.uniform(0.3, 3.0, size=(P, S)) * np.sqrt(D)
    if layout == "unpacked":
        n = norm.astype(np.float32)
        return tq.Values("unpacked", t(idx), t(n)), idx, n.astype(np.float64), Pi_v, cb
    n = opk.gamma_to_half(norm)
    return tq.Values("packed", t(opk.pack_indices(idx, bits)), t(n), bits), idx, n.astype(np.float64), Pi_v, cb


def run(seed, P, H, B, S, key_fmt, val_fmt, scale, modes=("fused", "two_pass", "auto")):
    rng = np.random.default_rng(seed)
    klay, kbits, kC = key_fmt
    vlay, vbits, vC = val_fmt
    idx_u, sign_u, gamma, gi, gs = random_codes(rng, P, S, D, kC, klay, kbits)
    keys = keys_to_gpu(klay, kbits, gi, gs, gamma)
    cbk = codebook_fp32(D, kC)
    A = (rng.standard_normal((P, B, D)) * 0.5).astype(np.float32)
    Tq = (rng.standard_normal((P, B, D)) * 0.5).astype(np.float32)
    vals, vidx, vnorm, Pi_v, cbv = values_case(rng, P, H, S, vC, vlay, vbits)
    scores = oracle_scores_transformed(A, Tq, idx_u, sign_u, gamma, cbk)
    ref = np.stack([oa.attend_rotated(scores[p], vidx[p], vnorm[p], Pi_v[p % H].astype(np.float64),
                                      cbv.astype(np.float64), scale) for p in range(P)])
    for mode in modes:
        got = tq.tq_score_attend(t(A), t(Tq), keys, t(cbk), vals, t(cbv), t(Pi_v), scale, mode=mode).cpu().numpy()
        err = rel_err(got, ref)
        assert err <= SCORE_TOL, f"{mode}: max rel err {err:.3e}"


KEY_FMTS = [("unpacked", 0, 4), ("packed", 2, 4), ("packed", 3, 8)]
VAL_FMTS = [("unpacked", 0, 4), ("packed", 2, 4), ("packed", 3, 8)]


@pytest.mark.parametrize("key_fmt", KEY_FMTS)
@pytest.mark.parametrize("val_fmt", VAL_FMTS)
def test_fused_formats(key_fmt, val_fmt):
    say(f"fused keys {key_fmt} values {val_fmt}")
    run(7, 2, 2, 9, 1000, key_fmt, val_fmt, 0.7)


@pytest.mark.parametrize("P,H,B,S", [(1, 1, 1, 1), (1, 1, 32, 32), (1, 1, 33, 129), (1, 1, 5, 5000),
                                     (4, 2, 70, 300), (1, 1, 32, 70000), (3, 3, 2, 31)])
def test_fused_shapes(P, H, B, S):
    say(f"fused shape P={P} H={H} B={B} S={S}")
    run(S + B, P, H, B, S, ("packed", 3, 8), ("packed", 3, 8), 1.0 / np.sqrt(D))


@pytest.mark.parametrize("scale", [0.0, 3.0, -1.0])
def test_fused_scales(scale):
    say(f"fused scale={scale}")
    run(11, 1, 1, 8, 600, ("unpacked", 0, 4), ("unpacked", 0, 4), scale)


def test_fused_matches_two_calls():
    """The fused step against tq_score then tq_attend on the same inputs (both GPU)."""
    say("fused vs score then attend")
    rng = np.random.default_rng(5)
    P, H, B, S = 2, 1, 16, 3000
    idx_u, sign_u, gamma, gi, gs = random_codes(rng, P, S, D, 8, "packed", 3)
    keys = keys_to_gpu("packed", 3, gi, gs, gamma)
    cbk = codebook_fp32(D, 8)
    A = rng.standard_normal((P, B, D)).astype(np.float32)
    Tq = rng.standard_normal((P, B, D)).astype(np.float32)
    vals, vidx, vnorm, Pi_v, cbv = values_case(rng, P, H, S, 4, "packed", 2)
    fused = tq.tq_score_attend(t(A), t(Tq), keys, t(cbk), vals, t(cbv), t(Pi_v), 0.3, mode="fused").cpu().numpy()
    sc = tq.tq_score(t(A), t(Tq), keys, t(cbk))
    two = tq.tq_attend(sc, vals, t(cbv), t(Pi_v), 0.3).cpu().numpy()
    assert rel_err(fused, two) <= 2 * SCORE_TOL


@pytest.mark.parametrize("name", ["decode", "packed", "gqa", "long"])
def test_fused_workload_sizes(name):
    """Each workload's full shape: its keys' layout and codebook, values in the
    same layout and codebook size."""
    w = synth.workload(name)
    say(f"fused workload {name}: P={w.P} B={w.B} S={w.S} {w.layout}")
    bits = w.bits if w.layout == "packed" else 0
    run(w.seed, w.P, w.H, w.B, w.S, (w.layout, bits, w.C), (w.layout, bits, w.C), 1.0 / np.sqrt(D))
