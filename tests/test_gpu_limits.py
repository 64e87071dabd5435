"""The size limits the C ABI states, at the limit and one past it.

tq_score's matrix-core family takes S < 2^24 keys per problem: S = 2^24 - 1
must run there, and S = 2^24 must be refused by it (TQ_ERR_UNSUPPORTED) while
the automatic choice hands it to the vector family. B <= 262144 queries and
P <= 65535 problems: the largest must run, the next must be refused.
Outputs are compared with the oracle on sampled entries that include every
edge the shapes have (first and last key and query, the ragged last tile);
transforms are checked row by row against the fp32 dot-product bound.
"""

import numpy as np
import pytest
import torch

import compressed_attention_scoring_amd as tq
import synth
from oracle import pack as opk
from oracle import query_transform as oqt
from oracle import score as osc
from tests.gpu_util import SCORE_TOL, dev, rel_err, say, t

pytestmark = pytest.mark.gpu

MAX_KEYS = 1 << 24


def _sample(n, extra, rng, edges=(0, 1, 31, 32, 33)):
    pick = [e for e in edges if e < n] + [n - 1 - e for e in edges if n - 1 - e >= 0]
    pick += list(rng.choice(n, min(extra, n), replace=False))
    return np.unique(np.array(pick, dtype=np.int64))


@pytest.fixture(scope="module")
def long_keys():
    """2^24 packed 3-bit keys at D = 128 (1.1 GB on the GPU) and their host copies."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    D, C = 128, 8
    say(f"limits: generating {MAX_KEYS} packed keys")
    idx, sign, gamma = synth.timing_code_streams(77, 1, MAX_KEYS, D, C, "packed", 3)
    cb = synth.timing_codebook(77, C, D)
    g = {"idx": t(idx), "sign": t(sign), "gamma": t(gamma), "cb": t(cb)}
    yield idx, sign, gamma, cb, g
    del g
    torch.cuda.empty_cache()


def _check_sampled(scores, A, T, idx, sign, gamma, cb, rng, D=128, bits=3):
    S = scores.shape[-1]
    sel = _sample(S, 1500, rng)
    got = scores[0][:, torch.from_numpy(sel).to(scores.device)].cpu().numpy()
    idx_u = opk.unpack_indices(idx[0][sel], bits, D)
    sign_u = opk.unpack_signs(sign[0][sel], D)
    ref = osc.scores_from_transformed(A[0], T[0], idx_u, sign_u, gamma[0][sel].astype(np.float64), cb)
    return rel_err(got, ref)


def test_score_largest_key_count(long_keys):
    idx, sign, gamma, cb, g = long_keys
    S, B, D = MAX_KEYS - 1, 33, 128
    name = tq.tq_score_kernel_name("packed", 3, 8, 1, B, S, D)
    assert name is not None and name.startswith("mfma"), name
    rng = np.random.default_rng(5)
    A = rng.standard_normal((1, B, D)).astype(np.float32)
    T = rng.standard_normal((1, B, D)).astype(np.float32)
    keys = tq.Keys("packed", g["idx"][:, :S], g["sign"][:, :S], g["gamma"][:, :S], 3)
    say(f"limits: tq_score S={S} B={B} kernel {name}")
    scores = tq.tq_score(t(A), t(T), keys, g["cb"])
    torch.cuda.synchronize()
    assert _check_sampled(scores, A, T, idx, sign, gamma, cb, rng) <= SCORE_TOL


def test_score_key_count_past_matrix_cores(long_keys):
    idx, sign, gamma, cb, g = long_keys
    S, B, D = MAX_KEYS, 3, 128
    assert tq.tq_score_kernel_name("packed", 3, 8, 1, B, S, D, "mfma_lds") is None
    name = tq.tq_score_kernel_name("packed", 3, 8, 1, B, S, D)
    assert name is not None and not name.startswith("mfma"), name
    rng = np.random.default_rng(6)
    A = rng.standard_normal((1, B, D)).astype(np.float32)
    T = rng.standard_normal((1, B, D)).astype(np.float32)
    keys = tq.Keys("packed", g["idx"], g["sign"], g["gamma"], 3)
    say(f"limits: tq_score S={S} B={B}: matrix cores refuse, automatic choice {name}")
    with pytest.raises(tq.TqError) as e:
        tq.tq_score_with_kernel(t(A), t(T), keys, g["cb"], "mfma_lds")
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
    scores = tq.tq_score(t(A), t(T), keys, g["cb"])
    torch.cuda.synchronize()
    assert _check_sampled(scores, A, T, idx, sign, gamma, cb, rng) <= SCORE_TOL


def _transform_rows_ok(q, Pi, Sm, A, T, rows):
    """Rows of the GPU's A, T against the oracle, within the fp32 dot-product bound."""
    rA, rT = oqt.transform_one(q[rows], Pi, Sm)
    for got, ref, W in ((A[rows], rA, Pi), (T[rows], rT, Sm)):
        bound = (np.abs(q[rows].astype(np.float64)) @ np.abs(W.astype(np.float64)).T) * W.shape[1] * 2.0 ** -24 * 1.01
        assert np.all(np.abs(got - ref) <= bound + 1e-30)


def test_largest_query_count():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P, B, S, D, C = 1, 262144, 37, 128, 4
    rng = np.random.default_rng(7)
    Pi, Sm = synth.head_matrices(7, 1, D)
    q = rng.standard_normal((P, B, D)).astype(np.float32)
    say(f"limits: transform and score B={B} S={S} unpacked")
    A, T = tq.tq_query_transform(t(q), t(Pi), t(Sm))
    idx, sign, gamma = synth.timing_code_streams(7, P, S, D, C, "unpacked", 0)
    cb = synth.timing_codebook(7, C, D)
    keys = tq.Keys("unpacked", t(idx), t(sign), t(gamma))
    scores = tq.tq_score(A, T, keys, t(cb))
    torch.cuda.synchronize()
    rows = _sample(B, 300, rng)
    A_h = A[0][torch.from_numpy(rows).to(dev())].cpu().numpy()
    T_h = T[0][torch.from_numpy(rows).to(dev())].cpu().numpy()
    _transform_rows_ok(q[0], Pi[0], Sm[0], A[0].cpu().numpy(), T[0].cpu().numpy(), rows)
    got = scores[0][torch.from_numpy(rows).to(dev())].cpu().numpy()
    ref = osc.scores_from_transformed(A_h, T_h, idx[0], sign[0], gamma[0].astype(np.float64), cb)
    assert rel_err(got, ref) <= SCORE_TOL
    say(f"limits: tq_score B={B + 1} must be refused")
    A1 = torch.zeros((1, B + 1, D), device=dev())
    with pytest.raises(tq.TqError) as e:
        tq.tq_score(A1, A1, keys, t(cb))
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED


def test_largest_problem_count():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P, H, B, S, D, C = 65535, 5, 3, 5, 64, 4
    rng = np.random.default_rng(8)
    Pi, Sm = synth.head_matrices(8, H, D)
    q = rng.standard_normal((P, B, D)).astype(np.float32)
    idx, sign, gamma = synth.timing_code_streams(8, P, S, D, C, "packed", 2)
    cb = synth.timing_codebook(8, C, D)
    say(f"limits: transform and score P={P} H={H} B={B} S={S} packed 2-bit D={D}")
    A, T = tq.tq_query_transform(t(q), t(Pi), t(Sm))
    keys = tq.Keys("packed", t(idx), t(sign), t(gamma), 2)
    scores = tq.tq_score(A, T, keys, t(cb))
    torch.cuda.synchronize()
    probs = _sample(P, 60, rng, edges=(0, 1, 4, 5))
    A_h, T_h, s_h = A.cpu().numpy(), T.cpu().numpy(), scores.cpu().numpy()
    worst = 0.0
    for p in probs:
        h = p % H
        _transform_rows_ok(q[p], Pi[h], Sm[h], A_h[p], T_h[p], np.arange(B))
        ref = osc.scores_from_transformed(A_h[p], T_h[p], opk.unpack_indices(idx[p], 2, D),
                                          opk.unpack_signs(sign[p], D), gamma[p].astype(np.float64), cb)
        worst = max(worst, rel_err(s_h[p], ref))
    assert worst <= SCORE_TOL
    say(f"limits: P={P + 1} must be refused")
    q1 = torch.zeros((P + 1, 1, D), device=dev())
    Pi1 = t(np.stack([np.eye(D, dtype=np.float32)]))
    with pytest.raises(tq.TqError) as e:
        tq.tq_query_transform(q1, Pi1, Pi1)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
