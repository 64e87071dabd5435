"""The single-pass f16 form of the matrix-core scorer (kernel family
"mfma_f16", TQ_KERNEL_MFMA_F16): every score within the reported bar of
2e-2 * (1 + |exact|) of the oracle, on ragged shapes that reach each of its
kernel forms (LDS-staged with one, two and four query tiles, the 16x16 four-query
form, the shared-decode form) and at the five workloads' full sizes. The split
forms' 1e-4 bar is not asked of it; the test also records how far it stays
inside 2e-2."""

import math
import zlib

import numpy as np
import pytest
import torch

import compressed_attention_scoring_amd as tq
import synth
from oracle import query_transform as oqt
from oracle import score as osc
from oracle import workload as ow
from tests.gpu_util import keys_to_gpu, oracle_scores_transformed, random_codes, rel_err, say, t

pytestmark = pytest.mark.gpu

F16_TOL = 2e-2


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = []
for layout, bits, C in (("unpacked", 0, 4), ("unpacked", 0, 8), ("packed", 2, 4), ("packed", 3, 8)):
    for D in ((32, 64, 128, 256) if layout == "unpacked" else (64, 128, 256)):
        for P, B, S in ((2, 1, 1), (2, 5, 257), (2, 32, 300), (1, 33, 64), (2, 96, 70), (1, 128, 95),
                        (1, 161, 40)):
            CASES.append((layout, bits, C, D, P, B, S))
# four queries over 2^20 keys or more: the 16x16 form
for layout, bits, C in (("unpacked", 0, 4), ("packed", 2, 4), ("packed", 3, 8)):
    CASES.append((layout, bits, C, 128, 4, 3, (1 << 18) + 5))
CASES.append(("packed", 3, 8, 256, 8, 4, (1 << 17) + 16))


@pytest.mark.parametrize("layout,bits,C,D,P,B,S", CASES)
def test_f16_random_codes(layout, bits, C, D, P, B, S):
    name = tq.tq_score_kernel_name(layout, bits, C, P, B, S, D, "mfma_f16")
    if name is None:
        pytest.skip("the f16 form does not cover this shape")
    say(f"f16 score {name}: {layout} bits={bits} C={C} D={D} P={P} B={B} S={S}")
    rng = np.random.default_rng(zlib.crc32(repr((layout, bits, C, D, P, B, S)).encode()))
    A = rng.standard_normal((P, B, D)).astype(np.float32)
    T = (rng.standard_normal((P, B, D)) * math.sqrt(D)).astype(np.float32)
    cb = np.sort(rng.standard_normal(C) / math.sqrt(D)).astype(np.float32)
    idx_u, sign_u, gamma_k, idx, sign = random_codes(rng, P, S, D, C, layout, bits)
    keys = keys_to_gpu(layout, bits, idx, sign, gamma_k)
    got = tq.tq_score_with_kernel(t(A), t(T), keys, t(cb), "mfma_f16").cpu().numpy()
    assert np.all(np.isfinite(got))
    ref = oracle_scores_transformed(A, T, idx_u, sign_u, gamma_k, cb)
    err = rel_err(got, ref)
    say(f"f16 score {name}: max rel err {err:.2e}")
    assert err <= F16_TOL


def test_f16_forms_follow_the_automatic_choice():
    n = tq.tq_score_kernel_name
    for w in (synth.workload(x) for x in ("tiny", "decode", "packed", "gqa", "long")):
        auto = n(w.layout, w.bits, w.C, w.P, w.B, w.S, w.D)
        f16 = n(w.layout, w.bits, w.C, w.P, w.B, w.S, w.D, "mfma_f16")
        # the integer four-query kernel (packed keys) has its f16 form in the f16 four-query kernel
        assert f16 == auto.replace("mfma16i8_", "mfma16_") + "_f16", (w.name, auto, f16)


@pytest.mark.parametrize("name", ["tiny", "decode", "packed", "gqa", "long"])
def test_f16_workload_full_size(name):
    w = synth.workload(name)
    say(f"f16 workload {name}: building inputs {w.describe()}")
    inp = ow.make_inputs(w)
    A, T = tq.tq_query_transform(t(inp.q), t(inp.Pi), t(inp.S_mat))
    keys = keys_to_gpu(w.layout, w.bits, inp.idx, inp.sign, inp.gamma_k)
    scores = tq.tq_score_with_kernel(A, T, keys, t(inp.codebook), "mfma_f16")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(scores).all())
    A64, T64 = oqt.query_transform(inp.q, inp.Pi, inp.S_mat)
    worst = 0.0
    for p in range(w.P):
        ref = osc.scores_from_transformed(A64[p], T64[p], inp.idx_u[p], inp.sign_u[p], inp.gamma_ref[p],
                                          inp.codebook)
        worst = max(worst, rel_err(scores[p].cpu().numpy(), ref))
    say(f"f16 workload {name}: max rel err {worst:.3e} over all {w.P * w.B * w.S} scores")
    assert worst <= F16_TOL
