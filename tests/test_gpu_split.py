"""The outlier split against the oracle (oracle.split): the split query
transform and scores against two-instance keys, for several instance layouts
and widths, ragged shapes, problems and heads, and a workload-sized case.
Keys are compressed by the oracle; the oracle scores the exact fp32 A (and
fp32 or fp16 norms) the GPU is given. Bar: max |gpu - exact| / (1 + |exact|)
<= 1e-4."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import compressed_attention_scoring_amd as tq
import synth
from oracle import pack as opk
from oracle import split as osp
from oracle.codebook import codebook_fp32
from tests.gpu_util import SCORE_TOL, rel_err, say, t

pytestmark = pytest.mark.gpu


def instance_to_gpu(idx, rho, layout, bits):
    if layout == "unpacked":
        r = rho.astype(np.float32)
        return tq.Values("unpacked", t(idx), t(r)), r.astype(np.float64)
    r = opk.gamma_to_half(rho)
    return tq.Values("packed", t(opk.pack_indices(idx, bits)), t(r), bits), r.astype(np.float64)


def split_case(seed, P, H, S, D, d_hi, hi_fmt, lo_fmt, nc=False):
    """hi_fmt / lo_fmt: (layout, bits, C). Returns GPU keys, oracle codes, rotations, codebooks, perm."""
    rng = np.random.default_rng([seed, 21])
    keys = [synth.unit_keys(rng, S, D, "outlier") * rng.uniform(0.5, 2.0, (S, 1)) for _ in range(P)]
    perm = osp.channel_permutation(D, osp.choose_hot_channels(np.concatenate(keys), d_hi))
    Pi_hi = np.stack([synth.haar_rotation(rng, d_hi) for _ in range(H)])
    Pi_lo = np.stack([synth.haar_rotation(rng, D - d_hi) for _ in range(H)])
    cb_hi = codebook_fp32(d_hi, hi_fmt[2])
    cb_lo = codebook_fp32(D - d_hi, lo_fmt[2])
    codes = [osp.compress_split(keys[p], perm, d_hi, Pi_hi[p % H], Pi_lo[p % H], cb_hi.astype(np.float64),
                                cb_lo.astype(np.float64), nc) for p in range(P)]
    ih = np.stack([c[0] for c in codes])
    il = np.stack([c[2] for c in codes])
    gh, rh = instance_to_gpu(ih, np.stack([c[1] for c in codes]), hi_fmt[0], hi_fmt[1])
    gl, rl = instance_to_gpu(il, np.stack([c[3] for c in codes]), lo_fmt[0], lo_fmt[1])
    return tq.SplitKeys(gh, gl), (ih, rh, il, rl), Pi_hi, Pi_lo, cb_hi, cb_lo, perm


@pytest.mark.parametrize("P,H,B,D,d_hi", [(1, 1, 1, 128, 32), (2, 2, 9, 128, 32), (4, 2, 33, 64, 16),
                                          (1, 1, 5, 256, 96),
                                          # matrix-core form: 16-row tiles across a head's problems,
                                          # the largest instance (15 wavefronts), partial query tiles
                                          (8, 2, 3, 128, 32), (1, 1, 4, 256, 16), (3, 3, 17, 96, 48),
                                          (16, 8, 4, 128, 32),
                                          # instance sizes that are not multiples of 16: the vector form
                                          (1, 1, 3, 128, 20), (2, 1, 5, 40, 8)])
def test_query_transform_split(P, H, B, D, d_hi):
    say(f"split transform P={P} H={H} B={B} D={D} d_hi={d_hi}")
    rng = np.random.default_rng(D + B)
    perm = osp.channel_permutation(D, rng.choice(D, d_hi, replace=False))
    Pi_hi = np.stack([synth.haar_rotation(rng, d_hi) for _ in range(H)])
    Pi_lo = np.stack([synth.haar_rotation(rng, D - d_hi) for _ in range(H)])
    q = synth.queries(B, P, B, D)
    A_hi, A_lo = tq.tq_query_transform_split(t(q), t(perm), t(Pi_hi), t(Pi_lo))
    for p in range(P):
        rh, rl = osp.query_transform_split(q[p], perm, d_hi, Pi_hi[p % H], Pi_lo[p % H])
        assert rel_err(A_hi[p].cpu().numpy(), rh) <= 1e-5
        assert rel_err(A_lo[p].cpu().numpy(), rl) <= 1e-5


FORMATS = [
    # (hot instance), (other instance), D, d_hi
    (("packed", 3, 8), ("packed", 2, 4), 128, 32),
    (("unpacked", 0, 8), ("unpacked", 0, 4), 128, 32),
    (("packed", 3, 8), ("unpacked", 0, 4), 128, 32),
    (("unpacked", 0, 16), ("packed", 3, 8), 128, 64),
    (("packed", 2, 4), ("packed", 2, 4), 64, 8),
]


@pytest.mark.parametrize("hi_fmt,lo_fmt,D,d_hi", FORMATS)
@pytest.mark.parametrize("P,H,B,S", [(1, 1, 1, 1), (1, 1, 3, 255), (2, 2, 9, 1000), (1, 1, 40, 777)])
def test_score_split_matches_oracle(hi_fmt, lo_fmt, D, d_hi, P, H, B, S):
    say(f"score_split {hi_fmt} {lo_fmt} D={D} d_hi={d_hi} P={P} B={B} S={S}")
    keys, (ih, rh, il, rl), Pi_hi, Pi_lo, cb_hi, cb_lo, perm = split_case(S + B, P, H, S, D, d_hi, hi_fmt, lo_fmt)
    rng = np.random.default_rng(S)
    A_hi = rng.standard_normal((P, B, d_hi)).astype(np.float32)
    A_lo = rng.standard_normal((P, B, D - d_hi)).astype(np.float32)
    got = tq.tq_score_split(t(A_hi), t(A_lo), keys, t(cb_hi), t(cb_lo)).cpu().numpy()
    ref = np.stack([osp.scores_split_from_transformed(A_hi[p].astype(np.float64), ih[p], rh[p], cb_hi,
                                                      A_lo[p].astype(np.float64), il[p], rl[p], cb_lo)
                    for p in range(P)])
    assert rel_err(got, ref) <= SCORE_TOL


@pytest.mark.parametrize("P,H,B,S", [(1, 1, 64, 1000), (2, 1, 130, 333), (1, 1, 256, 4099), (3, 3, 33, 70000),
                                     (16, 8, 4, 65537), (8, 1, 1, 131075), (32, 4, 3, 32769)])
def test_score_split_matrix_core_shapes(P, H, B, S):
    """The 2.5-bit setting (32 channels at 3 bits, 96 at 2, packed; the
    matrix-core forms) with one, two and four 32-query tiles per workgroup and,
    for up to four queries over 2^20 keys or more, the 16x16 tiles; ragged
    query and key counts."""
    say(f"score_split 2.5-bit P={P} B={B} S={S}")
    rng = np.random.default_rng([P, B, S])
    ih = rng.integers(0, 8, size=(P, S, 32), dtype=np.uint8)
    il = rng.integers(0, 4, size=(P, S, 96), dtype=np.uint8)
    gh, rh = instance_to_gpu(ih, rng.uniform(0.05, 1.5, (P, S)), "packed", 3)
    gl, rl = instance_to_gpu(il, rng.uniform(0.3, 2.0, (P, S)), "packed", 2)
    cb_hi, cb_lo = codebook_fp32(32, 8), codebook_fp32(96, 4)
    A_hi = (rng.standard_normal((P, B, 32)) * 4.0).astype(np.float32)
    A_lo = rng.standard_normal((P, B, 96)).astype(np.float32)
    got = tq.tq_score_split(t(A_hi), t(A_lo), tq.SplitKeys(gh, gl), t(cb_hi), t(cb_lo)).cpu().numpy()
    ref = np.stack([osp.scores_split_from_transformed(A_hi[p].astype(np.float64), ih[p], rh[p], cb_hi,
                                                      A_lo[p].astype(np.float64), il[p], rl[p], cb_lo)
                    for p in range(P)])
    assert rel_err(got, ref) <= SCORE_TOL


@pytest.mark.parametrize("nc", [False, True])
def test_split_end_to_end_equals_reconstruction(nc):
    say(f"split transform then score, nc={nc}")
    P, H, B, S, D = 2, 2, 7, 900, 128
    keys, (ih, rh, il, rl), Pi_hi, Pi_lo, cb_hi, cb_lo, perm = split_case(3, P, H, S, D, 32, ("packed", 3, 8),
                                                                          ("packed", 2, 4), nc)
    q = synth.queries(3, P, B, D)
    A_hi, A_lo = tq.tq_query_transform_split(t(q), t(perm), t(Pi_hi), t(Pi_lo))
    got = tq.tq_score_split(A_hi, A_lo, keys, t(cb_hi), t(cb_lo)).cpu().numpy()
    for p in range(P):
        ref = osp.scores_split_by_reconstruction(q[p].astype(np.float64), perm, 32, ih[p], rh[p], Pi_hi[p % H],
                                                 cb_hi, il[p], rl[p], Pi_lo[p % H], cb_lo)
        assert rel_err(got[p], ref) <= SCORE_TOL


def test_split_decode_workload_size():
    """The decode shape (B=32, S=32768, D=128) with the 32 + 96 split at 3 + 2
    bits: every score of a sample of keys."""
    say("score_split decode shape")
    P, B, S, D, d_hi = 1, 32, 32768, 128, 32
    rng = np.random.default_rng(9)
    ih = rng.integers(0, 8, size=(P, S, d_hi), dtype=np.uint8)
    il = rng.integers(0, 4, size=(P, S, D - d_hi), dtype=np.uint8)
    gh, rh = instance_to_gpu(ih, rng.uniform(0.1, 1.0, (P, S)), "packed", 3)
    gl, rl = instance_to_gpu(il, rng.uniform(0.5, 2.0, (P, S)), "packed", 2)
    cb_hi, cb_lo = codebook_fp32(d_hi, 8), codebook_fp32(D - d_hi, 4)
    A_hi = rng.standard_normal((P, B, d_hi)).astype(np.float32)
    A_lo = rng.standard_normal((P, B, D - d_hi)).astype(np.float32)
    got = tq.tq_score_split(t(A_hi), t(A_lo), tq.SplitKeys(gh, gl), t(cb_hi), t(cb_lo)).cpu().numpy()
    sample = np.unique(np.concatenate([np.arange(0, S, 37), [S - 1]]))
    ref = osp.scores_split_from_transformed(A_hi[0].astype(np.float64), ih[0][sample], rh[0][sample], cb_hi,
                                            A_lo[0].astype(np.float64), il[0][sample], rl[0][sample], cb_lo)
    assert rel_err(got[0][:, sample], ref) <= SCORE_TOL
    torch.cuda.synchronize()
