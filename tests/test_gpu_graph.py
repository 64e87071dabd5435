"""The entry points captured in HIP graphs (as the benchmark replays them): every
replay, with eager work and synchronisations between replays, must reproduce
the eager result exactly (same kernels, same inputs). The scoring path, the
fused decode step and tq_attend with their workspaces, the MSE-only and the
outlier-split paths."""

import numpy as np
import pytest
import torch

import compressed_attention_scoring_amd as tq
import synth
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["decode", "gqa"])
def test_graph_replays_match_eager(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = synth.workload(name)
    S = 4096
    say(f"graph replay {name} S={S}")
    Pi, S_mat = synth.head_matrices(w.seed, w.H, w.D)
    cb = torch.from_numpy(synth.timing_codebook(w.seed, w.C, w.D)).to(dev())
    sets = []
    for k in range(2):
        idx, sign, gamma = synth.timing_code_streams(w.seed + k, w.P, S, w.D, w.C, w.layout, w.bits)
        q = synth.queries(w.seed + k, w.P, w.B, w.D)
        s = {"q": torch.from_numpy(q).to(dev()),
             "keys": tq.Keys(w.layout, torch.from_numpy(idx).to(dev()), torch.from_numpy(sign).to(dev()),
                             torch.from_numpy(gamma).to(dev()), w.bits if w.layout == "packed" else 0),
             "A": torch.empty((w.P, w.B, w.D), device=dev()),
             "T": torch.empty((w.P, w.B, w.D), device=dev()),
             "out": torch.empty((w.P, w.B, S), device=dev())}
        sets.append(s)
    Pi_t, S_t = torch.from_numpy(Pi).to(dev()), torch.from_numpy(S_mat).to(dev())

    def step(s):
        tq.tq_query_transform(s["q"], Pi_t, S_t, s["A"], s["T"])
        tq.tq_score(s["A"], s["T"], s["keys"], cb, s["out"])

    for s in sets:
        step(s)
    torch.cuda.synchronize()
    eager = [s["out"].clone() for s in sets]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in sets:
            step(s)
    for r in range(4):
        for s in sets:
            s["out"].fill_(float("nan"))
        # eager work of the program's own between replays
        scratch = torch.empty_like(sets[0]["out"])
        tq.tq_score(sets[0]["A"], sets[0]["T"], sets[0]["keys"], cb, scratch)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s, ref in zip(sets, eager):
            assert torch.equal(s["out"], ref), f"replay {r} differs from eager"
        assert torch.equal(scratch, eager[0])


def _replays_match(step, outputs, disturb):
    """Run `step` eagerly, capture it, then replay it 4 times with eager work
    (`disturb`) and synchronisations between the replays; every replay must
    reproduce the eager outputs bit for bit."""
    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        for o in outputs:
            o.fill_(float("nan"))
        disturb()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outputs, eager):
            assert torch.equal(o, ref), f"replay {r} differs from eager"


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


@pytest.mark.parametrize("mode", ["fused", "two_pass"])
def test_score_attend_replays_match_eager(mode):
    """tq_score_attend (both forms, workspace reused) and tq_attend in a graph."""
    say(f"graph replay score_attend {mode}")
    P, H, B, S, D = 2, 2, 32, 3000, 128
    idx, sign, gamma = synth.timing_code_streams(11, P, S, D, 8, "packed", 3)
    keys = tq.Keys("packed", _t(idx), _t(sign), _t(gamma), 3)
    vi, vn = synth.timing_value_streams(11, P, S, D, 4, "packed", 2)
    vals = tq.Values("packed", _t(vi), _t(vn), 2)
    cb = _t(synth.timing_codebook(11, 8, D))
    cbv = _t(synth.timing_codebook(12, 4, D))
    Pi_v = _t(synth.head_matrices(11, H, D)[0])
    rng = np.random.default_rng(3)
    A = _t(rng.standard_normal((P, B, D)).astype(np.float32))
    T = _t(rng.standard_normal((P, B, D)).astype(np.float32))
    out = torch.empty((P, B, D), device=dev())
    ws = torch.empty(tq.tq_score_attend_workspace_bytes(P, B, S, D, mode), dtype=torch.uint8, device=dev())
    scores = _t(synth.timing_scores(11, P, B, S))
    out2 = torch.empty((P, B, D), device=dev())
    ws2 = torch.empty(tq.tq_attend_workspace_bytes(P, B, S, D), dtype=torch.uint8, device=dev())
    scratch = torch.empty((P, B, D), device=dev())

    def step():
        tq.tq_score_attend(A, T, keys, cb, vals, cbv, Pi_v, 0.2, out=out, workspace=ws, mode=mode)
        tq.tq_attend(scores, vals, cbv, Pi_v, 0.5, out=out2, workspace=ws2)

    _replays_match(step, [out, out2], lambda: tq.tq_attend(scores, vals, cbv, Pi_v, 0.5, out=scratch))


def test_mse_and_split_replay_match_eager():
    """The MSE-only and outlier-split paths (transforms and scorers) in a graph,
    on shapes that take the 16x16 and the 32x32 matrix-core forms."""
    say("graph replay mse and split")
    D = 128
    signs = _t(np.where(np.random.default_rng(1).random((1, D)) < 0.5, -1.0, 1.0).astype(np.float32))
    perm = _t(np.concatenate([np.arange(0, D, 4), np.setdiff1d(np.arange(D), np.arange(0, D, 4))]).astype(np.int32))
    rng = np.random.default_rng(2)
    Pi_hi = _t(synth.haar_rotation(rng, 32)[None])
    Pi_lo = _t(synth.haar_rotation(rng, 96)[None])
    cases = []
    for (P, B, S) in [(8, 4, 131075), (1, 40, 3001)]:
        q = _t(synth.queries(P + B, P, B, D))
        mi, mn = synth.timing_value_streams(5, P, S, D, 8, "packed", 3)
        mkeys = tq.Values("packed", _t(mi), _t(mn), 3)
        ih, nh = synth.timing_value_streams(6, P, S, 32, 8, "packed", 3)
        il, nl = synth.timing_value_streams(7, P, S, 96, 4, "packed", 2)
        skeys = tq.SplitKeys(tq.Values("packed", _t(ih), _t(nh), 3), tq.Values("packed", _t(il), _t(nl), 2))
        c = {"q": q, "mkeys": mkeys, "skeys": skeys, "A": torch.empty((P, B, D), device=dev()),
             "Ah": torch.empty((P, B, 32), device=dev()), "Al": torch.empty((P, B, 96), device=dev()),
             "ms": torch.empty((P, B, S), device=dev()), "ss": torch.empty((P, B, S), device=dev())}
        cases.append(c)
    cb8 = _t(synth.timing_codebook(5, 8, D))
    cbh, cbl = _t(synth.timing_codebook(6, 8, 32)), _t(synth.timing_codebook(7, 4, 96))

    def step():
        for c in cases:
            tq.tq_query_transform_hadamard(c["q"], signs, A=c["A"])
            tq.tq_score_mse(c["A"], c["mkeys"], cb8, scores=c["ms"])
            tq.tq_query_transform_split(c["q"], perm, Pi_hi, Pi_lo, A_hi=c["Ah"], A_lo=c["Al"])
            tq.tq_score_split(c["Ah"], c["Al"], c["skeys"], cbh, cbl, scores=c["ss"])

    outs = [c[k] for c in cases for k in ("A", "ms", "Ah", "Al", "ss")]
    scratch = torch.empty_like(cases[1]["ss"])
    _replays_match(step, outs, lambda: tq.tq_score_split(cases[1]["Ah"], cases[1]["Al"], cases[1]["skeys"],
                                                         cbh, cbl, scores=scratch))
