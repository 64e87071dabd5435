"""The hot path captured in a HIP graph (as the benchmark replays it): every
replay, with eager work and synchronisations between replays, must reproduce
the eager result exactly (same kernels, same inputs)."""

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
