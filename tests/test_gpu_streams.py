"""Stream semantics of the C ABI: every entry point enqueues its work on the
stream it is given and on no other.

- Each entry point run on a side stream gives, bit for bit, what it gives on
  the default stream.
- Ordering: on a side stream, a delay kernel followed by a write of new inputs
  and then the call; the call must see the new inputs (a launch on any other
  stream would run before the write and read the old ones).
- Two side streams scoring different batches at the same time give each
  batch's own result: the library keeps no state between calls.
All side streams have the default priority.
"""

import numpy as np
import pytest
import torch

import compressed_attention_scoring_amd as tq
import synth
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

DELAY_CYCLES = 20_000_000   # torch.cuda._sleep: a bounded spin of about 10 ms


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def _case(seed, P=2, H=2, B=33, S=3001, D=128):
    Pi, Sm = synth.head_matrices(seed, H, D)
    idx, sign, gamma = synth.timing_code_streams(seed, P, S, D, 8, "packed", 3)
    vi, vn = synth.timing_value_streams(seed, P, S, D, 4, "packed", 2)
    ih, nh = synth.timing_value_streams(seed + 1, P, S, 32, 8, "packed", 3)
    il, nl = synth.timing_value_streams(seed + 2, P, S, 96, 4, "packed", 2)
    rng = np.random.default_rng(seed)
    return {
        "q": _t(synth.queries(seed, P, B, D)), "Pi": _t(Pi), "S": _t(Sm),
        "keys": tq.Keys("packed", _t(idx), _t(sign), _t(gamma), 3),
        "vals": tq.Values("packed", _t(vi), _t(vn), 2),
        "split": tq.SplitKeys(tq.Values("packed", _t(ih), _t(nh), 3), tq.Values("packed", _t(il), _t(nl), 2)),
        "cb": _t(synth.timing_codebook(seed, 8, D)), "cbv": _t(synth.timing_codebook(seed + 1, 4, D)),
        "cbh": _t(synth.timing_codebook(seed + 2, 8, 32)), "cbl": _t(synth.timing_codebook(seed + 3, 4, 96)),
        "signs": _t(np.where(rng.random((H, D)) < 0.5, -1.0, 1.0).astype(np.float32)),
        "perm": _t(rng.permutation(D).astype(np.int32)),
        "Pih": _t(np.stack([synth.haar_rotation(rng, 32) for _ in range(H)])),
        "Pil": _t(np.stack([synth.haar_rotation(rng, 96) for _ in range(H)])),
        "kf": _t(rng.standard_normal((P, S, D)).astype(np.float32)),
    }


def _run_all(c, stream):
    """Every entry point once on `stream`; returns the outputs in a fixed order."""
    outs = []
    A, T = tq.tq_query_transform(c["q"], c["Pi"], c["S"], stream=stream)
    outs += [A, T]
    outs.append(tq.tq_score(A, T, c["keys"], c["cb"], stream=stream))
    for kernel in ("valu", "mfma_lds", "mfma_reg"):
        outs.append(tq.tq_score_with_kernel(A, T, c["keys"], c["cb"], kernel, stream=stream))
    outs.append(tq.tq_score_attend(A, T, c["keys"], c["cb"], c["vals"], c["cbv"], c["Pi"], 0.2, stream=stream,
                                   mode="fused"))
    outs.append(tq.tq_score_attend(A, T, c["keys"], c["cb"], c["vals"], c["cbv"], c["Pi"], 0.2, stream=stream,
                                   mode="two_pass"))
    outs.append(tq.tq_attend(outs[2], c["vals"], c["cbv"], c["Pi"], 0.3, stream=stream))
    Ah = tq.tq_query_transform_hadamard(c["q"], c["signs"], stream=stream)
    outs += [Ah, tq.tq_score_mse(Ah, c["vals"], c["cbv"], stream=stream)]
    Ahi, Alo = tq.tq_query_transform_split(c["q"], c["perm"], c["Pih"], c["Pil"], stream=stream)
    outs += [Ahi, Alo, tq.tq_score_split(Ahi, Alo, c["split"], c["cbh"], c["cbl"], stream=stream)]
    k2 = tq.tq_compress_keys(c["kf"], c["Pi"], c["S"], c["cb"], "packed", 3, stream=stream)
    outs += [k2.idx, k2.sign, k2.gamma]
    outs += list(tq.tq_decode_debug(c["keys"], 128, stream=stream))
    return outs


def test_side_stream_matches_default_stream():
    c = _case(3)
    say("streams: every entry point on the default stream")
    ref = [o.clone() for o in _run_all(c, None)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    say("streams: every entry point on a side stream")
    with torch.cuda.stream(side):
        got = _run_all(c, side)
    side.synchronize()
    assert len(got) == len(ref)
    for k, (g, r) in enumerate(zip(got, ref)):
        assert torch.equal(g, r), f"output {k} differs between streams"


def test_call_is_ordered_after_earlier_work_on_its_stream():
    c = _case(4)
    q_new = _t(synth.queries(99, 2, 33, 128))
    A_ref, T_ref = tq.tq_query_transform(q_new, c["Pi"], c["S"])
    s_ref = tq.tq_score(A_ref, T_ref, c["keys"], c["cb"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    q = c["q"].clone()
    torch.cuda.synchronize()
    say("streams: delay, input write and call on one side stream")
    with torch.cuda.stream(side):
        A = torch.empty_like(q)
        T = torch.empty_like(q)
        scores = torch.empty_like(s_ref)
        torch.cuda._sleep(DELAY_CYCLES)
        q.copy_(q_new)
        tq.tq_query_transform(q, c["Pi"], c["S"], A, T, stream=side)
        tq.tq_score(A, T, c["keys"], c["cb"], scores, stream=side)
    side.synchronize()
    assert torch.equal(A, A_ref) and torch.equal(T, T_ref)
    assert torch.equal(scores, s_ref)


def test_two_streams_at_once():
    cases = [_case(5), _case(6)]
    refs = []
    for c in cases:
        A, T = tq.tq_query_transform(c["q"], c["Pi"], c["S"])
        refs.append(tq.tq_score(A, T, c["keys"], c["cb"]).clone())
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    say("streams: two side streams, 20 steps each, interleaved launches")
    for it in range(20):
        for k, (c, s) in enumerate(zip(cases, streams)):
            with torch.cuda.stream(s):
                A, T = tq.tq_query_transform(c["q"], c["Pi"], c["S"], stream=s)
                outs[k].append(tq.tq_score(A, T, c["keys"], c["cb"], stream=s))
    for s in streams:
        s.synchronize()
    for k in range(2):
        for it, o in enumerate(outs[k]):
            assert torch.equal(o, refs[k]), f"stream {k} step {it} differs"
