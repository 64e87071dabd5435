"""tq_attend_no_alloc through the C ABI against tq_attend (the same kernels with
a caller workspace): two calls in a row, the second smaller than the first, each
equal to tq_attend's output bit for bit and within the fp32 bar of the oracle;
a shape whose workspace exceeds the fixed scratch is refused on the host."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import compressed_attention_scoring_amd as tq
from tests.gpu_util import SCORE_TOL, rel_err, say, t
from tests.test_gpu_attend import oracle_out, value_case

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def no_alloc_call(scores, vals, cb, Pi_v, scale, out):
    """The entry point called directly through ctypes: device pointers and sizes only."""
    P, B, S = scores.shape
    H, D = Pi_v.shape[0], Pi_v.shape[-1]
    cv, _, _ = vals._c(D)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return tq._lib.tq_attend_no_alloc(ctypes.c_void_p(scores.data_ptr()), ctypes.byref(cv),
                                      ctypes.c_void_p(cb.data_ptr()), cb.numel(), ctypes.c_void_p(Pi_v.data_ptr()),
                                      float(scale), ctypes.c_void_p(out.data_ptr()), P, H, B, S, D, st)


CASES = [
    # seed, P, H, B, S, D, C, layout, bits  (the second is smaller than the first)
    (61, 2, 2, 32, 20000, 128, 4, "packed", 2),
    (62, 1, 1, 5, 777, 64, 8, "unpacked", 0),
]


def test_no_alloc_matches_tq_attend_twice():
    for seed, P, H, B, S, D, C, layout, bits in CASES:
        say(f"tq_attend_no_alloc P={P} H={H} B={B} S={S} D={D} C={C} {layout}")
        vals, idx, norm, Pi_v, cb = value_case(seed, P, H, S, D, C, layout, bits)
        rng = np.random.default_rng([seed, 8])
        scores = (rng.standard_normal((P, B, S)) * 3.0).astype(np.float32)
        scale = 1.0 / np.sqrt(D)
        s_g, cb_g, Pv_g = t(scores), t(cb), t(Pi_v)
        ref_gpu = tq.tq_attend(s_g, vals, cb_g, Pv_g, scale)
        out = torch.full((P, B, D), float("nan"), dtype=torch.float32, device=s_g.device)
        rc = no_alloc_call(s_g, vals, cb_g, Pv_g, scale, out)
        assert rc == tq.TQ_OK, tq.tq_status_string(rc)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got, ref_gpu.cpu().numpy())
        ref = oracle_out(scores, idx, norm, Pi_v, cb, scale, H)
        assert rel_err(got, ref) <= SCORE_TOL


def test_no_alloc_refuses_more_than_the_scratch():
    # the most queries a call takes, over a thousand keys: about 130 MiB of partial records
    P, H, B, S, D = 1, 1, 262144, 1000, 128
    need = tq._lib.tq_attend_workspace_bytes(P, B, S, D)
    assert need > tq.TQ_NO_ALLOC_SCRATCH_BYTES
    dummy = torch.zeros(16, dtype=torch.float32, device="cuda:0")
    cv = tq._CValues(tq.TQ_UNPACKED, 0, dummy.data_ptr(), dummy.data_ptr())
    p = ctypes.c_void_p(dummy.data_ptr())
    rc = tq._lib.tq_attend_no_alloc(p, ctypes.byref(cv), p, 4, p, 0.1, p, P, H, B, S, D, None)
    assert rc == tq.TQ_ERR_UNSUPPORTED
