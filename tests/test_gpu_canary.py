"""Canary-guarded buffers: no entry point writes outside its outputs and
workspace, every output element is written, and no input is modified.

Each output (and workspace) is a view into a larger device buffer whose guard
regions before and after hold a sentinel byte. A call runs twice, with sentinel
0xA5 and then 0x5A filling guards, outputs and workspace: the guards must come
back untouched both times, and the outputs must agree bit for bit between the
two runs (an element never written would keep the sentinel and differ). The
guards span 64 rows of the output's last axis (a workspace: its own size), at
least 64 KiB and at most 64 MiB, so a tile that runs past the last query or
the last problem lands in them. Values themselves are checked against the
oracle elsewhere; this file checks only where the kernels write. Shapes are ragged (partial query tiles, key tails, odd problem counts)
and are chosen to reach every kernel form the dispatchers pick.
"""

import ctypes

import numpy as np
import pytest
import torch

import compressed_attention_scoring_amd as tq
import synth
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

SENTINELS = (0xA5, 0x5A)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


class Guarded:
    """A view of `shape` and `dtype` inside a byte buffer with guards on both sides."""

    def __init__(self, shape, dtype, written=True):
        self.shape, self.dtype, self.written = tuple(shape), dtype, written
        item = torch.empty((), dtype=dtype).element_size()
        self.nbytes = int(np.prod(self.shape, dtype=np.int64)) * item
        # 64 rows of the last axis (a workspace: its own size), 64 KiB to 64 MiB
        span = 64 * self.shape[-1] * item if len(self.shape) > 1 else self.nbytes
        self.guard = -(-min(max(span, 1 << 16), 1 << 26) // 256) * 256
        self.full = torch.empty(2 * self.guard + self.nbytes, dtype=torch.uint8, device=dev())
        self.view = self.full[self.guard:self.guard + self.nbytes].view(dtype).view(self.shape)

    def fill(self, byte):
        self.full.fill_(byte)

    def check_guards(self, byte, what):
        g, n = self.guard, self.nbytes
        head = torch.nonzero(self.full[:g] != byte)
        tail = torch.nonzero(self.full[g + n:] != byte)
        assert head.numel() == 0, f"{what}: write {g - int(head[0])} bytes before the buffer"
        assert tail.numel() == 0, f"{what}: write {int(tail[0])} bytes past the end of the buffer"

    def body(self):
        return self.full[self.guard:self.guard + self.nbytes].clone()


def run_guarded(call, outs, inputs, what):
    """Run `call()` once per sentinel over the guarded buffers `outs`; the
    guards must hold, outputs marked written must agree across the runs, and
    the tensors in `inputs` must be left as they were."""
    before = [x.clone() for x in inputs]
    bodies = []
    for byte in SENTINELS:
        for o in outs:
            o.fill(byte)
        torch.cuda.synchronize()
        call()
        torch.cuda.synchronize()
        for k, o in enumerate(outs):
            o.check_guards(byte, f"{what} buffer {k} (sentinel {byte:#x})")
        bodies.append([o.body() for o in outs])
    for k, o in enumerate(outs):
        if o.written:
            diff = torch.nonzero(bodies[0][k] != bodies[1][k])
            assert diff.numel() == 0, f"{what} buffer {k}: byte {int(diff[0])} of {o.nbytes} never written"
    for x, ref in zip(inputs, before):
        assert torch.equal(x, ref), f"{what}: an input was modified"


def keys_case(seed, P, S, D, C, layout, bits):
    idx, sign, gamma = synth.timing_code_streams(seed, P, S, D, C, layout, bits)
    return tq.Keys(layout, _t(idx), _t(sign), _t(gamma), bits)


def values_case(seed, P, S, D, C, layout, bits):
    idx, norm = synth.timing_value_streams(seed, P, S, D, C, layout, bits)
    return tq.Values(layout, _t(idx), _t(norm), bits)


def _keys_inputs(k):
    return [k.idx, k.sign, k.gamma]


def _values_inputs(v):
    return [v.idx, v.norm]


# ---------------------------------------------------------------------------
# transforms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("P,H,B,D", [(1, 1, 1, 128), (1, 1, 33, 128), (3, 3, 5, 64), (16, 8, 4, 128),
                                     (6, 2, 33, 64), (2, 1, 7, 256), (1, 1, 3, 40)])
def test_query_transform_guarded(P, H, B, D):
    say(f"canary query_transform P={P} H={H} B={B} D={D}")
    Pi, S_mat = synth.head_matrices(P + D, H, D)
    q, Pi, S_mat = _t(synth.queries(B, P, B, D)), _t(Pi), _t(S_mat)
    A, T = Guarded((P, B, D), torch.float32), Guarded((P, B, D), torch.float32)
    run_guarded(lambda: tq.tq_query_transform(q, Pi, S_mat, A.view, T.view), [A, T], [q, Pi, S_mat],
                "tq_query_transform")


@pytest.mark.parametrize("P,H,B,D", [(1, 1, 1, 128), (3, 3, 5, 64), (16, 8, 33, 128), (1, 1, 7, 256)])
def test_hadamard_transform_guarded(P, H, B, D):
    say(f"canary query_transform_hadamard P={P} H={H} B={B} D={D}")
    rng = np.random.default_rng(P * B + D)
    signs = _t(np.where(rng.random((H, D)) < 0.5, -1.0, 1.0).astype(np.float32))
    q = _t(synth.queries(D, P, B, D))
    A = Guarded((P, B, D), torch.float32)
    run_guarded(lambda: tq.tq_query_transform_hadamard(q, signs, A.view), [A], [q, signs],
                "tq_query_transform_hadamard")


@pytest.mark.parametrize("P,H,B", [(1, 1, 1), (8, 4, 4), (3, 1, 37)])
def test_split_transform_guarded(P, H, B):
    say(f"canary query_transform_split P={P} H={H} B={B}")
    D, Dh = 128, 32
    rng = np.random.default_rng(P + B)
    perm = _t(rng.permutation(D).astype(np.int32))
    Pi_hi = _t(np.stack([synth.haar_rotation(rng, Dh) for _ in range(H)]))
    Pi_lo = _t(np.stack([synth.haar_rotation(rng, D - Dh) for _ in range(H)]))
    q = _t(synth.queries(B, P, B, D))
    Ah, Al = Guarded((P, B, Dh), torch.float32), Guarded((P, B, D - Dh), torch.float32)
    run_guarded(lambda: tq.tq_query_transform_split(q, perm, Pi_hi, Pi_lo, Ah.view, Al.view), [Ah, Al],
                [q, perm, Pi_hi, Pi_lo], "tq_query_transform_split")


# ---------------------------------------------------------------------------
# tq_score: every kernel family the shape admits, and the automatic choice
# ---------------------------------------------------------------------------

SCORE_SHAPES = [
    # layout, bits, C, D, P, B, S
    ("unpacked", 0, 4, 128, 2, 5, 1001),
    ("unpacked", 0, 8, 256, 1, 96, 70),
    ("unpacked", 0, 4, 32, 3, 1, 33),
    ("packed", 3, 8, 128, 2, 33, 4099),
    ("packed", 3, 8, 128, 1, 161, 95),
    ("packed", 2, 4, 64, 3, 1, 257),
    ("packed", 3, 8, 128, 8, 4, 70001),
    ("packed", 2, 4, 256, 1, 128, 300),
    ("packed", 3, 8, 128, 2, 3, 0),
]


@pytest.mark.parametrize("kernel", ["auto", "valu", "mfma_lds", "mfma_reg", "mfma16", "mfma_shared"])
@pytest.mark.parametrize("layout,bits,C,D,P,B,S", SCORE_SHAPES)
def test_score_guarded(kernel, layout, bits, C, D, P, B, S):
    name = tq.tq_score_kernel_name(layout, bits, C, P, B, S, D, kernel)
    if name is None:
        pytest.skip("kernel does not cover this shape")
    say(f"canary score kernel={kernel} ({name}) {layout} bits={bits} C={C} D={D} P={P} B={B} S={S}")
    keys = keys_case(S + D, P, S, D, C, layout, bits)
    cb = _t(synth.timing_codebook(C, C, D))
    rng = np.random.default_rng(B + S)
    A = _t(rng.standard_normal((P, B, D)).astype(np.float32))
    T = _t(rng.standard_normal((P, B, D)).astype(np.float32))
    out = Guarded((P, B, S), torch.float32)
    run_guarded(lambda: tq.tq_score_with_kernel(A, T, keys, cb, kernel, out.view), [out],
                [A, T, cb] + _keys_inputs(keys), f"tq_score[{name}]")


# ---------------------------------------------------------------------------
# MSE-only and outlier-split scorers
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout,bits,C,D,P,B,S", [
    ("packed", 3, 8, 128, 1, 1, 131075),   # small batch, many keys
    ("packed", 3, 8, 128, 8, 4, 70001),
    ("packed", 2, 4, 128, 2, 40, 3001),
    ("packed", 3, 8, 128, 1, 161, 300),    # past the register form's batch
    ("packed", 2, 4, 64, 4, 33, 257),
    ("unpacked", 0, 4, 32, 2, 70, 333),
    ("unpacked", 0, 8, 256, 1, 9, 65),
    ("packed", 3, 8, 128, 1, 5, 0),
])
def test_score_mse_guarded(layout, bits, C, D, P, B, S):
    say(f"canary score_mse {layout} bits={bits} C={C} D={D} P={P} B={B} S={S}")
    keys = values_case(S + B, P, S, D, C, layout, bits)
    cb = _t(synth.timing_codebook(C + 1, C, D))
    A = _t(synth.queries(S, P, B, D))
    out = Guarded((P, B, S), torch.float32)
    run_guarded(lambda: tq.tq_score_mse(A, keys, cb, out.view), [out], [A, cb] + _values_inputs(keys),
                "tq_score_mse")


@pytest.mark.parametrize("Dh,Dl,P,B,S", [
    (32, 96, 1, 1, 1 << 20 | 3),   # 16x16 matrix-core form
    (32, 96, 8, 4, 131075),        # 16x16 matrix-core form
    (32, 96, 2, 40, 3001),         # 32x32 matrix-core form
    (32, 96, 1, 161, 300),
    (16, 48, 3, 5, 1001),          # other widths: the vector form
    (32, 96, 2, 3, 0),
])
def test_score_split_guarded(Dh, Dl, P, B, S):
    say(f"canary score_split D_hi={Dh} D_lo={Dl} P={P} B={B} S={S}")
    hi = values_case(S + 1, P, S, Dh, 8, "packed", 3)
    lo = values_case(S + 2, P, S, Dl, 4, "packed", 2)
    keys = tq.SplitKeys(hi, lo)
    cbh, cbl = _t(synth.timing_codebook(6, 8, Dh)), _t(synth.timing_codebook(7, 4, Dl))
    Ah, Al = _t(synth.queries(B, P, B, Dh)), _t(synth.queries(B + 1, P, B, Dl))
    out = Guarded((P, B, S), torch.float32)
    run_guarded(lambda: tq.tq_score_split(Ah, Al, keys, cbh, cbl, out.view), [out],
                [Ah, Al, cbh, cbl] + _values_inputs(hi) + _values_inputs(lo), "tq_score_split")


# ---------------------------------------------------------------------------
# attention over compressed values, and the fused decode step
# ---------------------------------------------------------------------------

ATTEND_SHAPES = [
    # layout, bits, C, D, P, H, B, S
    ("unpacked", 0, 4, 128, 1, 1, 1, 1),
    ("unpacked", 0, 4, 128, 1, 1, 33, 33),
    ("unpacked", 0, 8, 64, 3, 3, 7, 1000),
    ("packed", 2, 4, 128, 1, 1, 4, 70001),     # many chunks: the wide combine
    ("packed", 3, 8, 128, 4, 2, 70, 1500),
    ("packed", 2, 4, 128, 16, 8, 4, 8191),
    ("packed", 2, 4, 64, 2, 1, 5, 300),
]


@pytest.mark.parametrize("layout,bits,C,D,P,H,B,S", ATTEND_SHAPES)
def test_attend_guarded(layout, bits, C, D, P, H, B, S):
    say(f"canary attend {layout} bits={bits} C={C} D={D} P={P} H={H} B={B} S={S}")
    vals = values_case(S + D, P, S, D, C, layout, bits)
    cb = _t(synth.timing_codebook(C, C, D))
    Pi_v = _t(synth.head_matrices(D, H, D)[0])
    scores = _t(synth.timing_scores(S, P, B, S))
    out = Guarded((P, B, D), torch.float32)
    ws = Guarded((tq.tq_attend_workspace_bytes(P, B, S, D),), torch.uint8, written=False)
    run_guarded(lambda: tq.tq_attend(scores, vals, cb, Pi_v, 0.3, out.view, ws.view), [out, ws],
                [scores, cb, Pi_v] + _values_inputs(vals), "tq_attend")


@pytest.mark.parametrize("mode", ["fused", "two_pass", "auto"])
@pytest.mark.parametrize("layout,bits,C,D,P,H,B,S", [s for s in ATTEND_SHAPES if s[0] == "packed" and s[3] == 128])
def test_score_attend_guarded(mode, layout, bits, C, D, P, H, B, S):
    say(f"canary score_attend mode={mode} {layout} bits={bits} C={C} D={D} P={P} H={H} B={B} S={S}")
    keys = keys_case(S + 3, P, S, D, 8, "packed", 3)
    vals = values_case(S + D, P, S, D, C, layout, bits)
    cbk = _t(synth.timing_codebook(8, 8, D))
    cbv = _t(synth.timing_codebook(C, C, D))
    Pi_v = _t(synth.head_matrices(D, H, D)[0])
    rng = np.random.default_rng(B + S)
    A = _t(rng.standard_normal((P, B, D)).astype(np.float32))
    T = _t(rng.standard_normal((P, B, D)).astype(np.float32))
    out = Guarded((P, B, D), torch.float32)
    ws = Guarded((tq.tq_score_attend_workspace_bytes(P, B, S, D, mode),), torch.uint8, written=False)
    run_guarded(lambda: tq.tq_score_attend(A, T, keys, cbk, vals, cbv, Pi_v, 0.2, out.view, ws.view, mode=mode),
                [out, ws], [A, T, cbk, cbv, Pi_v] + _keys_inputs(keys) + _values_inputs(vals),
                f"tq_score_attend[{mode}]")


# ---------------------------------------------------------------------------
# key compression and the unpacking debug entry point, through the C ABI
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout,bits,D,P,H,S", [
    ("packed", 3, 128, 2, 2, 1001),
    ("packed", 2, 64, 3, 1, 129),
    ("unpacked", 0, 128, 1, 1, 257),
    ("unpacked", 0, 64, 4, 2, 33),
    ("packed", 3, 128, 1, 1, 0),
])
def test_compress_and_decode_guarded(layout, bits, D, P, H, S):
    say(f"canary compress/decode {layout} bits={bits} D={D} P={P} H={H} S={S}")
    C = 1 << (bits or 2)
    rng = np.random.default_rng(S + D)
    k = rng.standard_normal((P, S, D)).astype(np.float32)
    keys = _t(k / np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-30))
    Pi, S_mat = (_t(m) for m in synth.head_matrices(D, H, D))
    cb = _t(synth.timing_codebook(C, C, D))
    if layout == "packed":
        lay = tq.TQ_PACKED
        gidx = Guarded((P, S, D * bits // 8), torch.uint8)
        gsign = Guarded((P, S, D // 8), torch.uint8)
        ggam = Guarded((P, S), torch.float16)
    else:
        lay = tq.TQ_UNPACKED
        gidx = Guarded((P, S, D), torch.uint8)
        gsign = Guarded((P, S, D), torch.int8)
        ggam = Guarded((P, S), torch.float32)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def compress():
        out = tq._CKeysOut(lay, bits, gidx.view.data_ptr(), gsign.view.data_ptr(), ggam.view.data_ptr())
        tq._check(tq._lib.tq_compress_keys(ctypes.c_void_p(keys.data_ptr()), ctypes.c_void_p(Pi.data_ptr()),
                                           ctypes.c_void_p(S_mat.data_ptr()), ctypes.c_void_p(cb.data_ptr()),
                                           C, ctypes.byref(out), P, H, S, D, st), "tq_compress_keys")

    run_guarded(compress, [gidx, gsign, ggam], [keys, Pi, S_mat, cb], "tq_compress_keys")
    ck = tq.Keys(layout, gidx.view.clone(), gsign.view.clone(), ggam.view.clone(), bits)
    cks, _, _ = ck._c(D)
    didx, dsign, dgam = (Guarded((P, S, D), torch.uint8), Guarded((P, S, D), torch.int8),
                         Guarded((P, S), torch.float32))

    def decode():
        tq._check(tq._lib.tq_decode_debug(ctypes.byref(cks), ctypes.c_void_p(didx.view.data_ptr()),
                                          ctypes.c_void_p(dsign.view.data_ptr()),
                                          ctypes.c_void_p(dgam.view.data_ptr()), P, S, D, st), "tq_decode_debug")

    run_guarded(decode, [didx, dsign, dgam], _keys_inputs(ck), "tq_decode_debug")
