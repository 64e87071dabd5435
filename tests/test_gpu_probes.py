"""The streaming probes (tq_probe_*) launch and move what they say: the write
probe stores its pattern in every 16-byte word, the read-then-write probe
stores values derived from what each workgroup read (all-zero input gives the
words (0, 1, 2, 3)), and the read probe leaves its sink alone for input that
cannot fold to the sink's trigger value."""

import ctypes

import pytest
import torch

import compressed_attention_scoring_amd as tq
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _st():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 8519680])
def test_write_probe_pattern(nbytes):
    say(f"probe write {nbytes} bytes")
    dst = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda:0")
    assert tq._lib.tq_probe_write(ctypes.c_void_p(dst.data_ptr()), ctypes.c_size_t(nbytes), _st()) == 0
    torch.cuda.synchronize()
    w = dst.view(-1, 4).cpu()
    base = 0x01020304
    assert bool((w[:, 0] == base).all()) and bool((w[:, 1] == base + 1).all()) and bool((w[:, 2] == base + 2).all())
    # word 3 carries the word's position inside its lane's group of four
    assert bool(((w[:, 3] - base) >= 0).all()) and bool(((w[:, 3] - base) < 4).all())


@pytest.mark.parametrize("rbytes,wbytes", [(16, 16), (8519680, 4194304), (6553600 + 16, 16777216)])
def test_read_write_probe(rbytes, wbytes):
    say(f"probe read_write {rbytes} -> {wbytes} bytes")
    src = torch.zeros(rbytes // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.full((wbytes // 4,), -7, dtype=torch.int32, device="cuda:0")
    rc = tq._lib.tq_probe_read_write(ctypes.c_void_p(src.data_ptr()), ctypes.c_size_t(rbytes),
                                     ctypes.c_void_p(dst.data_ptr()), ctypes.c_size_t(wbytes), _st())
    assert rc == 0
    torch.cuda.synchronize()
    w = dst.view(-1, 4).cpu()
    assert bool((w == torch.tensor([0, 1, 2, 3], dtype=torch.int32)).all())


@pytest.mark.parametrize("B,S,D", [(32, 32768, 128), (5, 1000, 128), (32, 70, 64), (1, 33, 256)])
def test_tile_probe(B, S, D):
    """tq_probe_tile reads every code byte of the unpacked keys and writes every
    score slot once, in the scorer's lane order: out[row, key] holds the xor of
    the 32-bit words of key's half rows (half (row / 4) % 2) and gamma's bits,
    plus the accumulator element v of that row."""
    import numpy as np

    say(f"probe tile B={B} S={S} D={D}")
    rng = np.random.default_rng(S + D)
    idx = rng.integers(0, 256, size=(S, D), dtype=np.uint8)
    sign = rng.integers(0, 256, size=(S, D), dtype=np.uint8)
    gam = rng.standard_normal(S).astype(np.float32)
    keys = tq.Keys("unpacked", torch.from_numpy(idx).cuda(), torch.from_numpy(sign.view(np.int8)).cuda(),
                   torch.from_numpy(gam).cuda())
    ck, _, _ = keys._c(D)
    out = torch.full((B, S), float("nan"), dtype=torch.float32, device="cuda:0")
    rc = tq._lib.tq_probe_tile(ctypes.byref(ck), ctypes.c_void_p(out.data_ptr()), B, S, D, _st())
    assert rc == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    half = D // 2
    words = lambda a, g: np.bitwise_xor.reduce(a[:, g * half:(g + 1) * half].copy().view(np.uint32), axis=1)
    x = [words(idx, g) ^ words(sign, g) ^ gam.view(np.uint32) for g in (0, 1)]
    rows = np.arange(B)
    g = (rows >> 2) & 1
    v = 4 * (rows >> 3) + (rows & 3)
    want = np.stack([(x[g[r]] + np.uint32(v[r])).astype(np.uint32) for r in rows])
    assert np.array_equal(got, want)


def test_read_probe_leaves_sink():
    say("probe read")
    src = torch.zeros(8519680 // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.full((1,), 5, dtype=torch.int32, device="cuda:0")
    rc = tq._lib.tq_probe_read(ctypes.c_void_p(src.data_ptr()), ctypes.c_size_t(8519680),
                               ctypes.c_void_p(sink.data_ptr()), _st())
    assert rc == 0
    torch.cuda.synchronize()
    assert int(sink.item()) == 5
