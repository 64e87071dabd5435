"""The C-ABI library on the CPU: it loads, exports every function include/tq.h
declares, and rejects bad arguments with the documented codes before anything
reaches a GPU (no compute call is made here)."""

import ctypes
import subprocess

import pytest

import compressed_attention_scoring_amd as tq

EXPECTED = {
    "tq_query_transform", "tq_score", "tq_score_with_kernel", "tq_score_kernel_name",
    "tq_decode_debug", "tq_compress_keys", "tq_status_string", "tq_attend", "tq_attend_workspace_bytes",
    "tq_query_transform_hadamard", "tq_score_mse", "tq_query_transform_split", "tq_score_split",
    "tq_score_attend", "tq_score_attend_workspace_bytes", "tq_score_attend_with_mode", "tq_attend_no_alloc",
    "tq_probe_read", "tq_probe_write", "tq_probe_read_write", "tq_probe_tile",
}
OK, ARG, UNSUP, ALIGN = 0, -1, -2, -3


def test_header_declares_expected_functions():
    assert set(tq.header_functions()) == EXPECTED


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(tq.library_path())
    for name in tq.header_functions():
        assert getattr(lib, name) is not None
    out = subprocess.run(["nm", "-D", "--defined-only", tq.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert EXPECTED <= exported


def test_status_strings():
    assert tq.tq_status_string(0) == "ok"
    for code in (ARG, UNSUP, ALIGN, -4):
        assert tq.tq_status_string(code) not in ("ok", "unknown status")
    assert tq.tq_status_string(-99) == "unknown status"


def test_kernel_names_host_only():
    n = tq.tq_score_kernel_name
    assert n("unpacked", 0, 4, 1, 32, 32768, 128) == "mfma32_unpacked_mt1"
    assert n("packed", 2, 4, 1, 32, 131072, 128) == "mfma32_packed2_mt1"
    assert n("packed", 3, 8, 128, 4, 32768, 128) == "mfma16i8_packed3"
    assert n("packed", 3, 8, 128, 4, 32768, 128, "mfma_lds") == "mfma32_packed3_mt1"
    assert n("unpacked", 0, 4, 1, 4, 1 << 20, 128) == "mfma16_unpacked"
    assert n("unpacked", 0, 4, 1, 4, 32768, 128) == "mfma32_unpacked_mt1"     # few keys: LDS staging
    assert n("unpacked", 0, 4, 1, 5, 1 << 20, 128) == "mfma32_unpacked_mt1"
    assert n("unpacked", 0, 4, 1, 8, 100, 128, "mfma16") == "mfma16_unpacked"
    assert n("unpacked", 0, 4, 1, 4, 100, 64) == "mfma32_unpacked_mt1"        # 16x16 tiles need D >= 128
    assert n("unpacked", 0, 4, 1, 4, 100, 64, "mfma16") is None
    assert n("packed", 3, 8, 1, 128, 262144, 128, "mfma_shared") == "mfma32shared_packed3"
    assert n("packed", 3, 8, 1, 128, 262144, 256, "mfma_shared") is None
    assert n("packed", 3, 8, 1, 128, 262144, 128) == "mfma32shared_packed3"
    assert n("packed", 3, 8, 1, 96, 262144, 128) == "mfma32reg_packed3"
    assert n("packed", 3, 8, 1, 128, 262144, 128, "mfma_lds") == "mfma32_packed3_mt4"
    assert n("packed", 3, 8, 1, 128, 262144, 128, "mfma_reg") == "mfma32reg_packed3"
    assert n("unpacked", 0, 4, 1, 32, 32768, 128, "mfma_reg") == "mfma32reg_unpacked"
    assert n("unpacked", 0, 4, 1, 128, 100, 256) == "mfma32_unpacked_mt2"     # D = 256: LDS staging only
    assert n("unpacked", 0, 4, 1, 128, 100, 256, "mfma_reg") is None
    assert n("unpacked", 0, 4, 1, 32, 1 << 24, 128) == "valu_unpacked"        # S past the MFMA offset range
    assert n("unpacked", 0, 4, 1, 32, 1 << 24, 128, "mfma") is None
    assert n("unpacked", 0, 4, 1, 1, 2, 2) == "valu_unpacked"
    assert n("unpacked", 0, 16, 1, 32, 100, 128) == "valu_unpacked"
    assert n("unpacked", 0, 4, 1, 32, 100, 128, "valu") == "valu_unpacked"
    assert n("unpacked", 0, 4, 1, 32, 100, 128, "mfma") == "mfma32_unpacked_mt1"
    assert n("unpacked", 0, 4, 1, 64, 100, 128, "mfma") == "mfma32reg_unpacked"
    assert n("unpacked", 0, 4, 1, 64, 100, 128, "mfma_lds") == "mfma32_unpacked_mt2"
    assert n("packed", 2, 4, 1, 32, 100, 48, "mfma") is None
    assert n("packed", 2, 8, 1, 32, 100, 128) is None      # C != 2^bits
    assert n("packed", 4, 16, 1, 32, 100, 128) is None     # 4-bit not supported
    # the single-pass f16 form follows the automatic choice (register shapes take the LDS kernel)
    assert n("unpacked", 0, 4, 1, 32, 32768, 128, "mfma_f16") == "mfma32_unpacked_mt1_f16"
    assert n("packed", 2, 4, 1, 32, 131072, 128, "mfma_f16") == "mfma32_packed2_mt1_f16"
    assert n("packed", 3, 8, 128, 4, 32768, 128, "mfma_f16") == "mfma16_packed3_f16"
    assert n("packed", 3, 8, 1, 128, 262144, 128, "mfma_f16") == "mfma32shared_packed3_f16"
    assert n("packed", 3, 8, 1, 64, 262144, 128, "mfma_f16") == "mfma32_packed3_mt2_f16"
    assert n("unpacked", 0, 4, 1, 2, 256, 32, "mfma_f16") == "mfma32_unpacked_mt1_f16"
    assert n("unpacked", 0, 16, 1, 32, 100, 128, "mfma_f16") is None      # C > 8


def _keys(layout=0, bits=0, idx=16, sign=16, gamma=16):
    return tq._CKeys(layout, bits, idx, sign, gamma)


def _score(keys, C=4, P=1, B=2, S=8, D=32, A=16, T=16, cb=16, out=16, kernel=0):
    return tq._lib.tq_score_with_kernel(A, T, ctypes.byref(keys), cb, C, out, P, B, S, D, kernel, None)


def test_score_rejects_bad_arguments_before_launch():
    # pointers are never dereferenced on these paths; 16 is a stand-in aligned address
    assert _score(_keys(idx=None)) == ARG
    assert _score(_keys(), A=None) == ARG
    assert tq._lib.tq_score_with_kernel(16, 16, None, 16, 4, 16, 1, 2, 8, 32, 0, None) == ARG
    assert _score(_keys(layout=5)) == ARG
    assert _score(_keys(), S=-1) == ARG
    assert _score(_keys(), D=0) == ARG
    assert _score(_keys(), kernel=8) == ARG
    assert _score(_keys(), kernel=-1) == ARG
    assert _score(_keys(), S=1 << 24, kernel=2) == UNSUP
    assert _score(_keys(layout=1, bits=4), C=16) == UNSUP
    assert _score(_keys(layout=1, bits=2), C=8) == UNSUP
    assert _score(_keys(layout=1, bits=3), C=8, D=12) == UNSUP
    assert _score(_keys(), C=300) == UNSUP
    assert _score(_keys(), D=2048) == UNSUP
    assert _score(_keys(), P=70000) == UNSUP
    assert _score(_keys(), B=300000) == UNSUP
    assert _score(_keys(layout=1, bits=2), C=4, D=48, kernel=2) == UNSUP   # MFMA needs D in {64,128,256}
    assert _score(_keys(idx=17)) == ALIGN
    assert _score(_keys(gamma=18)) == ALIGN


def test_empty_calls_are_no_ops():
    assert _score(_keys(idx=None, sign=None, gamma=None), S=0, A=None, T=None, cb=None, out=None) == OK
    assert _score(_keys(), B=0) == OK
    assert _score(_keys(), P=0) == OK
    assert tq._lib.tq_query_transform(None, None, None, None, None, 0, 1, 4, 8, None) == OK
    assert tq._lib.tq_decode_debug(ctypes.byref(_keys()), None, None, None, 1, 0, 8, None) == OK


def test_query_transform_rejects_bad_arguments():
    f = tq._lib.tq_query_transform
    assert f(16, 16, 16, 16, None, 1, 1, 2, 8, None) == ARG
    assert f(16, 16, 16, 16, 16, 3, 2, 2, 8, None) == ARG        # P % H != 0
    assert f(16, 16, 16, 16, 16, 1, 0, 2, 8, None) == ARG
    assert f(16, 16, 16, 16, 16, 1, 1, 2, 0, None) == ARG
    assert f(16, 16, 16, 16, 16, 1, 1, 2, 2000, None) == UNSUP
    assert f(20, 16, 16, 16, 16, 1, 1, 2, 8, None) == ALIGN


def test_decode_rejects_bad_arguments():
    f = tq._lib.tq_decode_debug
    assert f(ctypes.byref(_keys()), None, 16, 16, 1, 4, 8, None) == ARG
    assert f(ctypes.byref(_keys(layout=1, bits=5)), 16, 16, 16, 1, 4, 8, None) == UNSUP
    assert f(ctypes.byref(_keys(sign=33)), 16, 16, 16, 1, 4, 8, None) == ALIGN


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(2, 8)
    Pi = torch.eye(8)
    with pytest.raises(ValueError, match="GPU"):
        tq.tq_query_transform(q, Pi, Pi)


def test_compress_rejects_bad_arguments():
    f = tq._lib.tq_compress_keys
    out = lambda layout=0, bits=0, idx=16, sign=16, gamma=16: ctypes.byref(tq._CKeysOut(layout, bits, idx, sign, gamma))
    assert f(16, 16, 16, 16, 4, None, 1, 1, 8, 128, None) == ARG
    assert f(16, 16, 16, 16, 4, out(layout=7), 1, 1, 8, 128, None) == ARG
    assert f(16, 16, 16, 16, 4, out(), 3, 2, 8, 128, None) == ARG           # P % H != 0
    assert f(16, 16, 16, 16, 4, out(), 1, 0, 8, 128, None) == ARG
    assert f(None, 16, 16, 16, 4, out(), 1, 1, 8, 128, None) == ARG
    assert f(16, 16, 16, 16, 4, out(idx=None), 1, 1, 8, 128, None) == ARG
    assert f(16, 16, 16, 16, 4, out(), 1, 1, 8, 96, None) == UNSUP          # D not in {64, 128}
    assert f(16, 16, 16, 16, 32, out(), 1, 1, 8, 128, None) == UNSUP        # C > 16
    assert f(16, 16, 16, 16, 4, out(layout=1, bits=3), 1, 1, 8, 128, None) == UNSUP   # C != 2^bits
    assert f(20, 16, 16, 16, 4, out(), 1, 1, 8, 128, None) == ALIGN
    assert f(16, 16, 16, 16, 4, out(gamma=24), 1, 1, 8, 128, None) == ALIGN
    assert f(None, None, None, None, 4, out(idx=None, sign=None, gamma=None), 1, 1, 0, 128, None) == OK
    assert f(None, None, None, None, 4, out(idx=None, sign=None, gamma=None), 0, 1, 8, 128, None) == OK


def test_attend_workspace_size():
    assert tq.tq_attend_workspace_bytes(0, 4, 100, 128) == 0
    assert tq.tq_attend_workspace_bytes(1, 4, 0, 128) == 0
    assert tq.tq_attend_workspace_bytes(1, 4, 100, -1) == 0
    for P, B, S, D in [(1, 32, 32768, 128), (128, 4, 32768, 128), (1, 1, 1, 64), (3, 70, 1000, 64)]:
        n = tq.tq_attend_workspace_bytes(P, B, S, D)
        chunks = n // (P * B * (D + 2) * 4)
        assert n == P * B * chunks * (D + 2) * 4
        assert 1 <= chunks <= (S + 31) // 32     # each chunk holds at least one 32-key tile


def test_attend_rejects_bad_arguments():
    f = tq._lib.tq_attend
    ws = 1 << 30
    vals = lambda layout=0, bits=0, idx=16, norm=16: ctypes.byref(tq._CValues(layout, bits, idx, norm))
    assert f(16, None, 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == ARG
    assert f(16, vals(layout=5), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == ARG
    assert f(16, vals(), 16, 4, 16, 1.0, 16, 16, ws, 3, 2, 4, 8, 128, None) == ARG     # P % H != 0
    assert f(16, vals(), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 0, 128, None) == ARG     # no keys
    assert f(None, vals(), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == ARG
    assert f(16, vals(norm=None), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == ARG
    assert f(16, vals(), 16, 4, 16, 1.0, 16, 16, 8, 1, 1, 4, 8, 128, None) == ARG       # workspace too small
    assert f(16, vals(), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 96, None) == UNSUP     # D
    assert f(16, vals(), 16, 16, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == UNSUP   # C > 8
    assert f(16, vals(layout=1, bits=3), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == UNSUP
    assert f(16, vals(layout=1, bits=4), 16, 16, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == UNSUP
    assert f(20, vals(), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == ALIGN
    assert f(16, vals(idx=24), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == ALIGN
    assert f(None, vals(idx=None, norm=None), None, 4, None, 1.0, None, None, 0, 1, 1, 0, 8, 128, None) == OK
    assert f(None, vals(idx=None, norm=None), None, 4, None, 1.0, None, None, 0, 0, 1, 4, 8, 128, None) == OK


def test_hadamard_transform_rejects_bad_arguments():
    f = tq._lib.tq_query_transform_hadamard
    assert f(None, 16, 16, 1, 1, 2, 128, None) == ARG
    assert f(16, 16, 16, 3, 2, 2, 128, None) == ARG        # P % H != 0
    assert f(16, 16, 16, 1, 0, 2, 128, None) == ARG
    assert f(16, 16, 16, 1, 1, 2, 96, None) == UNSUP       # not a power of two
    assert f(16, 16, 16, 1, 1, 2, 2048, None) == UNSUP
    assert f(20, 16, 16, 1, 1, 2, 128, None) == ALIGN
    assert f(None, None, None, 0, 1, 2, 128, None) == OK
    assert f(None, None, None, 1, 1, 0, 128, None) == OK


def test_score_mse_rejects_bad_arguments():
    f = tq._lib.tq_score_mse
    keys = lambda layout=0, bits=0, idx=16, norm=16: ctypes.byref(tq._CValues(layout, bits, idx, norm))
    assert f(16, None, 16, 4, 16, 1, 4, 8, 128, None) == ARG
    assert f(16, keys(layout=3), 16, 4, 16, 1, 4, 8, 128, None) == ARG
    assert f(None, keys(), 16, 4, 16, 1, 4, 8, 128, None) == ARG
    assert f(16, keys(norm=None), 16, 4, 16, 1, 4, 8, 128, None) == ARG
    assert f(16, keys(), 16, 4, 16, 1, 4, -1, 128, None) == ARG
    assert f(16, keys(), 16, 16, 16, 1, 4, 8, 128, None) == UNSUP          # C > 8
    assert f(16, keys(), 16, 4, 16, 1, 4, 8, 96, None) == UNSUP            # D
    assert f(16, keys(layout=1, bits=3), 16, 4, 16, 1, 4, 8, 128, None) == UNSUP
    assert f(16, keys(), 16, 4, 16, 1, 4, 1 << 24, 128, None) == UNSUP
    assert f(16, keys(idx=20), 16, 4, 16, 1, 4, 8, 128, None) == ALIGN
    assert f(None, keys(idx=None, norm=None), None, 4, None, 1, 4, 0, 128, None) == OK


def test_split_rejects_bad_arguments():
    qf = tq._lib.tq_query_transform_split
    assert qf(16, 16, 16, 16, 16, 16, 1, 1, 2, 128, 0, None) == ARG          # D_hi = 0
    assert qf(16, 16, 16, 16, 16, 16, 1, 1, 2, 128, 128, None) == ARG        # D_hi = D
    assert qf(16, 16, 16, 16, 16, 16, 3, 2, 2, 128, 32, None) == ARG         # P % H
    assert qf(16, None, 16, 16, 16, 16, 1, 1, 2, 128, 32, None) == ARG
    assert qf(16, 16, 16, 16, 16, 16, 1, 1, 2, 2048, 32, None) == UNSUP
    assert qf(16, 20, 16, 16, 16, 16, 1, 1, 2, 128, 32, None) == ALIGN
    assert qf(None, None, None, None, None, None, 1, 1, 0, 128, 32, None) == OK
    sf = tq._lib.tq_score_split
    inst = lambda layout=1, bits=3, idx=16, norm=16: tq._CValues(layout, bits, idx, norm)
    keys = lambda hi=None, lo=None: ctypes.byref(tq._CSplit(hi or inst(), lo or inst(bits=2)))
    assert sf(16, 16, None, 16, 8, 16, 4, 16, 1, 4, 8, 32, 96, None) == ARG
    assert sf(16, 16, keys(), 16, 8, 16, 4, 16, 1, 4, 8, 0, 96, None) == ARG
    assert sf(16, 16, keys(hi=inst(layout=7)), 16, 8, 16, 4, 16, 1, 4, 8, 32, 96, None) == ARG
    assert sf(16, 16, keys(), 16, 4, 16, 4, 16, 1, 4, 8, 32, 96, None) == UNSUP     # C_hi != 2^3
    assert sf(16, 16, keys(), 16, 8, 16, 4, 16, 1, 4, 8, 36, 92, None) == UNSUP     # not multiples of 8
    assert sf(16, 16, keys(hi=inst(layout=0, bits=0)), 16, 300, 16, 4, 16, 1, 4, 8, 32, 96, None) == UNSUP
    assert sf(None, 16, keys(), 16, 8, 16, 4, 16, 1, 4, 8, 32, 96, None) == ARG
    assert sf(16, 16, keys(lo=inst(bits=2, norm=None)), 16, 8, 16, 4, 16, 1, 4, 8, 32, 96, None) == ARG
    assert sf(16, 24, keys(), 16, 8, 16, 4, 16, 1, 4, 8, 32, 96, None) == ALIGN
    assert sf(None, None, keys(), None, 8, None, 4, None, 1, 4, 0, 32, 96, None) == OK


def test_score_attend_rejects_bad_arguments():
    f = tq._lib.tq_score_attend
    ws = 1 << 30
    vals = lambda layout=0, bits=0, idx=16, norm=16: ctypes.byref(tq._CValues(layout, bits, idx, norm))
    k = ctypes.byref(_keys())
    a = (16, 16)
    assert f(*a, k, 16, 4, None, 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == ARG
    assert f(*a, k, 16, 4, vals(), 16, 4, 16, 1.0, 16, 16, ws, 3, 2, 4, 8, 128, None) == ARG     # P % H
    assert f(*a, k, 16, 4, vals(), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 0, 128, None) == ARG     # no keys
    assert f(*a, k, 16, 4, vals(), 16, 4, 16, 1.0, 16, 16, 8, 1, 1, 4, 8, 128, None) == ARG      # workspace
    assert f(*a, k, 16, 4, vals(), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 64, None) == UNSUP    # D != 128
    assert f(*a, k, 16, 4, vals(), 16, 16, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == UNSUP  # C_v > 8
    assert f(*a, k, 16, 16, vals(), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == UNSUP  # C > 8
    assert f(*a, k, 16, 4, vals(layout=1, bits=3), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == UNSUP
    assert f(*a, k, 16, 4, vals(), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 1 << 24, 128, None) == UNSUP
    assert f(20, 16, k, 16, 4, vals(), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, None) == ALIGN
    assert f(None, None, k, None, 4, vals(), None, 4, None, 1.0, None, None, 0, 1, 1, 0, 8, 128, None) == OK
    for mode in ("auto", "fused", "two_pass"):
        assert tq.tq_score_attend_workspace_bytes(1, 32, 32768, 128, mode) > 0
    # two passes hold the scores; the fused form only the chunk records
    assert tq.tq_score_attend_workspace_bytes(1, 128, 262144, 128, "two_pass") > 128 * 262144 * 4
    assert tq.tq_score_attend_workspace_bytes(1, 128, 262144, 128, "fused") < 128 * 262144 * 4 / 16
    assert tq._lib.tq_score_attend_workspace_bytes(1, 32, 100, 128, 7) == 0
    g = tq._lib.tq_score_attend_with_mode
    assert g(*a, k, 16, 4, vals(), 16, 4, 16, 1.0, 16, 16, ws, 1, 1, 4, 8, 128, 3, None) == ARG    # unknown form


def test_probe_argument_checks_host_only():
    """The streaming probes validate on the host: no device call for these."""
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib = tq._lib
    a16, a8 = vp(4096), vp(4104)
    assert lib.tq_probe_read(None, sz(0), None, None) == OK
    assert lib.tq_probe_read(None, sz(16), a16, None) == ARG
    assert lib.tq_probe_read(a16, sz(24), a16, None) == ARG           # not a multiple of 16
    assert lib.tq_probe_read(a8, sz(16), a16, None) == ALIGN
    assert lib.tq_probe_read(a16, sz(16), None, None) == ARG          # no sink
    assert lib.tq_probe_read(a16, sz(1 << 37), a16, None) == ARG      # over 2^36
    assert lib.tq_probe_write(None, sz(0), None) == OK
    assert lib.tq_probe_write(a8, sz(32), None) == ALIGN
    assert lib.tq_probe_read_write(a16, sz(0), a16, sz(16), None) == ARG
    assert lib.tq_probe_read_write(a16, sz(16), a8, sz(16), None) == ALIGN
    t = lib.tq_probe_tile
    assert t(None, a16, 32, 64, 128, None) == ARG
    assert t(ctypes.byref(_keys()), a16, 0, 64, 128, None) == OK            # empty
    assert t(ctypes.byref(_keys()), a16, 32, 0, 128, None) == OK
    assert t(ctypes.byref(_keys()), None, 32, 64, 128, None) == ARG
    assert t(ctypes.byref(_keys()), a16, -1, 64, 128, None) == ARG
    assert t(ctypes.byref(_keys(layout=1, bits=2)), a16, 32, 64, 128, None) == UNSUP
    assert t(ctypes.byref(_keys()), a16, 33, 64, 128, None) == UNSUP        # one 32-query tile
    assert t(ctypes.byref(_keys()), a16, 32, 64, 96, None) == UNSUP
    assert t(ctypes.byref(_keys()), a16, 32, 1 << 24, 128, None) == UNSUP
    assert t(ctypes.byref(_keys(idx=17)), a16, 32, 64, 128, None) == ALIGN
    assert t(ctypes.byref(_keys()), a8, 32, 64, 128, None) == ALIGN
