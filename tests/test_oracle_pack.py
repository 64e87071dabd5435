"""Pins for the oracle's bit packing (CPU only): hand-derived bytes, an
independent big-integer decoder, and pack/unpack round trips."""

import numpy as np
import pytest

from oracle import pack as opk


def test_golden_bytes(golden):
    g = golden("packing.json")
    np.testing.assert_array_equal(opk.pack_indices(np.array(g["idx2"]["idx"]), 2), g["idx2"]["bytes"])
    np.testing.assert_array_equal(opk.pack_indices(np.array(g["idx3"]["idx"]), 3), g["idx3"]["bytes"])
    np.testing.assert_array_equal(opk.pack_signs(np.array(g["signs"]["sign"])), g["signs"]["bytes"])
    assert int(opk.gamma_to_half(np.float64(g["gamma_half"]["gamma"])).view(np.uint16)) == g["gamma_half"]["bits"]


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("D", [8, 32, 64, 96, 128, 256])
def test_roundtrip_and_bigint_decoder(bits, D):
    rng = np.random.default_rng(30 + D + bits)
    idx = rng.integers(0, 2 ** bits, size=(17, D)).astype(np.uint8)
    packed = opk.pack_indices(idx, bits)
    assert packed.shape == (17, D * bits // 8)
    np.testing.assert_array_equal(opk.unpack_indices(packed, bits, D), idx)
    for s in (0, 5, 16):
        v = int.from_bytes(bytes(packed[s]), "little")
        dec = [(v >> (bits * d)) & ((1 << bits) - 1) for d in range(D)]
        assert dec == list(idx[s])
    sign = np.where(rng.integers(0, 2, size=(17, D)) == 1, 1, -1).astype(np.int8)
    sp = opk.pack_signs(sign)
    assert sp.shape == (17, D // 8)
    np.testing.assert_array_equal(opk.unpack_signs(sp, D), sign)
    v = int.from_bytes(bytes(sp[3]), "little")
    assert [1 if (v >> d) & 1 else -1 for d in range(D)] == list(sign[3])


def test_three_bit_slot_is_48_bytes():
    assert opk.index_bytes_per_key(128, 3) == 48
    assert opk.index_bytes_per_key(128, 2) == 32
    with pytest.raises(ValueError):
        opk.index_bytes_per_key(4, 3)


def test_gamma_half_round_to_nearest_even():
    # 2049 is halfway between the fp16 neighbours 2048 and 2050: ties go to even (2048)
    assert float(opk.gamma_to_half(np.float64(2049.0))) == 2048.0
    assert float(opk.gamma_to_half(np.float64(2051.0))) == 2052.0


def test_rejects_out_of_range_index():
    with pytest.raises(ValueError):
        opk.pack_indices(np.array([4, 0, 0, 0, 0, 0, 0, 0]), 2)
