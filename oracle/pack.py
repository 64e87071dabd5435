"""Bit-packed key storage (oracle; test infrastructure only).

Index streams are LSB-first dense bitstreams per key: coordinate d of a b-bit
index occupies bits [b*d, b*d + b) of the key's byte string read as one
little-endian integer. For b = 2 this is four indices per byte, coordinate
4j + t at bits 2t..2t+1 of byte j, the order the vectorised Triton kernel
extracts them in ("Fitting 4.4x More Context on Jetson", section "v6: Fused
Vectorized Hybrid"). For b = 3 a 128-coordinate key takes 48 bytes, the slot
size "TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits" gives in section 8;
eight indices fill three bytes and some straddle byte boundaries.

Sign streams hold one bit per coordinate, LSB-first, bit 1 meaning +1.
Residual norms are stored as IEEE binary16, rounded to nearest even once here
(the same section 8 and section 3 store the per-vector norm in fp16).
"""

from __future__ import annotations

import numpy as np


def index_bytes_per_key(D: int, bits: int) -> int:
    if (D * bits) % 8:
        raise ValueError(f"D={D} with {bits}-bit indices is not a whole number of bytes")
    return D * bits // 8


def pack_indices(idx: np.ndarray, bits: int) -> np.ndarray:
    """idx [..., D] (values < 2**bits) -> packed bytes [..., D*bits/8]."""
    idx = np.asarray(idx, np.uint8)
    D = idx.shape[-1]
    index_bytes_per_key(D, bits)
    if idx.size and int(idx.max()) >= (1 << bits):
        raise ValueError("index does not fit in the bit width")
    # stream[..., bits*d + j] = bit j of idx[..., d]
    planes = (idx[..., :, None] >> np.arange(bits, dtype=np.uint8)) & 1
    stream = planes.reshape(idx.shape[:-1] + (D * bits,))
    return np.packbits(stream, axis=-1, bitorder="little")


def unpack_indices(packed: np.ndarray, bits: int, D: int) -> np.ndarray:
    """Inverse of :func:`pack_indices`."""
    packed = np.asarray(packed, np.uint8)
    stream = np.unpackbits(packed, axis=-1, bitorder="little")[..., : D * bits]
    planes = stream.reshape(packed.shape[:-1] + (D, bits)).astype(np.uint8)
    weights = (1 << np.arange(bits)).astype(np.uint8)
    return np.sum(planes * weights, axis=-1, dtype=np.uint8)


def pack_signs(sign: np.ndarray) -> np.ndarray:
    """sign [..., D] in {-1, +1} -> bytes [..., D/8], bit 1 = +1, LSB-first."""
    sign = np.asarray(sign)
    if sign.shape[-1] % 8:
        raise ValueError("D must be a multiple of 8 to pack signs")
    return np.packbits(sign > 0, axis=-1, bitorder="little")


def unpack_signs(packed: np.ndarray, D: int) -> np.ndarray:
    bits = np.unpackbits(np.asarray(packed, np.uint8), axis=-1, bitorder="little")[..., :D]
    return np.where(bits == 1, 1, -1).astype(np.int8)


def gamma_to_half(gamma: np.ndarray) -> np.ndarray:
    """Residual norms rounded once to binary16 (round to nearest even)."""
    return np.asarray(gamma, np.float64).astype(np.float16)
