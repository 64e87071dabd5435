"""Seeded synthetic inputs for compressed-key attention scoring.

This module only draws random numbers and describes workload shapes. It holds
none of the scoring method's arithmetic (no codebook design, no quantization,
no bit packing, no scoring), so both the CPU oracle and the GPU library's
tests and benchmark can use it without sharing any computation.

Draw recipe (every stream is an independent ``numpy.random.default_rng`` seeded
with a list, so a problem's data can be drawn without drawing the others):

* head ``h`` (one rotation and one QJL projection per head):
  ``default_rng([seed, 0, h])`` draws the rotation first, then the projection;
* keys of problem ``p``: ``default_rng([seed, 1, p])``;
* queries of all problems: ``default_rng([seed, 2])``;
* random code streams used only for timing: ``default_rng([seed, 3, p])``;
* random value streams and scores used only for timing: ``default_rng([seed, 5, p])``.

The rotation is a Haar-random orthogonal matrix (QR of a Gaussian matrix with
the signs of R's diagonal folded into Q), the QJL projection has iid N(0, 1)
entries, queries are iid N(0, 1). Keys are unit vectors: either uniform on the
sphere, or Gaussian with four outlier channels scaled 15x before normalising.
These are the input families of "TurboQuant Attention in CUDA: Transform the
Query, Reuse the Work" (the inputs described under "The keys arrived in
pieces") and of "TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits"
(section 3, the Haar rotation and Gaussian QJL matrix; section 5, the hot
channel set 3, 17, 64, 101).
"""

from __future__ import annotations

import numpy as np

from .configs import WORKLOADS, Workload, workload  # noqa: F401

#: Channels that carry outliers in the "outlier" key family.
OUTLIER_CHANNELS = (3, 17, 64, 101)
#: Scale applied to the outlier channels before normalising.
OUTLIER_SCALE = 15.0


def head_rng(seed: int, h: int) -> np.random.Generator:
    return np.random.default_rng([seed, 0, h])


def keys_rng(seed: int, p: int) -> np.random.Generator:
    return np.random.default_rng([seed, 1, p])


def queries_rng(seed: int) -> np.random.Generator:
    return np.random.default_rng([seed, 2])


def codes_rng(seed: int, p: int) -> np.random.Generator:
    return np.random.default_rng([seed, 3, p])


def haar_rotation(rng: np.random.Generator, D: int) -> np.ndarray:
    """Haar-random orthogonal D x D matrix, returned as float32 (row-major)."""
    g = rng.standard_normal((D, D))
    q, r = np.linalg.qr(g)
    q = q * np.where(np.diag(r) < 0, -1.0, 1.0)[None, :]
    return np.ascontiguousarray(q, dtype=np.float32)


def gaussian_projection(rng: np.random.Generator, D: int) -> np.ndarray:
    """QJL projection with iid N(0, 1) entries, D x D float32."""
    return np.ascontiguousarray(rng.standard_normal((D, D)), dtype=np.float32)


def head_matrices(seed: int, H: int, D: int):
    """(Pi[H, D, D], S_mat[H, D, D]) float32, one pair per head."""
    Pi = np.empty((H, D, D), np.float32)
    S = np.empty((H, D, D), np.float32)
    for h in range(H):
        rng = head_rng(seed, h)
        Pi[h] = haar_rotation(rng, D)
        S[h] = gaussian_projection(rng, D)
    return Pi, S


def unit_keys(rng: np.random.Generator, S: int, D: int, family: str) -> np.ndarray:
    """S unit keys of length D in float64.

    ``family`` is ``"uniform"`` (uniform on the unit sphere) or ``"outlier"``
    (Gaussian, channels 3, 17, 64, 101 that exist at this D scaled 15x, then
    normalised).
    """
    z = rng.standard_normal((S, D))
    if family == "outlier":
        ch = [c for c in OUTLIER_CHANNELS if c < D]
        z[:, ch] *= OUTLIER_SCALE
    elif family != "uniform":
        raise ValueError(f"unknown key family {family!r}")
    return z / np.linalg.norm(z, axis=1, keepdims=True)


def queries(seed: int, P: int, B: int, D: int) -> np.ndarray:
    """Queries q[P, B, D], iid N(0, 1), float32."""
    rng = queries_rng(seed)
    return np.ascontiguousarray(rng.standard_normal((P, B, D)), dtype=np.float32)


def timing_codebook(seed: int, C: int, D: int) -> np.ndarray:
    """A sorted random C-entry codebook with N(0, 1/D) entries, float32.

    Used only where the code values cannot change what is measured (the GPU
    kernels contain no value-dependent control flow or addressing).
    """
    rng = np.random.default_rng([seed, 4])
    return np.sort(rng.standard_normal(C) / np.sqrt(D)).astype(np.float32)


def timing_code_streams(seed: int, P: int, S: int, D: int, C: int,
                        layout: str, bits: int):
    """Random but valid compressed-key streams for timing.

    unpacked: idx uint8 [P, S, D] uniform in [0, C), sign int8 [P, S, D]
    uniform in {-1, +1}, gamma float32 [P, S].
    packed: idx bytes [P, S, D*bits/8] and sign bytes [P, S, D/8] uniform
    (every byte pattern is a valid code), gamma float16 [P, S].
    gamma is uniform in [0.2, 0.5], the range of residual norms at 2-3 bits.
    """
    if layout == "unpacked":
        idx = np.empty((P, S, D), np.uint8)
        sign = np.empty((P, S, D), np.int8)
        gamma = np.empty((P, S), np.float32)
    elif layout == "packed":
        idx = np.empty((P, S, D * bits // 8), np.uint8)
        sign = np.empty((P, S, D // 8), np.uint8)
        gamma = np.empty((P, S), np.float16)
    else:
        raise ValueError(f"unknown layout {layout!r}")
    for p in range(P):
        rng = codes_rng(seed, p)
        if layout == "unpacked":
            idx[p] = rng.integers(0, C, size=(S, D), dtype=np.uint8)
            sign[p] = np.where(rng.integers(0, 2, size=(S, D)) == 1, 1, -1)
        else:
            idx[p] = rng.integers(0, 256, size=idx.shape[1:], dtype=np.uint8)
            sign[p] = rng.integers(0, 256, size=sign.shape[1:], dtype=np.uint8)
        gamma[p] = rng.uniform(0.2, 0.5, size=S)
    return idx, sign, gamma


def timing_value_streams(seed: int, P: int, S: int, D: int, C: int, layout: str, bits: int):
    """Random but valid compressed-value streams for timing.

    unpacked: idx uint8 [P, S, D] uniform in [0, C), norm float32 [P, S];
    packed: idx bytes [P, S, D*bits/8] uniform, norm float16 [P, S].
    Norms are uniform in [0.5, 2] * sqrt(D), the length of a Gaussian vector.
    """
    if layout == "unpacked":
        idx = np.empty((P, S, D), np.uint8)
        norm = np.empty((P, S), np.float32)
    elif layout == "packed":
        idx = np.empty((P, S, D * bits // 8), np.uint8)
        norm = np.empty((P, S), np.float16)
    else:
        raise ValueError(f"unknown layout {layout!r}")
    for p in range(P):
        rng = np.random.default_rng([seed, 5, p])
        if layout == "unpacked":
            idx[p] = rng.integers(0, C, size=(S, D), dtype=np.uint8)
        else:
            idx[p] = rng.integers(0, 256, size=idx.shape[1:], dtype=np.uint8)
        norm[p] = rng.uniform(0.5, 2.0, size=S) * np.sqrt(D)
    return idx, norm


def timing_scores(seed: int, P: int, B: int, S: int) -> np.ndarray:
    """Scores [P, B, S] float32, N(0, 4^2): the spread of raw query-key scores
    of N(0, 1) queries against keys a few times the unit length."""
    rng = np.random.default_rng([seed, 6])
    return (rng.standard_normal((P, B, S), dtype=np.float32) * 4.0).astype(np.float32)
