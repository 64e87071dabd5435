"""TurboQuant_prod compressor for unit keys (oracle; test infrastructure only).

"TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits", section 3: the
inner-product quantizer runs the MSE quantizer with one bit fewer, takes the
residual r = x - x_mse, and stores sign(S r) (one bit per projection row) and
||r||. The MSE quantizer rotates the (normalised) vector, y = Pi x, and assigns
each coordinate the index of its nearest centroid by a search over the
midpoints (a value exactly on a midpoint takes the lower index); it
dequantizes as Pi^T c[idx].

"TurboQuant Attention in CUDA: Transform the Query, Reuse the Work", section
"The keys arrived in pieces": gamma is the length of the residual left after
subtracting the centroid-based approximation, not the key's length.

:func:`quantize_prod` is the whole store-side step as the kanthi.in page's
section 3 orders it ("normalize, then rotate"): each key is divided by its
length first (a zero key stays the zero vector), the unit key is compressed by
:func:`quantize_prod_unit`, and the length is returned beside the codes. The
scores the path computes are against the unit key; the length is what a caller
multiplies back for scores against the key as given.

The sign of an exactly zero projection is taken as +1, so every stored sign is
+-1 (the page's ``np.sign`` would give 0 there; the case has probability zero).
Inputs Pi, S_mat and codebook are the float32 arrays handed to the GPU; the
arithmetic here is float64.
"""

from __future__ import annotations

import numpy as np

from .codebook import midpoints


def rotate(keys: np.ndarray, Pi: np.ndarray) -> np.ndarray:
    """y_s = Pi k_s for each row k_s of ``keys``."""
    return np.asarray(keys, np.float64) @ np.asarray(Pi, np.float64).T


def nearest_indices(y: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """Index of the nearest centroid of each coordinate, by midpoint search."""
    return np.searchsorted(midpoints(codebook), y, side="left").astype(np.uint8)


def dequantize_mse(idx: np.ndarray, Pi: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """x_mse_s = Pi^T codebook[idx_s] for each key s (rows)."""
    c = np.asarray(codebook, np.float64)[np.asarray(idx, np.intp)]
    return c @ np.asarray(Pi, np.float64)


def quantize_mse_unit(keys: np.ndarray, Pi: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """MSE-stage indices of unit keys."""
    return nearest_indices(rotate(keys, Pi), codebook)


def quantize_prod_unit(keys: np.ndarray, Pi: np.ndarray, S_mat: np.ndarray,
                       codebook: np.ndarray):
    """Compress unit keys [S, D] into (idx uint8 [S, D], sign int8 [S, D], gamma float64 [S])."""
    k = np.asarray(keys, np.float64)
    idx = quantize_mse_unit(k, Pi, codebook)
    r = k - dequantize_mse(idx, Pi, codebook)
    gamma = np.sqrt(np.sum(r * r, axis=1))
    proj = r @ np.asarray(S_mat, np.float64).T          # (S_mat r_s) for each key
    sign = np.where(proj >= 0.0, 1, -1).astype(np.int8)
    return idx, sign, gamma


def quantize_prod(keys: np.ndarray, Pi: np.ndarray, S_mat: np.ndarray, codebook: np.ndarray):
    """Normalise, then compress keys [S, D] of any length into (idx uint8 [S, D],
    sign int8 [S, D], gamma float64 [S], norm float64 [S]); a zero key is
    compressed as the zero vector and gets norm 0."""
    k = np.asarray(keys, np.float64)
    norm = np.sqrt(np.sum(k * k, axis=1))
    unit = k / np.where(norm > 0.0, norm, 1.0)[:, None]
    idx, sign, gamma = quantize_prod_unit(unit, Pi, S_mat, codebook)
    return idx, sign, gamma, norm
