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
subtracting the centroid-based approximation, not the key's length. The keys
here are unit vectors, so no key norm is stored.

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
