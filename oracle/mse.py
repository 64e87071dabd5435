"""MSE-only keys: stored norm, norm correction and the randomized Hadamard
rotation (oracle; test infrastructure only).

"TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits":
  * section 2 (the three facts): a dense Haar rotation costs O(d^2) per vector;
    production code rotates with y = H D x instead, D a random +-1 diagonal and
    H the orthonormal Walsh-Hadamard matrix, which is exactly orthogonal and
    costs O(d log d);
  * section 3 (the MSE quantizer and its notes): normalise, rotate, take the
    nearest centroid of each coordinate by a search over the midpoints, store
    the indices and the vector's norm; dequantize as ||x|| Pi^T c[idx]. With
    norm correction the codeword c[idx] is rescaled to unit length before it is
    un-rotated;
  * section 6 and the vLLM notes: attention in production uses this MSE-only
    variant (no QJL term), with norm correction.

The score of query q against a key stored this way is <q, k_hat> with
    k_hat = rho * Pi^T c[idx],   rho = ||k||   (or ||k|| / ||c[idx]|| corrected),
    <q, k_hat> = rho * sum_d (Pi q)[d] * c[idx_d],
so the query transform is A = Pi q (for the Hadamard rotation A = H (D q)) and
the scorer multiplies the MSE dot by one scalar per key. Norm correction only
changes that scalar, so :func:`compress_mse` folds it into the stored value.

All arithmetic is float64.
"""

from __future__ import annotations

import numpy as np

from .compress import nearest_indices


def fwht(x: np.ndarray) -> np.ndarray:
    """Orthonormal Walsh-Hadamard transform along the last axis (length 2^m), in
    Sylvester order: H_n = [[H, H], [H, -H]] / sqrt(2) with H = H_(n/2), so the
    top half of H_n x is H (x_lo + x_hi) / sqrt(2) and the bottom half is
    H (x_lo - x_hi) / sqrt(2)."""
    x = np.asarray(x, np.float64)
    n = x.shape[-1]
    if n & (n - 1):
        raise ValueError("the Walsh-Hadamard length must be a power of two")
    if n == 1:
        return x.copy()
    lo, hi = x[..., : n // 2], x[..., n // 2:]
    return np.concatenate([fwht(lo + hi), fwht(lo - hi)], axis=-1) / np.sqrt(2.0)


def hadamard_forward(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """y = H D x for each row x (D = diag(signs))."""
    return fwht(np.asarray(x, np.float64) * np.asarray(signs, np.float64))


def hadamard_inverse(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """x = D H y (H is symmetric and orthogonal, D its own inverse)."""
    return fwht(y) * np.asarray(signs, np.float64)


def hadamard_rotation(signs: np.ndarray) -> np.ndarray:
    """The dense matrix R = H D with R x = hadamard_forward(x, signs)."""
    s = np.asarray(signs, np.float64)
    return fwht(np.diag(s)).T


def compress_mse(keys: np.ndarray, Pi: np.ndarray, codebook: np.ndarray, norm_correction: bool = False):
    """Keys [S, D] -> (idx uint8 [S, D], rho float64 [S]).

    idx: nearest centroid of each coordinate of Pi (k / ||k||) (a zero key maps
    to the zero vector). rho: ||k||, or ||k|| / ||c[idx]|| with norm correction."""
    k = np.asarray(keys, np.float64)
    norm = np.sqrt(np.sum(k * k, axis=1))
    unit = k / np.where(norm > 0.0, norm, 1.0)[:, None]
    idx = nearest_indices(unit @ np.asarray(Pi, np.float64).T, codebook)
    if not norm_correction:
        return idx, norm
    c = np.asarray(codebook, np.float64)[idx.astype(np.intp)]
    cn = np.sqrt(np.sum(c * c, axis=1))
    return idx, norm / np.where(cn > 0.0, cn, 1.0)


def dequantize_mse_keys(idx, rho, Pi, codebook) -> np.ndarray:
    """k_hat [S, D] = rho_s * Pi^T c[idx_s]."""
    c = np.asarray(codebook, np.float64)[np.asarray(idx, np.intp)]
    return np.asarray(rho, np.float64)[:, None] * (c @ np.asarray(Pi, np.float64))


def scores_mse_by_reconstruction(q, idx, rho, Pi, codebook) -> np.ndarray:
    """[B, S]: <q_b, k_hat_s>, every key rebuilt."""
    return np.asarray(q, np.float64) @ dequantize_mse_keys(idx, rho, Pi, codebook).T


def scores_mse_from_transformed(A, idx, rho, codebook) -> np.ndarray:
    """[B, S]: rho_s * sum_d A[b, d] c[idx[s, d]] (the scoring kernel's output)."""
    c = np.asarray(codebook, np.float64)[np.asarray(idx, np.intp)]
    return (np.asarray(A, np.float64) @ c.T) * np.asarray(rho, np.float64)[None, :]


def query_transform_hadamard(q: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """A = H D q for each query row."""
    return hadamard_forward(q, signs)
