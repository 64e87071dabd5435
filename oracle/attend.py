"""Decode attention output over compressed values (oracle; test infrastructure only).

The step downstream of scoring. "TurboQuant: Rotate-then-Quantize KV Caches at
3 Bits", section 8 ("Kernel view: never un-rotate a key"): values are stored
by the MSE quantizer (rotation Pi_v, Lloyd-Max codebook, one norm per vector),
the attention weights are a softmax over the scaled scores, and the output is
the weighted sum of the dequantized values. Because Pi_v is orthogonal the sum
can be accumulated in the rotated basis and un-rotated once per query:

    o_b = sum_s p_bs ||v_s|| Pi_v^T c[idx_s] = Pi_v^T ( sum_s p_bs ||v_s|| c[idx_s] ),
    p_bs = exp(scale * score_bs - m_b) / sum_t exp(scale * score_bt - m_b),
    m_b = max_t scale * score_bt.

"Fitting 4.4x More Context on Jetson", section "What is online softmax": the
maximum and the normaliser can be carried through one pass over the keys; a
split over key ranges (each with its own maximum, normaliser and partial sum)
combines into the same result. :func:`combine_partials` is that combination.

:func:`compress_values` follows the MSE quantizer of the first page's section 3
(normalise, rotate, nearest centroid by midpoint search) with the norm stored
separately; :func:`attend_explicit` rebuilds every value vector and applies
the softmax directly; :func:`attend_rotated` is the rotated-domain form. All
arithmetic is float64.
"""

from __future__ import annotations

import numpy as np

from .compress import dequantize_mse, nearest_indices, rotate


def compress_values(values: np.ndarray, Pi_v: np.ndarray, codebook: np.ndarray):
    """Values [S, D] -> (idx uint8 [S, D], norm float64 [S]): v = norm * unit, unit quantized."""
    v = np.asarray(values, np.float64)
    norm = np.sqrt(np.sum(v * v, axis=1))
    unit = v / np.where(norm > 0.0, norm, 1.0)[:, None]
    idx = nearest_indices(rotate(unit, Pi_v), codebook)
    return idx, norm


def dequantize_values(idx, norm, Pi_v, codebook) -> np.ndarray:
    """v_hat [S, D] = norm_s * Pi_v^T c[idx_s]."""
    return np.asarray(norm, np.float64)[:, None] * dequantize_mse(idx, Pi_v, codebook)


def softmax_weights(scores: np.ndarray, scale: float) -> np.ndarray:
    """p [B, S] = softmax over s of scale * scores[b, s] (max subtracted first)."""
    z = float(scale) * np.asarray(scores, np.float64)
    z = z - np.max(z, axis=-1, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=-1, keepdims=True)


def attend_explicit(scores, idx, norm, Pi_v, codebook, scale) -> np.ndarray:
    """o [B, D] = softmax(scale * scores) @ v_hat, rebuilding every value."""
    return softmax_weights(scores, scale) @ dequantize_values(idx, norm, Pi_v, codebook)


def attend_rotated(scores, idx, norm, Pi_v, codebook, scale) -> np.ndarray:
    """The same output accumulated in the rotated basis: Pi_v^T (sum_s p_s norm_s c[idx_s])."""
    p = softmax_weights(scores, scale) * np.asarray(norm, np.float64)[None, :]
    acc = p @ np.asarray(codebook, np.float64)[np.asarray(idx, np.intp)]
    return acc @ np.asarray(Pi_v, np.float64)


def partial_state(scores, idx, norm, codebook, scale):
    """(m [B], l [B], acc [B, D]) of one key range, in the rotated basis:
    m = max scale*score, l = sum exp(scale*score - m), acc = sum exp(...) norm c[idx]."""
    z = float(scale) * np.asarray(scores, np.float64)
    m = np.max(z, axis=-1)
    e = np.exp(z - m[:, None])
    l = np.sum(e, axis=-1)
    acc = (e * np.asarray(norm, np.float64)[None, :]) @ np.asarray(codebook, np.float64)[np.asarray(idx, np.intp)]
    return m, l, acc


def combine_partials(parts, Pi_v) -> np.ndarray:
    """Merge per-range states (m, l, acc) into o = Pi_v^T (sum acc_r e^(m_r - M)) / (sum l_r e^(m_r - M))."""
    M = np.max(np.stack([m for m, _, _ in parts]), axis=0)
    num = sum(acc * np.exp(m - M)[:, None] for m, _, acc in parts)
    den = sum(l * np.exp(m - M) for m, l, _ in parts)
    return (num / den[:, None]) @ np.asarray(Pi_v, np.float64)
