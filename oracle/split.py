"""The outlier split: two quantizer instances per head (oracle; test
infrastructure only).

"TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits", section 7 (fractional
bits and the outlier split): the 2.5- and 3.5-bit settings run two instances
per head over disjoint channel sets, the hot ("outlier") channels with one bit
more than the rest, e.g. 32 channels at 3 bits and 96 at 2 bits for 2.5 bits
per channel. Each instance has its own rotation over its own channels and its
own norm. Section 9 (exercises) picks the hot channels as those with the
largest mean |k|.

Each instance is the MSE quantizer of :mod:`oracle.mse` on its sub-vector. A
key is stored as (idx_hi, rho_hi) for its hot channels and (idx_lo, rho_lo) for
the rest, and stands for k_hat with
    k_hat[hot]  = rho_hi * Pi_hi^T c_hi[idx_hi],
    k_hat[rest] = rho_lo * Pi_lo^T c_lo[idx_lo].
Its score against q is the sum of the instances' MSE scores:
    <q, k_hat> = rho_hi <Pi_hi q[hot], c_hi[idx_hi]> + rho_lo <Pi_lo q[rest], c_lo[idx_lo]>.

The channel order is a permutation ``perm`` of 0..D-1: its first D_hi entries
are the hot channels, the rest the others.
"""

from __future__ import annotations

import numpy as np

from . import mse


def channel_permutation(D: int, hot) -> np.ndarray:
    """perm [D] int32: the hot channels in increasing order, then the others."""
    hot = np.unique(np.asarray(hot, np.int64))
    if hot.size and (hot[0] < 0 or hot[-1] >= D):
        raise ValueError("hot channels must lie in [0, D)")
    rest = np.setdiff1d(np.arange(D), hot)
    return np.concatenate([hot, rest]).astype(np.int32)


def choose_hot_channels(keys: np.ndarray, n: int) -> np.ndarray:
    """The n channels with the largest mean |k| over the given keys, increasing."""
    m = np.mean(np.abs(np.asarray(keys, np.float64)), axis=0)
    return np.sort(np.argsort(-m, kind="stable")[:n])


def bits_per_channel(d_hi: int, b_hi: int, d_lo: int, b_lo: int) -> float:
    """Index bits per channel of a split: (d_hi b_hi + d_lo b_lo) / (d_hi + d_lo)."""
    return (d_hi * b_hi + d_lo * b_lo) / (d_hi + d_lo)


def compress_split(keys, perm, d_hi, Pi_hi, Pi_lo, cb_hi, cb_lo, norm_correction=False):
    """Keys [S, D] -> (idx_hi [S, d_hi], rho_hi [S], idx_lo [S, D - d_hi], rho_lo [S])."""
    k = np.asarray(keys, np.float64)
    perm = np.asarray(perm, np.intp)
    idx_hi, rho_hi = mse.compress_mse(k[:, perm[:d_hi]], Pi_hi, cb_hi, norm_correction)
    idx_lo, rho_lo = mse.compress_mse(k[:, perm[d_hi:]], Pi_lo, cb_lo, norm_correction)
    return idx_hi, rho_hi, idx_lo, rho_lo


def dequantize_split(perm, d_hi, idx_hi, rho_hi, Pi_hi, cb_hi, idx_lo, rho_lo, Pi_lo, cb_lo) -> np.ndarray:
    """k_hat [S, D] with each instance's reconstruction in its own channels."""
    perm = np.asarray(perm, np.intp)
    hi = mse.dequantize_mse_keys(idx_hi, rho_hi, Pi_hi, cb_hi)
    lo = mse.dequantize_mse_keys(idx_lo, rho_lo, Pi_lo, cb_lo)
    out = np.empty((hi.shape[0], perm.size))
    out[:, perm[:d_hi]] = hi
    out[:, perm[d_hi:]] = lo
    return out


def scores_split_by_reconstruction(q, perm, d_hi, idx_hi, rho_hi, Pi_hi, cb_hi, idx_lo, rho_lo, Pi_lo,
                                   cb_lo) -> np.ndarray:
    """[B, S]: <q_b, k_hat_s>, every key rebuilt."""
    return np.asarray(q, np.float64) @ dequantize_split(perm, d_hi, idx_hi, rho_hi, Pi_hi, cb_hi,
                                                        idx_lo, rho_lo, Pi_lo, cb_lo).T


def query_transform_split(q, perm, d_hi, Pi_hi, Pi_lo):
    """(A_hi [B, d_hi], A_lo [B, D - d_hi]) = (Pi_hi q[hot], Pi_lo q[rest])."""
    q = np.asarray(q, np.float64)
    perm = np.asarray(perm, np.intp)
    return q[:, perm[:d_hi]] @ np.asarray(Pi_hi, np.float64).T, q[:, perm[d_hi:]] @ np.asarray(Pi_lo, np.float64).T


def scores_split_from_transformed(A_hi, idx_hi, rho_hi, cb_hi, A_lo, idx_lo, rho_lo, cb_lo) -> np.ndarray:
    """[B, S]: the two instances' MSE scores added (the scoring kernel's output)."""
    return (mse.scores_mse_from_transformed(A_hi, idx_hi, rho_hi, cb_hi)
            + mse.scores_mse_from_transformed(A_lo, idx_lo, rho_lo, cb_lo))
