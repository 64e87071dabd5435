"""Raw attention scores from compressed keys (oracle; test infrastructure only).

Definition. A compressed key s (indices idx_s, signs sigma_s, residual norm
gamma_s) stands for the reconstructed key

    k_hat_s = Pi^T codebook[idx_s] + (sqrt(pi/2) / D) * gamma_s * S_mat^T sigma_s

("TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits", section 3, the
inner-product quantizer's dequantization with unit norm; "Fitting 4.4x More
Context on Jetson", Theorem 2, the same inner product). The raw score of query
q_b against key s is <q_b, k_hat_s>: no softmax, no 1/sqrt(D), no values
("TurboQuant Attention in CUDA: Transform the Query, Reuse the Work",
introduction). The QJL divisor is D because S_mat has D rows.

:func:`scores_by_reconstruction` computes exactly that, building every key.
:func:`scores_from_transformed` is the definition of the scoring kernel's output
in terms of the transformed queries A = Pi q and T = S_mat q (same page,
sections "Move the transforms to the query" and "Two kernels, two jobs"):

    scores[b, s] = sum_d A[b, d] codebook[idx[s, d]]
                   + (sqrt(pi/2) / D) * gamma_s * sum_d T[b, d] sigma[s, d]

The two agree up to rounding (the query-side identity); tests pin both.
All arithmetic is float64; inputs are widened from whatever the GPU is given.
"""

from __future__ import annotations

import math

import numpy as np

#: sqrt(pi / 2), the QJL de-biasing constant (divided by the number of rows D).
QJL_SQRT_HALF_PI = math.sqrt(math.pi / 2.0)


def reconstruct_keys(idx, sign, gamma, Pi, S_mat, codebook) -> np.ndarray:
    """k_hat [S, D] float64 for one problem."""
    idx = np.asarray(idx, np.intp)
    D = idx.shape[-1]
    c = np.asarray(codebook, np.float64)[idx]                       # centroid vectors c_s
    mse_part = c @ np.asarray(Pi, np.float64)                       # (Pi^T c_s)^T
    sig = np.asarray(sign, np.float64)
    qjl_part = sig @ np.asarray(S_mat, np.float64)                  # (S_mat^T sigma_s)^T
    g = np.asarray(gamma, np.float64)[:, None]
    return mse_part + (QJL_SQRT_HALF_PI / D) * g * qjl_part


def scores_by_reconstruction(q, idx, sign, gamma, Pi, S_mat, codebook,
                             key_chunk: int = 16384) -> np.ndarray:
    """scores [B, S] = q k_hat^T for one problem, building keys in chunks."""
    q64 = np.asarray(q, np.float64)
    S = np.asarray(idx).shape[0]
    out = np.empty((q64.shape[0], S), np.float64)
    for s0 in range(0, S, key_chunk):
        s1 = min(S, s0 + key_chunk)
        k_hat = reconstruct_keys(idx[s0:s1], sign[s0:s1], gamma[s0:s1], Pi, S_mat, codebook)
        out[:, s0:s1] = q64 @ k_hat.T
    return out


def scores_from_transformed(A, T, idx, sign, gamma, codebook,
                            key_chunk: int = 16384) -> np.ndarray:
    """scores [B, S] from A, T [B, D] for one problem."""
    A64 = np.asarray(A, np.float64)
    T64 = np.asarray(T, np.float64)
    D = A64.shape[-1]
    cb = np.asarray(codebook, np.float64)
    S = np.asarray(idx).shape[0]
    out = np.empty((A64.shape[0], S), np.float64)
    for s0 in range(0, S, key_chunk):
        s1 = min(S, s0 + key_chunk)
        c = cb[np.asarray(idx[s0:s1], np.intp)]                      # [s, D]
        mse = A64 @ c.T
        res = T64 @ np.asarray(sign[s0:s1], np.float64).T
        g = np.asarray(gamma[s0:s1], np.float64)[None, :]
        out[:, s0:s1] = mse + (QJL_SQRT_HALF_PI / D) * g * res
    return out
