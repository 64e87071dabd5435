"""Query-side transform (oracle; test infrastructure only).

"TurboQuant Attention in CUDA: Transform the Query, Reuse the Work", section
"Move the transforms to the query": each query is transformed once into
A_b = Pi q_b and T_b = S_mat q_b, with row-major matrices, so
A[b, d] = sum_j Pi[d, j] q[b, j] (the comment over the first kernel in "Full
CUDA solution" states the same indexing). Problem p of a batch uses head
p mod H.
"""

from __future__ import annotations

import numpy as np


def transform_one(q: np.ndarray, Pi: np.ndarray, S_mat: np.ndarray):
    """q [B, D], Pi and S_mat [D, D] -> (A, T) [B, D] float64."""
    q64 = np.asarray(q, np.float64)
    A = q64 @ np.asarray(Pi, np.float64).T
    T = q64 @ np.asarray(S_mat, np.float64).T
    return A, T


def query_transform(q: np.ndarray, Pi: np.ndarray, S_mat: np.ndarray):
    """q [P, B, D], Pi and S_mat [H, D, D] -> (A, T) [P, B, D] float64."""
    q = np.asarray(q)
    Pi = np.asarray(Pi)
    S_mat = np.asarray(S_mat)
    if q.ndim == 2:
        q = q[None]
    if Pi.ndim == 2:
        Pi, S_mat = Pi[None], S_mat[None]
    P, H = q.shape[0], Pi.shape[0]
    A = np.empty(q.shape, np.float64)
    T = np.empty(q.shape, np.float64)
    for p in range(P):
        A[p], T[p] = transform_one(q[p], Pi[p % H], S_mat[p % H])
    return A, T
