"""Seeded end-to-end input sets for the named workloads (oracle; test infrastructure only).

Draws come from :mod:`synth` (the seed recipe lives there); everything that is
the method's own arithmetic -- the Lloyd-Max codebook, compression of the keys,
bit packing and fp16 rounding of gamma -- is done here by the oracle. The GPU
library receives the resulting arrays and never this code.

Reading taken for the workloads' codebook: the N(0, 1/D) coordinate law (the
sphere law's approximation), solved with the grid Lloyd-Max iteration of
:mod:`oracle.codebook`. The scorer itself is codebook-agnostic.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import synth

from .codebook import codebook_fp32
from .compress import quantize_prod_unit
from .pack import gamma_to_half, pack_indices, pack_signs


@dataclass
class InputSet:
    workload: "synth.Workload"
    q: np.ndarray            # float32 [P, B, D]
    Pi: np.ndarray           # float32 [H, D, D]
    S_mat: np.ndarray        # float32 [H, D, D]
    codebook: np.ndarray     # float32 [C]
    idx_u: np.ndarray        # uint8 [P, S, D]   indices, one byte each
    sign_u: np.ndarray       # int8  [P, S, D]   +-1
    gamma_k: np.ndarray      # gamma exactly as the kernel sees it: float32 or float16 [P, S]
    idx: np.ndarray          # the layout's index stream (== idx_u if unpacked)
    sign: np.ndarray         # the layout's sign stream (== sign_u if unpacked)

    @property
    def gamma_ref(self) -> np.ndarray:
        """gamma widened to float64 from the stored precision."""
        return self.gamma_k.astype(np.float64)


def compress_problem(keys, Pi, S_mat, codebook):
    return quantize_prod_unit(keys, Pi, S_mat, codebook)


def make_inputs(w: "synth.Workload", S: int | None = None, P: int | None = None) -> InputSet:
    """Build the full input set of workload ``w`` (optionally with fewer keys or problems)."""
    S = w.S if S is None else S
    P = w.P if P is None else P
    D, H = w.D, w.H
    Pi, S_mat = synth.head_matrices(w.seed, H, D)
    codebook = codebook_fp32(D, w.C)
    q = synth.queries(w.seed, P, w.B, D)
    idx_u = np.empty((P, S, D), np.uint8)
    sign_u = np.empty((P, S, D), np.int8)
    gamma = np.empty((P, S), np.float64)
    for p in range(P):
        keys = synth.unit_keys(synth.keys_rng(w.seed, p), S, D, w.keys)
        idx_u[p], sign_u[p], gamma[p] = compress_problem(keys, Pi[p % H], S_mat[p % H], codebook)
    if w.layout == "unpacked":
        gamma_k = gamma.astype(np.float32)
        idx, sign = idx_u, sign_u
    elif w.layout == "packed":
        gamma_k = gamma_to_half(gamma)
        idx = pack_indices(idx_u, w.bits)
        sign = pack_signs(sign_u)
    else:
        raise ValueError(w.layout)
    return InputSet(w, q, Pi, S_mat, codebook, idx_u, sign_u, gamma_k, idx, sign)
