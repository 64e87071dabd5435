"""Helpers shared by the GPU tests: device placement, oracle references and
the parity measure. Imported only by tests marked ``gpu``."""

from __future__ import annotations

import sys

import numpy as np
import torch

import compressed_attention_scoring_amd as tq
from oracle import pack as opk
from oracle import score as osc

#: parity bar for fp32 scores: max |gpu - exact| / (1 + |exact|)
SCORE_TOL = 1e-4


def say(msg: str) -> None:
    """Name the case on stdout before a GPU step, so a crash log shows it."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev() -> torch.device:
    return torch.device("cuda:0")


def t(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def keys_to_gpu(layout: str, bits: int, idx, sign, gamma) -> tq.Keys:
    return tq.Keys(layout, t(idx), t(sign), t(gamma), bits)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref))))


def random_codes(rng, P, S, D, C, layout, bits):
    """Random valid codes: unpacked copies for the oracle, layout streams for the GPU."""
    idx_u = rng.integers(0, C, size=(P, S, D)).astype(np.uint8)
    sign_u = np.where(rng.integers(0, 2, size=(P, S, D)) == 1, 1, -1).astype(np.int8)
    gamma = rng.uniform(0.05, 0.6, size=(P, S))
    if layout == "unpacked":
        return idx_u, sign_u, gamma.astype(np.float32), idx_u, sign_u
    return (idx_u, sign_u, opk.gamma_to_half(gamma),
            opk.pack_indices(idx_u, bits), opk.pack_signs(sign_u))


def oracle_scores_transformed(A, T, idx_u, sign_u, gamma_k, codebook):
    """Oracle [P,B,S] from the fp32 A, T the GPU was given."""
    P = A.shape[0]
    return np.stack([osc.scores_from_transformed(A[p], T[p], idx_u[p], sign_u[p],
                                                 gamma_k[p].astype(np.float64), codebook)
                     for p in range(P)])
