"""Lloyd-Max scalar codebooks (oracle; test infrastructure only).

"TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits", section 2 (mental
model) and section 3 (the quantizer in NumPy): after a uniformly random
rotation, one coordinate of a unit vector in R^d has density proportional to
(1 - x^2)^((d - 3) / 2) on [-1, 1], close to N(0, 1/d) for d >= 64. The codebook
is the Lloyd-Max quantizer of that one-dimensional law, found by the grid
iteration the page describes: nearest-centroid cells bounded by midpoints, then
each centroid moved to its cell's conditional mean, repeated a fixed number of
times from a start spread over +-2 standard deviations. The returned model MSE
is d times the per-coordinate squared error, i.e. E||u - Q(u)||^2 for unit u.

Two densities are offered. ``"sphere"`` is the exact coordinate law (used to
pin this solver against the page's printed table). ``"gaussian"`` is the
N(0, 1/d) law that the workloads' codebooks use.
"""

from __future__ import annotations

import functools

import numpy as np

GRID_POINTS = 400_001
ITERATIONS = 300


def _density(x: np.ndarray, d: int, density: str) -> np.ndarray:
    if density == "sphere":
        return np.clip(1.0 - x * x, 0.0, None) ** ((d - 3) / 2.0)
    if density == "gaussian":
        return np.exp(-0.5 * d * x * x)
    raise ValueError(f"unknown density {density!r}")


def _cells(edges: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Cell index of each grid point: cell i holds edges[i-1] < x <= edges[i]."""
    return np.searchsorted(edges, x, side="left")


def midpoints(centroids: np.ndarray) -> np.ndarray:
    """Nearest-centroid boundaries of a sorted codebook."""
    c = np.asarray(centroids, np.float64)
    return 0.5 * (c[1:] + c[:-1])


@functools.lru_cache(maxsize=None)
def lloyd_max(d: int, bits: int, density: str = "gaussian",
              grid: int = GRID_POINTS, iters: int = ITERATIONS):
    """Lloyd-Max codebook with 2**bits levels for dimension d.

    Returns (centroids, edges, model_mse) in float64. The arrays are marked
    read-only because results are cached.
    """
    x = np.linspace(-1.0, 1.0, grid)
    w = _density(x, d, density)
    w = w / w.sum()
    levels = 2 ** bits
    sd = 1.0 / np.sqrt(d)
    c = np.linspace(-2.0 * sd, 2.0 * sd, levels)
    for _ in range(iters):
        cell = _cells(midpoints(c), x)
        mass = np.bincount(cell, weights=w, minlength=levels)
        first_moment = np.bincount(cell, weights=w * x, minlength=levels)
        c = first_moment / mass
    edges = midpoints(c)
    err = x - c[_cells(edges, x)]
    model_mse = d * float(np.sum(w * err * err))
    c.setflags(write=False)
    edges.setflags(write=False)
    return c, edges, model_mse


def codebook_fp32(D: int, C: int, density: str = "gaussian") -> np.ndarray:
    """The C-entry codebook handed to the scorer: Lloyd-Max centroids as float32."""
    bits = int(C).bit_length() - 1
    if 2 ** bits != C:
        raise ValueError(f"C={C} is not a power of two")
    c, _, _ = lloyd_max(D, bits, density)
    return np.ascontiguousarray(c, dtype=np.float32)
