"""CPU oracle for compressed-key attention scoring.  TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy implementation of what the scoring path computes,
plus the offline and store-side steps that produce its inputs (Lloyd-Max
codebook, TurboQuant_prod compressor, bit packing). It shares no code with the
HIP library and is never imported by it. Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may use it.

Modules
  codebook         Lloyd-Max codebook for one coordinate of a rotated unit vector
  compress         TurboQuant_prod quantizer for unit keys (MSE stage + QJL signs)
  pack             LSB-first index bitstreams, 1-bit sign streams, fp16 gamma
  query_transform  A = Pi q and T = S_mat q
  score            scores by explicit key reconstruction, and from (A, T)
  workload         seeded end-to-end input sets for the named workloads
  attend           decode output over compressed values: softmax and rotated-domain sum
  mse              MSE-only keys (stored norm, norm correction), randomized Hadamard rotation
  split            the outlier split: two MSE instances per head over disjoint channel sets

Every function is pinned by tests under ``tests/`` against values the pages
print, closed forms, library routines or brute force; see each module.
"""

from . import attend, codebook, compress, mse, pack, query_transform, score, split, workload  # noqa: F401
