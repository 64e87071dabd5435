"""Workload shapes for compressed-key attention scoring.

Shapes follow the decode workloads the TurboQuant pages describe: the
performance shape of "TurboQuant Attention in CUDA: Transform the Query, Reuse
the Work" (32 queries, 32,768 cached keys, 128 coordinates; section "What the
rearrangement saves"), bit-packed 2- and 3-bit index streams with 1-bit QJL
signs and a 16-bit norm ("TurboQuant: Rotate-then-Quantize KV Caches at 3
Bits", section 8, packed slot sizes), and the 8-KV-head, head-dim-128 decode of
"Fitting 4.4x More Context on Jetson" (section "The Numbers"), batched as
independent per-head problems (its FAQ on grouped-query attention).
"""

from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    P: int          # independent scoring problems in one launch
    H: int          # distinct (rotation, projection) pairs; problem p uses head p % H
    B: int          # queries per problem
    S: int          # cached keys per problem
    D: int          # coordinates per key
    C: int          # codebook entries
    layout: str     # "unpacked" (byte per index and sign) or "packed" (bitstreams)
    bits: int       # index width in bits for "packed"; log2(C)
    keys: str       # "uniform" or "outlier" key family
    seed: int

    @property
    def pairs(self) -> int:
        """Number of (query, key) scores one pass computes."""
        return self.P * self.B * self.S

    def key_bytes(self) -> int:
        """Compressed key bytes one pass must read: indices, signs, gamma."""
        if self.layout == "unpacked":
            per_key = 2 * self.D + 4
        else:
            per_key = self.D * self.bits // 8 + self.D // 8 + 2
        return self.P * self.S * per_key

    def score_bytes(self) -> int:
        return self.P * self.B * self.S * 4

    def query_bytes(self) -> int:
        """Transformed queries A and T (fp32) and the fp32 codebook the score pass reads."""
        return 2 * self.P * self.B * self.D * 4 + self.C * 4

    def algorithmic_bytes(self) -> int:
        """Bytes the score pass must move once: compressed keys, A, T and the
        codebook in, fp32 scores out."""
        return self.key_bytes() + self.query_bytes() + self.score_bytes()

    def algorithmic_flops(self) -> int:
        """4D + 3 flops per (query, key) pair: two D-long dots and the combine."""
        return self.pairs * (4 * self.D + 3)

    def describe(self) -> dict:
        return {
            "workload": self.name, "P": self.P, "H": self.H, "B": self.B,
            "S": self.S, "D": self.D, "C": self.C, "layout": self.layout,
            "bits": self.bits, "keys": self.keys, "seed": self.seed,
        }


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny", P=1, H=1, B=2, S=256, D=32, C=4,
                 layout="unpacked", bits=2, keys="uniform", seed=0),
        Workload("decode", P=1, H=1, B=32, S=32768, D=128, C=4,
                 layout="unpacked", bits=2, keys="outlier", seed=1),
        Workload("packed", P=1, H=1, B=32, S=131072, D=128, C=4,
                 layout="packed", bits=2, keys="outlier", seed=2),
        Workload("gqa", P=128, H=8, B=4, S=32768, D=128, C=8,
                 layout="packed", bits=3, keys="outlier", seed=3),
        Workload("long", P=1, H=1, B=128, S=262144, D=128, C=8,
                 layout="packed", bits=3, keys="outlier", seed=4),
    )
}


def workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None
