"""Workload shapes used by the tests and the benchmark (sizes only, no arithmetic).

Each workload is one rank's share of a ring-attention layer: a global sequence of
``S`` tokens split over a ring of ``P`` ranks, ``B`` batch entries, ``Hq`` query
heads sharing ``Hkv`` key/value heads, head dimension ``D``.  ``order`` is the
chunk-to-rank assignment ("contiguous" or "zigzag") and ``causal`` the mask.
``k_scale`` multiplies the drawn K values (a power of two, so exact).
``ulysses`` is the head-group count of the sequence/head relayout measured with
the workload, or 0.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    seed_id: int
    dtype: str
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int
    P: int
    order: str
    causal: bool
    k_scale: float = 1.0
    ulysses: int = 0

    @property
    def s_loc(self) -> int:
        return self.S // self.P

    @property
    def scale(self) -> float:
        return 1.0 / (self.D ** 0.5)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("f32_mha2_d64_s512_ring4_contiguous_causal", 1, "f32",
                 1, 2, 2, 64, 512, 4, "contiguous", True),
        Workload("bf16_gqa32x8_d128_s32k_ring8_zigzag_causal", 2, "bf16",
                 1, 32, 8, 128, 32768, 8, "zigzag", True),
        Workload("bf16_gqa32x8_d128_s128k_ring16_zigzag_causal", 3, "bf16",
                 1, 32, 8, 128, 131072, 16, "zigzag", True),
        Workload("bf16_mha16_b2_d128_s64k_ring8_contiguous_full", 4, "bf16",
                 2, 16, 16, 128, 65536, 8, "contiguous", False, 1.0, 8),
        Workload("bf16_gqa32x8_d128_s512k_ring32_zigzag_causal_khalf", 5, "bf16",
                 1, 32, 8, 128, 524288, 32, "zigzag", True, 0.5),
    ]
}

# The workload the headline throughput is quoted on (131,072-token zigzag ring of 16).
HEADLINE = "bf16_gqa32x8_d128_s128k_ring16_zigzag_causal"
# The small fp32 workload on which every rank is checked.
SMALL = "f32_mha2_d64_s512_ring4_contiguous_causal"


def workload(name: str) -> Workload:
    return WORKLOADS[name]
