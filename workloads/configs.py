"""The five workloads, named by what they are.

Value distributions stand in for the pages' unnamed models and data: channel outliers in keys
([P1] "Paradigm 2", [P4] "Outlier Isolation and Block-wise Quantization"), a 256B-parameter
GQA MoE layer at batch 64 and 32k context ([P1] "The Bottleneck"), 128k contexts
([P1] introduction, [P4] "Attention Phase / Flash-Decoding Engine"), and two-tier paged caches
([P2] "2. Entropy-Guided Tiered KV-Cache Quantization").
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    H: int
    D: int
    S: int                       # context length (upper bound when S_range is set)
    fmt: str                     # "int4" | "fp4" | "c2" (tier 2) ; FP8 tier in paged configs
    group: int
    outlier: str                 # "fp16" | "e4m3"
    sigma: float
    seed: int
    dist: str                    # value distribution recipe, see generate.py
    S_range: Optional[Tuple[int, int]] = None   # per-sequence S ~ U[lo, hi]
    paged: bool = False
    page_size: int = 16
    fp8_page_frac: float = 0.0
    split_chunk: int = 0         # tokens per split-K chunk (0: library default)
    lloyd_iters: int = 8
    chan_mask: int = 0           # >0: static mask of this many channels per (KV head, K or V)
                                 # kept as outlier records in every row (see generate.py)


CONFIGS = {
    # single layer, B=1, 8 query / 2 KV heads, INT4 g32, 4 channels per head scaled x20
    "int4_b1_s1k": Workload("int4_b1_s1k", 1, 8, 2, 128, 1024, "int4", 32, "fp16", 3.0, 0,
                            "normal_x20_channels"),
    # B=16, 32/8 heads, S=8192, 2-bit centroids g64, N(0,1) plus 1% Laplace(0, 8) spikes
    "c2_b16_s8k": Workload("c2_b16_s8k", 16, 32, 8, 128, 8192, "c2", 64, "e4m3", 3.0, 1,
                           "normal_laplace_spikes"),
    # one layer of a 256B GQA MoE model: B=64, 64/8 heads, S=32768, 2-bit g64, LogNormal K
    "c2_b64_s32k": Workload("c2_b64_s32k", 64, 64, 8, 128, 32768, "c2", 64, "e4m3", 3.0, 2,
                            "lognormal_key_channels"),
    # entropy-tiered paged cache: B=32, 32/8 heads, S ~ U[4096, 65536], 10% FP8 pages
    "tiered_b32_paged": Workload("tiered_b32_paged", 32, 32, 8, 128, 65536, "c2", 64, "e4m3",
                                 3.0, 3, "normal", S_range=(4096, 65536), paged=True,
                                 fp8_page_frac=0.10),
    # long-context flash-decoding: B=4, 64/8 heads, S=131072, FP4 g32 + E4M3 scale
    "fp4_b4_s128k": Workload("fp4_b4_s128k", 4, 64, 8, 128, 131072, "fp4", 32, "fp16", 3.0, 4,
                             "normal"),
}

HEADLINE = "c2_b64_s32k"
