"""CPU oracle for entropy-guided tiering of a paged cache: the attention mass of every page,
the pages that keep the FP8 tier, and the demotion of the other FP8 pages to the 2-bit tier.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[P2] "Hierarchical Token Gating and Tiered KV-Cache Paging: Architecting Sub-10ms MoE Engines",
section "2. Entropy-Guided Tiered KV-Cache Quantization": its "Dual-Tier Paged Compression
Protocol" box keeps the top 15% of high-attention tokens in FP8 and moves the rest to 2-bit;
its list ranks pages by cumulative attention weight (90th percentile and above stay FP8); its
"Operational Blueprint for AI Systems Engineers" item 2 refreshes the ranking asynchronously
every N decode steps.

Readings taken here (the pages give no formulas):
  * the attention weight of token t for query head hq is the decode step's softmax weight
    a[hq, t] = exp(s_t - max s) / sum exp(s - max s), s_t = sm_scale * q_hq . k_t over the S
    cached tokens with the dequantized keys, in float64;
  * the mass of page p (tokens 16p .. 16p + 15 below S) of a sequence is the mean over all Hq
    query heads of the summed weights of its tokens, so the masses of a sequence sum to 1;
  * the hot pages of a sequence are its ceil(keep_frac * n_pages) pages of largest mass (ties
    to the lower page number); keep_frac = 0.15 is the box's "top 15%";
  * an FP8 page that is not hot is demoted: every row of it (each KV head, K and V) is
    dequantized from FP8 in float32, x' = fl32(e4m3(code) * row scale), and quantized again by
    the 2-bit fit with outlier isolation, exactly as an append of x' would; its records enter
    the sorted outlier list at its tokens' place.  A 2-bit page never moves up (its original
    values are gone) and new pages enter FP8 (the caller picks the tier when it appends).
"""

from __future__ import annotations

import math
from typing import Dict

import numpy as np

from . import formats as F
from .cache import BLOCK, ListSlice, build_list
from .quantize import QuantSpec, dequantize_codes

F32 = np.float32


def attention_weights(q: np.ndarray, K: np.ndarray, sm_scale: float) -> np.ndarray:
    """Softmax weights [S] (float64) of query q [D] against keys K [S, D] (float64)."""
    s = (K @ q) * float(sm_scale)
    e = np.exp(s - np.max(s))
    return e / np.sum(e)


def page_mass(q: np.ndarray, K: Dict[int, np.ndarray], Hq: int, H: int, sm_scale: float,
              S: int) -> np.ndarray:
    """Attention mass of every page of one sequence: q [Hq, D] float64 queries, K[h] [S, D]
    float64 dequantized keys of KV head h.  Query head hq reads KV head floor(hq * H / Hq).
    Returns [ceil(S / 16)] float64."""
    npages = (S + BLOCK - 1) // BLOCK
    mass = np.zeros(npages)
    for hq in range(Hq):
        a = attention_weights(q[hq], K[(hq * H) // Hq][:S], sm_scale)
        per_page = np.zeros(npages * BLOCK)
        per_page[:S] = a
        mass += per_page.reshape(npages, BLOCK).sum(axis=1)
    return mass / Hq


def hot_pages(mass: np.ndarray, keep_frac: float) -> np.ndarray:
    """bool [n_pages]: the ceil(keep_frac * n) pages of largest mass, ties to the lower page."""
    n = len(mass)
    k = min(n, int(math.ceil(keep_frac * n)))
    order = sorted(range(n), key=lambda p: (-mass[p], p))
    hot = np.zeros(n, dtype=bool)
    hot[order[:k]] = True
    return hot


def pages_to_demote(tier1: np.ndarray, mass: np.ndarray, keep_frac: float) -> np.ndarray:
    """bool [n_pages]: FP8 pages (tier1) that are not hot."""
    return np.asarray(tier1, dtype=bool) & ~hot_pages(mass, keep_frac)


def fp8_rows_f32(lst: ListSlice, spec8: QuantSpec, D: int) -> np.ndarray:
    """x' = fl32(e4m3(code) * row scale) of every row stored in the FP8 tier ([S, D] float32;
    rows of other tiers are zero)."""
    S = lst.packed8.shape[0]
    codes = lst.packed8.astype(np.uint8)
    vals = F.e4m3_decode(codes).astype(F32)                      # exact
    scale = lst.meta8.copy().view(F32).reshape(S, 1)
    out = (vals * scale).astype(F32)                             # one float32 product per element
    return np.where(lst.tier1[:, None], out, F32(0.0)).astype(F32)


def demote(x: np.ndarray, tier1_pages: np.ndarray, demoted: np.ndarray, spec: QuantSpec,
           spec8: QuantSpec) -> ListSlice:
    """The list of one (sequence, KV head, K or V) after demoting the pages ``demoted``: rows of
    demoted pages are replaced by their FP8-dequantized values and quantized by the 2-bit fit;
    every other row keeps what it had (FP8 rows of hot pages, 2-bit rows of 2-bit pages).
    x [S, D] float32: the rows as originally appended."""
    tier1_pages = np.asarray(tier1_pages, dtype=bool)
    demoted = np.asarray(demoted, dtype=bool)
    assert not np.any(demoted & ~tier1_pages), "only FP8 pages are demoted"
    before = build_list(x, spec, tier1_pages, spec8)
    S, D = x.shape
    x8 = fp8_rows_f32(before, spec8, D)
    rows = np.repeat(demoted, BLOCK)[:S]
    x_new = np.where(rows[:, None], x8, x).astype(F32)
    return build_list(x_new, spec, tier1_pages & ~demoted, spec8)


def dequantized_fp8_check(lst: ListSlice, spec8: QuantSpec, D: int) -> np.ndarray:
    """float64 dequantization of the FP8 rows through the oracle's FP8 decoder (for pins)."""
    return dequantize_codes(lst.packed8.astype(np.uint8), lst.meta8, spec8)
