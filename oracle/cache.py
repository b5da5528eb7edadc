"""CPU oracle for one logical cache list: the rows of one (sequence, KV head, K-or-V) slice in
token order, with its sorted COO outlier list.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The outlier side list follows [P1] "1. Dynamic Outlier Isolation" (extracted values kept at
higher precision, stored apart from the codes) and the fp16 "Outlier Tensor" box of [P3]
"Sub-Byte KV-Cache Quantization".  Its layout is this library's reading: one list per
(sequence, KV head, K or V) holding (index = token * D + channel, value) records in ascending
(token, channel) order, a record count, and the record count before every 16-token block
("block start"), so that any token range finds its records without a scan.

Tiering follows [P2] "Hierarchical Token Gating and Tiered KV-Cache Paging ...", section
"2. Entropy-Guided Tiered KV-Cache Quantization": a 16-token page is stored either as FP8
(tier 1, no outliers) or as 2-bit centroids with outliers (tier 2).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .quantize import QuantRows, QuantSpec, decode_outlier, dequantize_codes, quantize_rows

BLOCK = 16  # tokens per outlier block and per page


@dataclass
class ListSlice:
    codes: np.ndarray        # [S, D] uint8 logical codes
    packed: np.ndarray       # [S, code_bytes] for tier-2 rows; FP8 rows hold their own bytes
    meta: np.ndarray         # [S, meta_bytes] (tier-2 layout); FP8 rows: 4 bytes in meta8
    idx: np.ndarray          # [n] uint32 records, ascending
    vals: np.ndarray         # [n] uint16 (fp16 bits) or uint8 (E4M3 codes)
    block_start: np.ndarray  # [ceil(S/16)] int32
    count: int
    tier1: Optional[np.ndarray] = None    # [S] bool, rows stored in the FP8 tier
    packed8: Optional[np.ndarray] = None  # [S, D] uint8 FP8 codes (tier-1 rows valid)
    meta8: Optional[np.ndarray] = None    # [S, 4] uint8 fp32 row scale (tier-1 rows valid)


def build_list(x: np.ndarray, spec: QuantSpec, tier1_pages: Optional[np.ndarray] = None,
               spec8: Optional[QuantSpec] = None) -> ListSlice:
    """Quantize rows x [S, D] of one list in token order and collect its outlier records.
    ``tier1_pages`` (bool per 16-token page) selects rows quantized with ``spec8``."""
    S, D = x.shape
    q = quantize_rows(x, spec)
    tier1 = None
    packed8 = meta8 = None
    mask = q.mask.copy()
    if tier1_pages is not None:
        tier1 = np.repeat(np.asarray(tier1_pages, dtype=bool), BLOCK)[:S]
        q8 = quantize_rows(x, spec8)
        packed8, meta8 = q8.packed, q8.meta
        mask[tier1] = False  # FP8 rows keep no outliers
    t, c = np.nonzero(mask)  # row-major order = ascending (token, channel)
    idx = (t.astype(np.uint64) * D + c).astype(np.uint32)
    vals = q.outlier_bits[t, c]
    vals = vals.astype(np.uint8) if spec.outlier == "e4m3" else vals.astype(np.uint16)
    nblk = (S + BLOCK - 1) // BLOCK
    block_start = np.searchsorted(t, np.arange(nblk) * BLOCK, side="left").astype(np.int32)
    return ListSlice(q.codes, q.packed, q.meta, idx, vals, block_start, int(len(idx)), tier1,
                     packed8, meta8)


def dequantize_list(codes, meta, idx, vals, spec: QuantSpec, D: int, tier1=None, codes8=None,
                    meta8=None, spec8: Optional[QuantSpec] = None) -> np.ndarray:
    """Dequantized rows [S, D] in float64 (O8): codes through the group quantizer, outlier
    positions overwritten with the stored outlier value, FP8-tier rows through their scale."""
    out = dequantize_codes(codes, meta, spec)
    if tier1 is not None and np.any(tier1):
        out8 = dequantize_codes(codes8, meta8, spec8)
        out[tier1] = out8[tier1]
    if len(idx):
        t = np.asarray(idx, dtype=np.int64) // D
        c = np.asarray(idx, dtype=np.int64) % D
        out[t, c] = decode_outlier(vals, spec.outlier)
    return out


def records_before(idx: np.ndarray, D: int, token: int) -> int:
    """Number of records whose token is below ``token`` (list truncation point)."""
    return int(np.searchsorted(np.asarray(idx, dtype=np.int64) // D, token, side="left"))
