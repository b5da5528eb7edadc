"""CPU oracle for decode attention over a dequantized cache, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages name the operation only as FlashAttention / flash-decoding fed by the dequantized
cache ([P1] figure in "The Bottleneck: Why Standard MoE Inference Stalls" and section
"Hardware-Kernel Fusion: Eliminating DRAM Round-Trips"; [P4] figure in "The Twin Bottlenecks"
with its "Attention Phase / Flash-Decoding Engine").  The plainest reading is standard scaled
dot-product attention of one new query token against the cached tokens:

    s_t = (q . k_t) * sm_scale,  p_t = exp(s_t - max_t s_t),  o = sum_t p_t v_t / sum_t p_t

with grouped-query attention (H KV heads shared by Hq query heads, [P1] "The Bottleneck",
"Grouped-Query Attention") mapping query head h to KV head floor(h * H / Hq), no mask (the
caller appends the current token first), and sm_scale = 1/sqrt(D) by default.

Flash-decoding splits the tokens into chunks whose partial results (m, l, o) are merged by
log-sum-exp; ``lse_merge`` is that merge written out, used only to pin the oracle.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64


def gqa_kv_head(hq: int, Hq: int, H: int) -> int:
    return (hq * H) // Hq


def attention_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """q [D], K [S, D], V [S, D] (float64) -> o [D] float64."""
    s = (K @ q) * float(sm_scale)
    m = np.max(s)
    p = np.exp(s - m)
    return (p @ V) / np.sum(p)


def decode_attention(q_bf16: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float,
                     heads=None) -> np.ndarray:
    """q_bf16 [Hq, D] bfloat16 bit patterns (uint16) of one sequence; K, V [H, S, D] float64
    dequantized cache of that sequence.  Returns o [Hq, D] float64 (rows not in ``heads`` are
    NaN when a subset is requested)."""
    Hq, D = q_bf16.shape
    H = K.shape[0]
    q = bf16_to_f64(q_bf16)
    out = np.full((Hq, D), np.nan)
    for hq in (range(Hq) if heads is None else heads):
        h = gqa_kv_head(hq, Hq, H)
        out[hq] = attention_one(q[hq], K[h], V[h], sm_scale)
    return out


def partial_state(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """Unnormalized flash-decoding state of one chunk: (m, l, o) with o = sum_t p_t v_t."""
    s = (K @ q) * float(sm_scale)
    m = np.max(s)
    p = np.exp(s - m)
    return m, np.sum(p), p @ V


def lse_merge(parts):
    """Merge chunk states: M = max m_c; o = sum_c e^{m_c - M} o_c / sum_c e^{m_c - M} l_c."""
    M = max(m for m, _, _ in parts)
    num = sum(np.exp(m - M) * o for m, _, o in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    return num / den
