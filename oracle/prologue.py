"""CPU oracle for the attention prologue of one decode step: RMSNorm of every sequence's hidden
state, the joint Q / K / V projection, and the rows that the KV-cache write appends.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[P3] "Sub-5ms MoE Inference: Sub-Byte KV Quantization and Expert Pipelining at Scale", section
"Engineering Real-Time Autonomous Workflows", item 1: RMSNorm, the self-attention projection
and the KV-cache write run as one kernel.

Readings taken here (the page names the three operations and gives no formulas):
  * RMSNorm of a hidden row h [d] with gain g [d]: x = h / sqrt(mean_i h_i^2 + eps) * g, the
    usual root-mean-square normalisation with a small eps;
  * the projection is one matrix W [(Hq + 2 H) * D, d] applied to x (no bias, and no rotary
    position embedding: the page names none), rows in the order Q heads 0 .. Hq - 1, K heads
    0 .. H - 1, V heads 0 .. H - 1, D rows each, so q[hq] = W[hq D : (hq + 1) D] x;
  * the KV-cache write appends the K and V rows of KV head h of sequence b at that sequence's
    token position, quantized exactly as an append of those rows (``oracle.cache``).
Everything is float64 on the bfloat16 inputs' exact values.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64


def rms_norm(h: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x [B, d] = h / sqrt(mean(h^2) + eps) * gain, per row, float64."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + float(eps)) * np.asarray(gain, dtype=np.float64)


def split_heads(y: np.ndarray, Hq: int, H: int, D: int):
    """y [B, (Hq + 2H) D] -> q [B, Hq, D], k [B, H, D], v [B, H, D] (the row order above)."""
    B = y.shape[0]
    q = y[:, :Hq * D].reshape(B, Hq, D)
    k = y[:, Hq * D:(Hq + H) * D].reshape(B, H, D)
    v = y[:, (Hq + H) * D:].reshape(B, H, D)
    return q, k, v


def prologue(h_bf16: np.ndarray, gain_bf16: np.ndarray, w_bf16: np.ndarray, eps: float,
             Hq: int, H: int, D: int):
    """The decode step's prologue from bfloat16 bit patterns: hidden states [B, d], gain [d],
    projection [(Hq + 2H) D, d].  Returns float64 (q [B, Hq, D], k [B, H, D], v [B, H, D])."""
    x = rms_norm(bf16_to_f64(h_bf16), bf16_to_f64(gain_bf16), eps)
    W = bf16_to_f64(w_bf16)
    assert W.shape == ((Hq + 2 * H) * D, x.shape[1])
    return split_heads(x @ W.T, Hq, H, D)
