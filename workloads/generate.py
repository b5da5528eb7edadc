"""Seeded generators.  Every slice regenerates independently of the others:

    rows of (sequence b, KV head h, kind) for tokens [2048*c, 2048*(c+1))
        <- numpy Generator(PCG64(SeedSequence([seed, b, h, kind, c])))

kind: 0 = keys, 1 = values, 2 = queries, 3/4 = keys/values appended at decode step ``c``,
5 = hidden states (decode step ``c``), 6 = RMSNorm gain, 7 = projection rows [1024 c, 1024 (c+1)).
Per-head constants (the x20 channels, the LogNormal channel scales) come from
SeedSequence([seed, 9999, h, kind]); sequence lengths, page tiers and block tables from
SeedSequence([seed, 7777, ...]).

Distributions ("dist" of a workload):
  normal                  N(0, 1)
  normal_x20_channels     N(0, 1); 4 channels per (KV head, K or V), drawn without
                          replacement, multiplied by 20
  normal_laplace_spikes   N(0, 1) + Bernoulli(0.01) * Laplace(loc 0, scale 8)
  lognormal_key_channels  keys: sigma_c * N(0, 1) with sigma_c ~ LogNormal(0, 0.5) per
                          (KV head, channel); values: N(0, 1)
Queries are N(0, 1) rounded to bfloat16 (round to nearest even).

Attention-prologue inputs (bfloat16, round to nearest even), for a model width d (Hq * D unless
given): hidden states N(0, 1) [B, d]; RMSNorm gain 1 + 0.1 N(0, 1) [d]; projection
N(0, 1 / d) [(Hq + 2 H) D, d], so the projected rows have unit variance.
"""

from __future__ import annotations

import numpy as np

from .configs import Workload

GEN_CHUNK = 2048
K, V, Q, NEW_K, NEW_V = 0, 1, 2, 3, 4
HIDDEN, GAIN, WEIGHT = 5, 6, 7
W_CHUNK = 1024


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _head_constants(w: Workload, h: int, kind: int):
    r = _rng(w.seed, 9999, h, kind)
    if w.dist == "normal_x20_channels":
        ch = r.choice(w.D, size=4, replace=False)
        scale = np.ones(w.D, dtype=np.float32)
        scale[ch] = 20.0
        return scale
    if w.dist == "lognormal_key_channels" and kind in (K, NEW_K):
        return r.lognormal(0.0, 0.5, size=w.D).astype(np.float32)
    return None


def _chunk(w: Workload, b: int, h: int, kind: int, c: int, n: int) -> np.ndarray:
    r = _rng(w.seed, b, h, kind, c)
    x = r.standard_normal((n, w.D), dtype=np.float32)
    if w.dist == "normal_laplace_spikes":
        spike = r.random((n, w.D)) < 0.01
        lap = r.laplace(0.0, 8.0, size=(n, w.D)).astype(np.float32)
        x = np.where(spike, x + lap, x).astype(np.float32)
    base_kind = K if kind in (K, NEW_K) else V
    sc = _head_constants(w, h, base_kind)
    if sc is not None:
        x = (x * sc[None, :]).astype(np.float32)
    return x


def kv_rows(w: Workload, b: int, h: int, kind: int, t0: int, t1: int) -> np.ndarray:
    """float32 [t1 - t0, D] rows of keys (kind 0) or values (kind 1)."""
    out = np.empty((max(t1 - t0, 0), w.D), dtype=np.float32)
    c0, c1 = t0 // GEN_CHUNK, (t1 + GEN_CHUNK - 1) // GEN_CHUNK
    for c in range(c0, c1):
        blk = _chunk(w, b, h, kind, c, GEN_CHUNK)
        lo, hi = max(t0, c * GEN_CHUNK), min(t1, (c + 1) * GEN_CHUNK)
        out[lo - t0:hi - t0] = blk[lo - c * GEN_CHUNK:hi - c * GEN_CHUNK]
    return out


def mask_channels(w: Workload, h: int, kind: int, calib_tokens: int = 256) -> tuple:
    """Static channel mask of a (KV head, K or V) list: the ``w.chan_mask`` channels of largest
    mean |x| over the first ``calib_tokens`` rows of sequence 0 (float64 means, ties to the lower
    channel), as a caller would calibrate it once."""
    x = kv_rows(w, 0, h, K if kind in (K, NEW_K) else V, 0, calib_tokens).astype(np.float64)
    m = np.abs(x).mean(axis=0)
    order = np.lexsort((np.arange(w.D), -m))
    return tuple(sorted(int(c) for c in order[:w.chan_mask]))


def new_rows(w: Workload, b: int, h: int, kind: int, step: int, n: int = 1) -> np.ndarray:
    """Rows appended at decode step ``step`` (kind 3 = keys, 4 = values)."""
    return _chunk(w, b, h, kind, step, n)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def queries(w: Workload, b: int) -> np.ndarray:
    """bfloat16 bit patterns [Hq, D] of the decode query of sequence b."""
    x = _rng(w.seed, b, 0, Q, 0).standard_normal((w.Hq, w.D), dtype=np.float32)
    return f32_to_bf16_bits(x)


def seq_lens(w: Workload) -> np.ndarray:
    if w.S_range is None:
        return np.full(w.B, w.S, dtype=np.int32)
    lo, hi = w.S_range
    return _rng(w.seed, 7777, 0).integers(lo, hi + 1, size=w.B).astype(np.int32)


def page_tiers(w: Workload, lens: np.ndarray) -> list:
    """Per sequence: bool array over its logical pages, True = FP8 tier (Bernoulli)."""
    out = []
    for b, s in enumerate(lens):
        npg = (int(s) + w.page_size - 1) // w.page_size
        out.append(_rng(w.seed, 7777, 1, b).random(npg) < w.fp8_page_frac)
    return out


def block_tables(w: Workload, tiers: list, max_pages: int):
    """Random-permutation block tables.  Entry = (tier << 31) | slot, where slot indexes the
    page pool of that tier; each pool is filled by a random permutation of its slots.
    Returns (table [B, max_pages] int32 with -1 padding, n_slots_tier2, n_slots_tier1)."""
    n1 = int(sum(int(t.sum()) for t in tiers))
    n2 = int(sum(len(t) for t in tiers)) - n1
    r = _rng(w.seed, 7777, 2)
    perm2 = r.permutation(n2)
    perm1 = r.permutation(n1)
    table = np.full((len(tiers), max_pages), -1, dtype=np.int64)
    i1 = i2 = 0
    for b, t in enumerate(tiers):
        for p, is1 in enumerate(t):
            if is1:
                table[b, p] = (1 << 31) | int(perm1[i1])
                i1 += 1
            else:
                table[b, p] = int(perm2[i2])
                i2 += 1
    return table.astype(np.uint32).view(np.int32), n2, n1


def model_width(w: Workload) -> int:
    return w.Hq * w.D


def hidden_states(w: Workload, step: int = 0, d: int = 0) -> np.ndarray:
    """bfloat16 bit patterns [B, d] of the hidden states entering the attention at ``step``."""
    d = d or model_width(w)
    return np.stack([f32_to_bf16_bits(_rng(w.seed, b, 0, HIDDEN, step).standard_normal(d, dtype=np.float32))
                     for b in range(w.B)])


def norm_gain(w: Workload, d: int = 0) -> np.ndarray:
    """bfloat16 bit patterns [d] of the RMSNorm gain."""
    d = d or model_width(w)
    g = 1.0 + 0.1 * _rng(w.seed, 0, 0, GAIN, 0).standard_normal(d, dtype=np.float32)
    return f32_to_bf16_bits(g.astype(np.float32))


def projection(w: Workload, d: int = 0) -> np.ndarray:
    """bfloat16 bit patterns [(Hq + 2 H) D, d] of the joint Q/K/V projection."""
    d = d or model_width(w)
    n = (w.Hq + 2 * w.H) * w.D
    out = np.empty((n, d), dtype=np.uint16)
    sd = np.float32(1.0 / np.sqrt(d))
    for c in range((n + W_CHUNK - 1) // W_CHUNK):
        r0, r1 = c * W_CHUNK, min(n, (c + 1) * W_CHUNK)
        x = _rng(w.seed, 0, 0, WEIGHT, c).standard_normal((r1 - r0, d), dtype=np.float32) * sd
        out[r0:r1] = f32_to_bf16_bits(x)
    return out
