"""CPU oracle for the quantize-on-append step: group statistics, outlier isolation, quantizer
fit, encoding and packing of one KV row at a time.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Pages cited (titles abridged):
  [P1] "Hierarchical Token Routing and Sub-2-Bit Non-Linear KV Compression ..."
       section "Paradigm 2: Sub-2-Bit Non-Linear KV-Cache Quantization": subsection
       "1. Dynamic Outlier Isolation", subsection "2. Centroid Vector Quantization for
       Residuals" and the ``Sub2BitQuantizedKVCache.compress_kv_head`` listing that follows.
  [P3] "Sub-5ms MoE Inference: Sub-Byte KV Quantization and Expert Pipelining at Scale",
       section "Sub-Byte KV-Cache Quantization" (fp16 outlier tensor, 2-bit packing).
  [P4] "The Sub-10ms Barrier: Fusing Sparse MoE Routing with FP4 KV-Cache Quantization",
       section "2. FP4/INT4 KV-Cache Quantization" (the equations Q = Round(Clamp(X/Scale +
       ZeroPoint, Min, Max)) and S = (max - min)/(2^b - 1), groups of 32 or 64 along the head
       dimension, E2M1) and the ``quantize_kv_cache_fp4`` listing of the same section
       (symmetric INT4: absmax/7 scale clamped at 1e-5, round, clamp to [-8, 7]).

Format variants (stored like their base formats, decoded by the same kernels):
  * "u2": the [P1] listing's uniform codebook, linspace(min, max, 4) over the group's slots with
    the outlier slots zero-filled (the listing's residuals), as torch.linspace forms it (the
    first two points from min, the last two from max, step fl32((max - min) / 3)); stored and
    decoded as "c2" (4 fp16 centroids per group of 64);
  * "int4s": the [P4] listing's symmetric INT4, stored as "int4" with scale S = fp16(max(absmax
    / 7, 1e-5)) over the non-outliers, zero -8 S, code = Clamp(Round(x / S), -8, 7) + 8 (the
    fp16 scale is the one that divides, so that the stored scale reproduces the codes);
  * static channel mask ([P4] "Key Production Engineering Takeaways", item 2: a reserved
    high-precision mask of the top channels by absolute magnitude, kept in FP16): with
    ``channels`` set, the outliers of every row are exactly those channels (instead of the tau
    test), stored as records like any outlier, and the fit runs on the other channels;
    ``top_channels`` picks the mask from calibration rows.

Readings taken where the pages are silent (each is listed in the design doc):
  * every quantity that decides a code is computed in float32 with IEEE round-to-nearest-even,
    no fused multiply-add, correctly rounded division, subnormals kept;
  * every sum over a group uses one fixed pairwise tree (``tree_sum``);
  * statistics are per (row, group of ``g`` channels); the spread is the unbiased standard
    deviation (the listing's ``std``), the comparison is strict, one pass, and the statistics
    include the outliers themselves (the listing computes mean/std before masking);
  * the quantizer is fitted on the non-outliers only ([P1] "remaining non-outlier" values);
    an outlier position is encoded as the code of 0.0 (the listing zero-fills those slots
    before quantizing them);
  * outlier records keep the ORIGINAL value rounded to the outlier dtype (the listing casts
    ``kv_tensor[outlier_mask]``);
  * 2-bit centroids: 4 per group, seeded at the midpoints of the four quartile bins of the
    sorted non-outliers, then a fixed number of Lloyd (k-means) iterations; nearest centroid by
    absolute difference with the first index on ties (the listing's ``argmin``); an empty
    cluster keeps its centroid; centroids stored as fp16;
  * INT4: offset form of the equation: zero = fp16(min), code = Round(Clamp((x - zero)/S, 0,
    15)), which is the page's ZeroPoint = -zero/S written without a quantized-unit zero; a zero
    min or max is taken as +0; a quotient with no value (scale and zero both beyond the fp16
    range) gives code 0;
  * INT3 ([P3] "Sub-Byte KV-Cache Quantization": asymmetric 3-bit packed codes beside the
    outliers): the INT4 fit with b = 3 (S = (max - min)/7, codes 0..7), codes packed LSB-first
    as one bit stream along the channels;
  * FP4: E4M3 block scale = absmax/6 (6 is the largest E2M1 magnitude);
  * FP8 tier: per-row scale absmax/448 in fp32, no outliers.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats as F

F32 = np.float32

FORMATS = ("int4", "fp4", "c2", "fp8row", "u2", "int4s", "int3")
OUTLIER_DTYPES = ("none", "fp16", "e4m3")
CODE_BITS = {"int4": 4, "fp4": 4, "c2": 2, "fp8row": 8, "u2": 2, "int4s": 4, "int3": 3}


@dataclass(frozen=True)
class QuantSpec:
    fmt: str            # one of FORMATS
    group: int          # channels per group (ignored by fp8row)
    outlier: str        # one of OUTLIER_DTYPES
    sigma: float = 3.0  # outlier threshold tau, in standard deviations
    lloyd_iters: int = 8
    channels: tuple = ()  # static channel mask: these channels are the outliers of every row

    def __post_init__(self):
        assert self.fmt in FORMATS and self.outlier in OUTLIER_DTYPES
        if self.fmt == "fp8row":
            assert self.outlier == "none", "the FP8 tier keeps no outliers"
        if self.channels:
            assert self.outlier != "none", "a channel mask keeps its channels as records"


def meta_bytes_per_row(spec: QuantSpec, D: int) -> int:
    if spec.fmt == "fp8row":
        return 4
    ng = D // spec.group
    return ng * {"int4": 4, "fp4": 1, "c2": 8, "u2": 8, "int4s": 4, "int3": 4}[spec.fmt]


def code_bytes_per_row(spec: QuantSpec, D: int) -> int:
    return D * CODE_BITS[spec.fmt] // 8


# ----------------------------------------------------------------------------- reductions
def tree_sum(a: np.ndarray) -> np.ndarray:
    """Fixed pairwise tree over the last axis (length a power of two): for w = n/2, n/4, ..., 1
    set a[i] <- fl32(a[i] + a[i + w]) for i < w; the result is a[0]."""
    a = np.asarray(a, dtype=F32)
    n = a.shape[-1]
    assert n & (n - 1) == 0
    w = n // 2
    while w >= 1:
        a = (a[..., :w] + a[..., w:2 * w]).astype(F32)
        w //= 2
    return a[..., 0]


# ----------------------------------------------------------------------------- outliers
def outlier_mask(xg: np.ndarray, sigma: float) -> np.ndarray:
    """[P1] "1. Dynamic Outlier Isolation" and the listing's mask: |x - mean| > tau * std, with
    mean and unbiased std over the g channels of the group.  Evaluated without sqrt or division:
    x_i is an outlier iff fl32(e_i * (g-1)) > fl32(fl32(tau*tau) * Q2), where d_i = x_i - mean,
    e_i = d_i^2 and Q2 = sum of e over the group."""
    g = xg.shape[-1]
    mean = (tree_sum(xg) * F32(1.0 / g)).astype(F32)  # 1/g is a power of two: exact
    d = (xg - mean[..., None]).astype(F32)
    e = (d * d).astype(F32)
    q2 = tree_sum(e)
    tau2 = (F32(sigma) * F32(sigma)).astype(F32)
    lhs = (e * F32(g - 1)).astype(F32)
    rhs = (tau2 * q2).astype(F32)
    return lhs > rhs[..., None]


def top_channels(x: np.ndarray, k: int) -> tuple:
    """[P4] "Key Production Engineering Takeaways" item 2: the k channels of largest mean absolute
    value over calibration rows x [R, D] (float64 means; ties to the lower channel)."""
    m = np.mean(np.abs(np.asarray(x, dtype=np.float64)), axis=0)
    order = sorted(range(m.shape[0]), key=lambda c: (-m[c], c))
    return tuple(sorted(order[:k]))


# ----------------------------------------------------------------------------- fits
def _fit_int4(xg, keep, levels: int = 15):
    """[P4] S = (max - min)/(2^b - 1) with b = 4 (levels = 15; b = 3 for INT3: 7) over the
    non-outliers; fp16 scale and zero."""
    # min / max are order-free; a zero result is taken as +0 so the stored fp16 bits are
    # defined (x + 0.0 maps -0.0 to +0.0 and leaves every other value unchanged)
    mn = (np.min(np.where(keep, xg, np.inf), axis=-1).astype(F32) + F32(0.0)).astype(F32)
    mx = (np.max(np.where(keep, xg, -np.inf), axis=-1).astype(F32) + F32(0.0)).astype(F32)
    s = ((mx - mn).astype(F32) / F32(levels)).astype(F32)
    s_h = F.fp16_round(s)
    z_h = F.fp16_round(mn)
    xx = np.where(keep, xg, F32(0.0)).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = ((xx - z_h[..., None]).astype(F32) / s_h[..., None]).astype(F32)
    # a quotient with no value (scale and zero both overflowed fp16, inf / inf) gives code 0
    y = np.where(np.isnan(y), F32(0.0), y)
    q = np.rint(np.clip(y, F32(0.0), F32(levels)))
    q = np.where(s_h[..., None] > 0, q, 0).astype(np.uint8)
    meta = np.stack([F.fp16_bits(s_h), F.fp16_bits(z_h)], axis=-1)  # [..., ng, 2] uint16
    return q, meta.view(np.uint8).reshape(*xg.shape[:-2], -1)


def _fit_int4s(xg, keep):
    """[P4] listing ``quantize_kv_cache_fp4``: symmetric scale absmax/7 clamped at 1e-5 (here
    rounded to the fp16 that is stored), codes Clamp(Round(x / S), -8, 7) offset by 8; stored
    as INT4 with zero -8 S, so that code * S + zero = (code - 8) * S."""
    a = np.max(np.where(keep, np.abs(xg), F32(0.0)), axis=-1).astype(F32)
    s = np.maximum((a / F32(7.0)).astype(F32), F32(1e-5)).astype(F32)
    s_h = F.fp16_round(s)
    z_h = F.fp16_round((F32(-8.0) * s_h).astype(F32))
    xx = np.where(keep, xg, F32(0.0)).astype(F32)
    y = (xx / s_h[..., None]).astype(F32)
    q = np.clip(np.rint(y), F32(-8.0), F32(7.0)).astype(np.int32) + 8
    meta = np.stack([F.fp16_bits(s_h), F.fp16_bits(z_h)], axis=-1)
    return q.astype(np.uint8), meta.view(np.uint8).reshape(*xg.shape[:-2], -1)


def _fit_u2(xg, keep):
    """[P1] listing: residuals = the values with the outlier slots set to 0; centroids =
    linspace(min, max, 4) of the residuals (here per group of g channels, the "block" of the
    listing's comment); code = argmin |residual - centroid| (first index on ties).  linspace as
    torch forms it: step = fl32((max - min) / 3), points min, min + step, max - step, max."""
    xx = np.where(keep, xg, F32(0.0)).astype(F32)
    mn = (np.min(xx, axis=-1).astype(F32) + F32(0.0)).astype(F32)   # a zero end is +0
    mx = (np.max(xx, axis=-1).astype(F32) + F32(0.0)).astype(F32)
    step = ((mx - mn).astype(F32) / F32(3.0)).astype(F32)
    c = np.stack([mn, (mn + step).astype(F32), (mx - step).astype(F32), mx], axis=-1)
    c_h = F.fp16_round(c)
    g = xg.shape[-1]
    codes = _nearest(xx.reshape(-1, g), c_h.reshape(-1, 4)).astype(np.uint8).reshape(xg.shape)
    meta = F.fp16_bits(c_h)   # [..., ng, 4] uint16
    return codes, meta.view(np.uint8).reshape(*xg.shape[:-2], -1)


def _fit_fp4(xg, keep):
    """E2M1 codes with an E4M3 block scale absmax/6 over the non-outliers."""
    a = np.max(np.where(keep, np.abs(xg), F32(0.0)), axis=-1).astype(F32)
    s8 = F.e4m3_encode((a / F32(6.0)).astype(F32))
    s8v = F.e4m3_decode(s8).astype(F32)  # exact
    xx = np.where(keep, xg, F32(0.0)).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (xx / s8v[..., None]).astype(F32)
    y = np.where(s8v[..., None] > 0, y, F32(0.0))
    codes = F.e2m1_encode(y)
    codes = np.where(s8v[..., None] > 0, codes, 0).astype(np.uint8)
    return codes, s8.reshape(*xg.shape[:-2], -1)


def _nearest(x, c):
    """argmin_j fl32(|x - c_j|), first index on ties ([P1] listing: distances.argmin)."""
    dist = np.abs((x[..., None] - c[..., None, :]).astype(F32))
    return np.argmin(dist, axis=-1)


def _fit_c2(xg, keep, iters):
    """[P1] "2. Centroid Vector Quantization for Residuals": a 4-centroid codebook per group
    fitted by k-means (Lloyd) on the non-outliers."""
    g = xg.shape[-1]
    lead = xg.shape[:-1]
    flat_x = xg.reshape(-1, g)
    flat_k = keep.reshape(-1, g)
    n = flat_k.sum(axis=-1)
    v = np.sort(np.where(flat_k, flat_x, np.inf), axis=-1)
    j = np.arange(4)
    seed_idx = ((2 * j[None, :] + 1) * n[:, None]) // 8
    c = np.take_along_axis(v, seed_idx, axis=-1).astype(F32)  # [G, 4]
    for _ in range(iters):
        a = _nearest(flat_x, c)
        new_c = c.copy()
        for k in range(4):
            member = flat_k & (a == k)
            cnt = member.sum(axis=-1)
            ssum = tree_sum(np.where(member, flat_x, F32(0.0)).astype(F32))
            upd = cnt > 0
            new_c[upd, k] = (ssum[upd] / cnt[upd].astype(F32)).astype(F32)
        c = new_c
    c_h = F.fp16_round(c)
    xx = np.where(flat_k, flat_x, F32(0.0)).astype(F32)
    codes = _nearest(xx, c_h).astype(np.uint8).reshape(*lead, g)
    meta = F.fp16_bits(c_h).reshape(*lead[:-1], -1, 4)  # [..., ng, 4] uint16
    return codes, meta.view(np.uint8).reshape(*lead[:-1], -1)


def _fit_fp8row(x):
    """FP8 tier ([P2] "Tier 1: High-Precision FP8"): per-row scale absmax/448 (1 if the row is
    all zero), codes = E4M3(x / scale)."""
    a = np.max(np.abs(x), axis=-1).astype(F32)
    s = np.where(a > 0, (a / F32(F.E4M3_MAX)).astype(F32), F32(1.0)).astype(F32)
    codes = F.e4m3_encode((x / s[..., None]).astype(F32))
    return codes, s.view(np.uint8).reshape(*x.shape[:-1], 4)


# ----------------------------------------------------------------------------- packing
def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Packing along the channel axis.  2-bit: every block of 16 channels fills 4 bytes; byte j
    of a block holds channels j, 4+j, 8+j, 12+j in bit pairs 0, 1, 2, 3 (channel 4s+j in bits
    2s..2s+1).  4-bit: byte k holds channel 2k in bits 0-3 and 2k+1 in bits 4-7.  3-bit: one
    little-endian bit stream, channel c in bits 3c..3c+2.  8-bit codes are stored as they are."""
    c = np.asarray(codes, dtype=np.uint8)
    if bits == 8:
        return c.copy()
    if bits == 3:
        D = c.shape[-1]
        bitpos = 3 * np.arange(D)
        out = np.zeros(c.shape[:-1] + (3 * D // 8,), dtype=np.uint8)
        for b in range(3):   # bit b of channel ch goes to stream bit 3 ch + b
            pos = bitpos + b
            vals = ((c >> b) & 1).astype(np.uint8) << (pos % 8).astype(np.uint8)
            for ch in range(D):
                out[..., pos[ch] // 8] |= vals[..., ch]
        return out
    if bits == 2:
        blk = c.reshape(*c.shape[:-1], -1, 4, 4).astype(np.uint16)   # [..., block, s, j]
        out = np.zeros(blk.shape[:-2] + (4,), dtype=np.uint16)       # [..., block, j]
        for sp in range(4):
            out |= blk[..., sp, :] << (2 * sp)
        return out.reshape(*c.shape[:-1], -1).astype(np.uint8)
    c = c.reshape(*c.shape[:-1], -1, 2).astype(np.uint16)
    return (c[..., 0] | (c[..., 1] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray, bits: int, D: int) -> np.ndarray:
    """Inverse of pack_codes: [..., D * bits / 8] bytes -> [..., D] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    if bits == 8:
        return p.copy()
    if bits == 3:
        out = np.zeros(p.shape[:-1] + (D,), dtype=np.uint8)
        for ch in range(D):
            for b in range(3):
                pos = 3 * ch + b
                out[..., ch] |= ((p[..., pos // 8] >> (pos % 8)) & 1) << b
        return out
    if bits == 2:
        blk = p.reshape(*p.shape[:-1], -1, 4)                         # [..., block, j]
        parts = [(blk >> (2 * sp)) & 3 for sp in range(4)]            # bit pair s
        return np.stack(parts, axis=-2).reshape(*p.shape[:-1], D).astype(np.uint8)
    return np.stack([p & 15, p >> 4], axis=-1).reshape(*p.shape[:-1], D).astype(np.uint8)


# ----------------------------------------------------------------------------- rows
@dataclass
class QuantRows:
    codes: np.ndarray      # [R, D] uint8, one logical code per element
    packed: np.ndarray     # [R, code_bytes] uint8
    meta: np.ndarray       # [R, meta_bytes] uint8
    mask: np.ndarray       # [R, D] bool, outlier positions
    outlier_bits: np.ndarray  # [R, D] uint16: fp16 bits or E4M3 code of the original value


def quantize_rows(x: np.ndarray, spec: QuantSpec) -> QuantRows:
    """Quantize rows x [R, D] (float32) independently (O1-O7)."""
    x = np.asarray(x, dtype=F32)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_rows: non-finite input is rejected")
    R, D = x.shape
    if spec.fmt == "fp8row":
        codes, meta = _fit_fp8row(x)
        mask = np.zeros((R, D), dtype=bool)
        obits = np.zeros((R, D), dtype=np.uint16)
        return QuantRows(codes, pack_codes(codes, 8), meta, mask, obits)
    g = spec.group
    assert D % g == 0 and g & (g - 1) == 0
    xg = x.reshape(R, D // g, g)
    if spec.outlier == "none":
        mask_g = np.zeros(xg.shape, dtype=bool)
    elif spec.channels:
        chan = np.zeros(D, dtype=bool)
        chan[list(spec.channels)] = True
        mask_g = np.broadcast_to(chan.reshape(D // g, g), xg.shape).copy()
    else:
        mask_g = outlier_mask(xg, spec.sigma)
    keep = ~mask_g
    if spec.fmt == "int4":
        codes, meta = _fit_int4(xg, keep)
    elif spec.fmt == "int3":
        codes, meta = _fit_int4(xg, keep, 7)
    elif spec.fmt == "int4s":
        codes, meta = _fit_int4s(xg, keep)
    elif spec.fmt == "fp4":
        codes, meta = _fit_fp4(xg, keep)
    elif spec.fmt == "u2":
        codes, meta = _fit_u2(xg, keep)
    else:
        codes, meta = _fit_c2(xg, keep, spec.lloyd_iters)
    codes = codes.reshape(R, D)
    mask = mask_g.reshape(R, D)
    if spec.outlier == "fp16":
        obits = F.fp16_bits(x)
    elif spec.outlier == "e4m3":
        obits = F.e4m3_encode(x).astype(np.uint16)
    else:
        obits = np.zeros((R, D), dtype=np.uint16)
    obits = np.where(mask, obits, 0).astype(np.uint16)
    return QuantRows(codes, pack_codes(codes, CODE_BITS[spec.fmt]), meta.reshape(R, -1), mask,
                     obits)


# ----------------------------------------------------------------------------- dequant
def decode_outlier(bits: np.ndarray, outlier: str) -> np.ndarray:
    if outlier == "fp16":
        return F.fp16_from_bits(bits)
    if outlier == "e4m3":
        return F.e4m3_decode(np.asarray(bits).astype(np.uint8))
    raise ValueError(outlier)


def dequantize_codes(codes: np.ndarray, meta: np.ndarray, spec: QuantSpec) -> np.ndarray:
    """Code + per-group metadata -> float64 values, before outlier patching (O8)."""
    codes = np.asarray(codes, dtype=np.int64)
    R, D = codes.shape
    meta = np.ascontiguousarray(meta, dtype=np.uint8)
    if spec.fmt == "fp8row":
        s = meta.view(np.float32).reshape(R).astype(np.float64)
        return F.e4m3_decode(codes.astype(np.uint8)) * s[:, None]
    g = spec.group
    ng = D // g
    cg = codes.reshape(R, ng, g)
    if spec.fmt in ("int4", "int4s", "int3"):
        sz = F.fp16_from_bits(meta.view(np.uint16).reshape(R, ng, 2))
        out = cg * sz[..., 0:1] + sz[..., 1:2]
    elif spec.fmt == "fp4":
        s8 = F.e4m3_decode(meta.reshape(R, ng))
        out = F.e2m1_decode(cg) * s8[..., None]
    else:
        cent = F.fp16_from_bits(meta.view(np.uint16).reshape(R, ng, 4))
        out = np.take_along_axis(cent, cg, axis=-1)
    return out.reshape(R, D)


def dequantize_rows(q: QuantRows, spec: QuantSpec) -> np.ndarray:
    """Dequantized rows with outlier positions overwritten by the stored outlier value."""
    base = dequantize_codes(q.codes, q.meta, spec)
    if spec.outlier == "none":
        return base
    return np.where(q.mask, decode_outlier(q.outlier_bits, spec.outlier), base)
