"""Number formats used by the quantized KV cache, written from their published definitions.

TEST INFRASTRUCTURE ONLY: nothing under ``oracle/`` is part of the product path.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may use it.

Formats (each encoder rounds to nearest, ties to even, as ``torch.round`` does in the FP4/INT4
listing on "The Sub-10ms Barrier: Fusing Sparse MoE Routing with FP4 KV-Cache Quantization",
section "Implementation: High-Throughput Fused Kernel Pipeline"):

* binary16 (IEEE 754-2008): 1 sign, 5 exponent (bias 15), 10 mantissa bits, subnormals kept.
  Used for outlier values (the "FP16 Outlier Tensor (Protected)" box of the figure in section
  "Sub-Byte KV-Cache Quantization" on "Sub-5ms MoE Inference ..."), INT4 scale/zero and
  2-bit centroids.
* E4M3FN (OCP 8-bit floating point spec): 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
  infinities, 0x7F/0xFF are NaN, largest finite value 448.  The outlier store named in section
  "1. Dynamic Outlier Isolation" of "Hierarchical Token Routing and Sub-2-Bit Non-Linear KV
  Compression ..." (and its listing's ``.to(torch.float8_e4m3fn)``).  Encoding here saturates
  to +-448 instead of producing NaN.
* E2M1 (OCP MX spec FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Section "2. FP4/INT4 KV-Cache Quantization" of
  "The Sub-10ms Barrier ...".

Everything is plain NumPy; arithmetic that decides a rounding is done in float64, where every
float32 input and every candidate value is exact.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


# ----------------------------------------------------------------------------- binary16
def fp16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest binary16 (ties to even), returned as float32.  NumPy's cast is the
    IEEE conversion."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def fp16_bits(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def fp16_from_bits(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


# ----------------------------------------------------------------------------- E4M3FN
def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Finite float32 -> E4M3FN code, round to nearest even, saturating to +-448."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode: non-finite input")
    a = np.abs(x.astype(np.float64))
    neg = np.signbit(x)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: value = q * 2^-9; q == 8 is the smallest normal (code 8), so the
    # integer q is the code itself
    code = np.where(sub, np.rint(a * 2.0 ** 9).astype(np.int64), code)
    nrm = ~sub
    mant, ex = np.frexp(np.where(nrm, a, 1.0))  # a = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1  # a = (2*mant) * 2^e with 2*mant in [1, 2)
    mq = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)
    carry = mq == 8
    e = np.where(carry, e + 1, e)
    mq = np.where(carry, 0, mq)
    ncode = ((e + 7) << 3) | mq
    code = np.where(nrm, ncode, code)
    code = np.where(a >= E4M3_MAX, 0x7E, code)  # saturate (also covers values that round up)
    code = np.minimum(code, 0x7E)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


# ----------------------------------------------------------------------------- E2M1
def e2m1_decode(code: np.ndarray) -> np.ndarray:
    c = np.asarray(code, dtype=np.int64)
    v = E2M1_VALUES[c & 7]
    return np.where(c & 8, -v, v)


def e2m1_encode(y: np.ndarray) -> np.ndarray:
    """float32 -> 4-bit code: nearest magnitude in E2M1_VALUES (ties -> even code, |y| > 6
    -> 6), sign bit = signbit(y)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))[..., None]
    dist = np.abs(a - E2M1_VALUES)
    best = dist.min(axis=-1, keepdims=True)
    tie = dist == best
    # among the nearest candidates take the even code; candidates are at most two adjacent
    # codes, so exactly one of them is even
    even = (np.arange(8) % 2 == 0)
    pick_even = tie & even
    has_even = pick_even.any(axis=-1)
    mag = np.where(has_even, np.argmax(pick_even, axis=-1), np.argmax(tie, axis=-1))
    return (mag | np.where(np.signbit(y), 8, 0)).astype(np.uint8)


# ----------------------------------------------------------------------------- bfloat16
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
