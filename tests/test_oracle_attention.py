"""Pins for the float64 attention oracle, the list structure and the byte counts:
50-digit brute force, closed-form special cases, GQA head mapping, torch's SDPA (library),
log-sum-exp merge over arbitrary partitions, and the pages' KV-size formula."""

import json
import os

import mpmath
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import cache as C
from oracle import kvbytes as KB
from oracle import quantize as Q
from workloads.generate import f32_to_bf16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand_qkv(rng, S, D):
    return rng.standard_normal(D), rng.standard_normal((S, D)), rng.standard_normal((S, D))


def test_bruteforce_mpmath_tiny():
    mpmath.mp.dps = 50
    rng = np.random.default_rng(0)
    for S in (1, 2, 5, 8):
        for D in (1, 3, 8):
            q, K, V = _rand_qkv(rng, S, D)
            sc = 0.7
            s = [mpmath.fsum(mpmath.mpf(q[d]) * mpmath.mpf(K[t, d]) for d in range(D)) * sc
                 for t in range(S)]
            e = [mpmath.e ** x for x in s]
            z = mpmath.fsum(e)
            ref = [float(mpmath.fsum(e[t] * mpmath.mpf(V[t, d]) for t in range(S)) / z)
                   for d in range(D)]
            got = A.attention_one(q, K, V, sc)
            assert np.allclose(got, ref, rtol=0, atol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(1)
    q, K, V = _rand_qkv(rng, 9, 16)
    assert np.allclose(A.attention_one(q, K[:1], V[:1], 0.3), V[0])            # S = 1
    assert np.allclose(A.attention_one(np.zeros(16), K, V, 0.3), V.mean(0))   # q = 0
    Ks = np.repeat(K[:1], 9, axis=0)
    assert np.allclose(A.attention_one(q, Ks, V, 0.3), V.mean(0))             # equal keys
    s = K @ q
    t = int(np.argmax(s))
    assert np.allclose(A.attention_one(q, K, V, 1e4), V[t])                    # hard max
    perm = rng.permutation(9)
    assert np.allclose(A.attention_one(q, K[perm], V[perm], 0.3),
                       A.attention_one(q, K, V, 0.3))                          # permutation


def test_gqa_mapping_and_mha_reduction():
    rng = np.random.default_rng(2)
    H, Hq, D = 3, 6, 8
    Kc = rng.standard_normal((H, 1, D))
    Vc = rng.standard_normal((H, 1, D))
    qb = f32_to_bf16_bits(rng.standard_normal((Hq, D)).astype(np.float32))
    o = A.decode_attention(qb, Kc, Vc, 0.5)
    for hq in range(Hq):
        assert np.allclose(o[hq], Vc[hq // 2, 0])  # heads 2h, 2h+1 read KV head h
    # Hq = H: multi-head attention
    K2 = rng.standard_normal((H, 7, D))
    V2 = rng.standard_normal((H, 7, D))
    qb2 = f32_to_bf16_bits(rng.standard_normal((H, D)).astype(np.float32))
    o2 = A.decode_attention(qb2, K2, V2, 0.5)
    from oracle.formats import bf16_to_f64
    qf = bf16_to_f64(qb2)
    for h in range(H):
        assert np.allclose(o2[h], A.attention_one(qf[h], K2[h], V2[h], 0.5))


def test_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(3)
    H, Hq, S, D = 2, 8, 300, 64
    K = rng.standard_normal((H, S, D)) * 2
    V = rng.standard_normal((H, S, D))
    qb = f32_to_bf16_bits(rng.standard_normal((Hq, D)).astype(np.float32))
    got = A.decode_attention(qb, K, V, 1 / np.sqrt(D))
    from oracle.formats import bf16_to_f64
    qt = torch.from_numpy(bf16_to_f64(qb)).view(1, Hq, 1, D)
    kt = torch.from_numpy(np.repeat(K, Hq // H, axis=0)).view(1, Hq, S, D)
    vt = torch.from_numpy(np.repeat(V, Hq // H, axis=0)).view(1, Hq, S, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).view(Hq, D).numpy()
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_lse_merge_any_partition():
    rng = np.random.default_rng(4)
    q, K, V = _rand_qkv(rng, 100, 16)
    K *= 3
    full = A.attention_one(q, K, V, 0.25)
    for _ in range(10):
        cuts = np.sort(rng.choice(np.arange(1, 100), size=rng.integers(1, 8), replace=False))
        bounds = [0, *cuts.tolist(), 100]
        parts = [A.partial_state(q, K[a:b], V[a:b], 0.25) for a, b in zip(bounds, bounds[1:])]
        assert np.allclose(A.lse_merge(parts), full, atol=1e-13)


# ----------------------------------------------------------------------------- lists
def test_list_block_starts_and_dequant():
    rng = np.random.default_rng(5)
    S, D = 203, 128
    x = rng.standard_normal((S, D)).astype(np.float32)
    x[rng.random(x.shape) < 0.02] *= 12
    spec = Q.QuantSpec("c2", 64, "e4m3")
    L = C.build_list(x, spec)
    t = L.idx.astype(np.int64) // D
    assert np.all(np.diff(L.idx.astype(np.int64)) > 0)
    for blk in range(len(L.block_start)):
        assert L.block_start[blk] == np.sum(t < 16 * blk)   # brute-force count
    assert L.count == len(L.idx) == int(Q.quantize_rows(x, spec).mask.sum())
    assert C.records_before(L.idx, D, 100) == np.sum(t < 100)
    d1 = C.dequantize_list(L.codes, L.meta, L.idx, L.vals, spec, D)
    d2 = Q.dequantize_rows(Q.quantize_rows(x, spec), spec)
    assert np.array_equal(d1, d2)


def test_tiered_list_fp8_rows_have_no_records():
    rng = np.random.default_rng(6)
    S, D = 100, 128
    x = (rng.standard_normal((S, D)) * 3).astype(np.float32)
    x[:, 7] = 40.0
    spec = Q.QuantSpec("c2", 64, "e4m3")
    spec8 = Q.QuantSpec("fp8row", 0, "none")
    tiers = np.array([False, True, False, True, True, False, False])
    L = C.build_list(x, spec, tiers, spec8)
    t = L.idx.astype(np.int64) // D
    assert not np.any(L.tier1[t])
    d = C.dequantize_list(L.codes, L.meta, L.idx, L.vals, spec, D, L.tier1, L.packed8,
                          L.meta8, spec8)
    d8 = Q.dequantize_rows(Q.quantize_rows(x, spec8), spec8)
    assert np.array_equal(d[L.tier1], d8[L.tier1])


# ----------------------------------------------------------------------------- bytes
def test_kv_size_formula_spot_values():
    with open(os.path.join(GOLD, "kv_size_formula.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        got = KB.kv_bytes("fp16", case["L"], case["H"], case["D"], case["tokens"])
        assert got == case["bytes"]
        if "at_least" in case:
            assert got >= case["at_least"]
    r = g["ratios"]
    # 2-bit codes vs 8-bit codes, 4-bit codes vs 16-bit: code bits only
    assert 8 / 2 == r["fp8_to_2bit_codes_footprint"]["value"]
    assert 1 - 4 / 16 == r["fp16_to_4bit_codes_traffic_reduction"]["value"]


def test_kv_bytes_quantized_rows_match_oracle_buffers():
    D = 128
    for fmt, g, out in [("int4", 32, "fp16"), ("fp4", 32, "fp16"), ("c2", 64, "e4m3"),
                        ("fp8row", 0, "none")]:
        spec = Q.QuantSpec(fmt, g, out)
        per_row = Q.code_bytes_per_row(spec, D) + Q.meta_bytes_per_row(spec, D)
        assert KB.kv_bytes(fmt, 1, 1, D, 1, g) == 2 * per_row
        assert KB.kv_bytes(fmt, 2, 3, D, 5, g, 7, out) == 2 * 2 * 3 * 5 * per_row + 7 * (
            KB.OUTLIER_VALUE_BYTES[out] + 4)
