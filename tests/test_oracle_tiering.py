"""Pins for the tiering oracle (per-page attention mass, hot pages, demotion of FP8 pages):
50-digit brute force of the weights, closed forms of the mass (equal keys, a dominant token,
query heads split between pages), brute-force ranking with constructed ties, exact
reconstruction of demoted rows that the 2-bit codebook can hold, untouched rows, and list
invariants (sorted records, block starts equal to brute-force counts)."""

import math

import mpmath
import numpy as np
import pytest

from oracle import cache as OC
from oracle import quantize as OQ
from oracle import tiering as T

F32 = np.float32
SPEC = OQ.QuantSpec("c2", 64, "e4m3", 3.0, 8)
SPEC8 = OQ.QuantSpec("fp8row", 0, "none")


# ----------------------------------------------------------------------------- weights, mass
def test_weights_match_50_digit_brute_force():
    rng = np.random.default_rng(0)
    for S, D in ((1, 4), (5, 8), (8, 3)):
        q = rng.standard_normal(D)
        K = rng.standard_normal((S, D)) * 3
        sm = 0.7
        got = T.attention_weights(q, K, sm)
        mpmath.mp.dps = 50
        s = [mpmath.fsum(mpmath.mpf(float(q[d])) * mpmath.mpf(float(K[t, d])) for d in range(D)) * mpmath.mpf(sm)
             for t in range(S)]
        e = [mpmath.exp(x) for x in s]
        tot = mpmath.fsum(e)
        ref = np.array([float(x / tot) for x in e])
        assert np.max(np.abs(got - ref)) < 1e-15


def test_mass_of_equal_keys_is_the_token_share_of_each_page():
    # every score equal: each token weighs 1/S, a page its token count / S (partial last page)
    S, D = 37, 8
    K = {0: np.tile(np.arange(D, dtype=float), (S, 1)), 1: np.ones((S, D))}
    q = np.random.default_rng(1).standard_normal((4, D))
    m = T.page_mass(q, K, 4, 2, 0.3, S)
    assert np.allclose(m, [16 / 37, 16 / 37, 5 / 37], rtol=0, atol=1e-15)


def test_mass_of_a_dominant_token_and_the_head_average():
    # query heads 0, 1 read KV head 0, whose token 20 dominates; heads 2, 3 read KV head 1,
    # whose token 40 dominates: half the mass on page 1, half on page 2
    S, D = 50, 4
    K0 = np.zeros((S, D)); K0[20] = 100.0
    K1 = np.zeros((S, D)); K1[40] = 100.0
    q = np.ones((4, D))
    m = T.page_mass(q, {0: K0, 1: K1}, 4, 2, 1.0, S)
    assert abs(m[1] - 0.5) < 1e-12 and abs(m[2] - 0.5) < 1e-12 and abs(np.sum(m) - 1) < 1e-15
    assert m[0] < 1e-12 and m[3] < 1e-12


def test_masses_sum_to_one():
    rng = np.random.default_rng(2)
    S, D, H, Hq = 300, 128, 2, 8
    K = {h: rng.standard_normal((S, D)) for h in range(H)}
    q = rng.standard_normal((Hq, D))
    m = T.page_mass(q, K, Hq, H, 1 / math.sqrt(D), S)
    assert len(m) == 19 and abs(np.sum(m) - 1.0) < 1e-12 and np.all(m > 0)


# ----------------------------------------------------------------------------- hot pages
def test_hot_pages_brute_force_and_ties():
    rng = np.random.default_rng(3)
    for n in (1, 7, 20, 333):
        mass = rng.random(n)
        mass[rng.integers(n, size=n // 3)] = 0.5           # ties
        for frac in (0.0, 0.1, 0.15, 0.5, 1.0):
            hot = T.hot_pages(mass, frac)
            k = min(n, math.ceil(frac * n))
            assert hot.sum() == k
            # brute force: page p is hot iff fewer than k pages beat it (larger mass, or equal
            # mass and a lower page number)
            for p in range(n):
                beat = np.sum((mass > mass[p]) | ((mass == mass[p]) & (np.arange(n) < p)))
                assert hot[p] == (beat < k)


def test_only_cold_fp8_pages_are_demoted():
    mass = np.array([0.4, 0.05, 0.3, 0.05, 0.2])
    tier1 = np.array([True, True, False, True, False])
    d = T.pages_to_demote(tier1, mass, 0.4)   # 2 hot pages: 0 and 2
    assert d.tolist() == [False, True, False, True, False]


# ----------------------------------------------------------------------------- demotion
def _rows(S, rng, D=128):
    return (rng.standard_normal((S, D)) * rng.uniform(0.5, 3, (1, D))).astype(F32)


def test_fp8_rows_are_one_float32_product():
    # fl32(e4m3(code) * scale) equals the float64 product rounded once (the product of a 4-bit
    # and a 24-bit significand is exact in float64)
    x = _rows(64, np.random.default_rng(4))
    lst = OC.build_list(x, SPEC, np.array([True, False, True, True]), SPEC8)
    got = T.fp8_rows_f32(lst, SPEC8, 128)
    ref = T.dequantized_fp8_check(lst, SPEC8, 128).astype(F32)
    rows = lst.tier1
    assert np.array_equal(got[rows], ref[rows]) and np.all(got[~rows] == 0)


def test_no_demotion_is_the_identity():
    x = _rows(90, np.random.default_rng(5))
    tiers = np.array([False, True, False, True, True, False])
    a = OC.build_list(x, SPEC, tiers, SPEC8)
    b = T.demote(x, tiers, np.zeros(6, dtype=bool), SPEC, SPEC8)
    for f in ("packed", "meta", "idx", "vals", "block_start", "packed8", "meta8", "tier1"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_demoted_rows_that_the_codebook_holds_come_back_exactly():
    # rows of the values -2, -1, 1, 2 (16 channels each per group): the FP8 row scale is 2/448,
    # every x / scale is E4M3-exact (+-224, +-448), and the 2-bit fit reproduces the four values
    rng = np.random.default_rng(6)
    S = 32
    base = np.array([-2.0, -1.0, 1.0, 2.0], dtype=F32)
    x = np.stack([rng.permutation(np.tile(base, 32)) for _ in range(S)]).astype(F32)
    tiers = np.array([True, True])
    lst = T.demote(x, tiers, np.array([True, False]), SPEC, SPEC8)
    assert lst.tier1.tolist() == [False] * 16 + [True] * 16
    deq = OC.dequantize_list(lst.codes, lst.meta, lst.idx, lst.vals, SPEC, 128, lst.tier1,
                             lst.packed8, lst.meta8, SPEC8)
    assert np.array_equal(deq[:16], x[:16].astype(np.float64))
    assert lst.count == 0


def test_demotion_keeps_other_rows_and_list_invariants():
    rng = np.random.default_rng(7)
    S = 16 * 9 + 5
    x = _rows(S, rng)
    x[rng.integers(S, size=40), rng.integers(128, size=40)] *= 30      # spikes: outliers
    tiers = np.array([True, False, True, True, False, True, False, True, True, True])
    dem = np.array([True, False, False, True, False, False, False, True, False, True])
    before = OC.build_list(x, SPEC, tiers, SPEC8)
    after = T.demote(x, tiers, dem, SPEC, SPEC8)
    rows_dem = np.repeat(dem, 16)[:S]
    rows_2 = np.repeat(~tiers, 16)[:S]
    rows_hot8 = np.repeat(tiers & ~dem, 16)[:S]
    assert np.array_equal(after.packed[rows_2], before.packed[rows_2])
    assert np.array_equal(after.meta[rows_2], before.meta[rows_2])
    assert np.array_equal(after.packed8[rows_hot8], before.packed8[rows_hot8])
    assert np.array_equal(after.tier1, rows_hot8)
    # records of 2-bit rows unchanged, records of demoted rows present, none on FP8 rows
    t_after = after.idx.astype(np.int64) // 128
    t_before = before.idx.astype(np.int64) // 128
    keep = rows_2[t_before]
    kept_after = rows_2[t_after]
    assert np.array_equal(before.idx[keep], after.idx[kept_after])
    assert np.array_equal(before.vals[keep], after.vals[kept_after])
    assert not np.any(rows_hot8[t_after]) and np.any(rows_dem[t_after])
    # sorted, block starts equal to brute-force counts
    assert np.all(np.diff(after.idx.astype(np.int64)) > 0)
    for blk in range((S + 15) // 16):
        assert after.block_start[blk] == np.sum(t_after < 16 * blk)
    # a demoted row's records carry the E4M3 code of its FP8-dequantized value
    x8 = T.fp8_rows_f32(before, SPEC8, 128)
    sel = rows_dem[t_after]
    c = after.idx[sel].astype(np.int64) % 128
    from oracle import formats as F
    assert np.array_equal(after.vals[sel], F.e4m3_encode(x8[t_after[sel], c]).astype(np.uint8))


def test_demoting_a_2bit_page_is_rejected():
    x = _rows(32, np.random.default_rng(8))
    with pytest.raises(AssertionError):
        T.demote(x, np.array([False, True]), np.array([True, False]), SPEC, SPEC8)
