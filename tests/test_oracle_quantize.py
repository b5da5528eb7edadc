"""Pins for the oracle's quantizer: reduction tree structure, outlier predicate (closed-form rate,
hard per-group cap, Samuelson bound, fp64 re-expression of the listing's rule, a constructed
equality case), INT4 / FP4 / FP8 round-trip bounds and exact grids, 2-bit seeds, Lloyd against
an independent float64 implementation, and brute-force optimal partitions."""

import itertools

import numpy as np
import pytest
from scipy import stats

from oracle import formats as F
from oracle import quantize as Q

F32 = np.float32


# ----------------------------------------------------------------------------- tree
def test_tree_sum_pairs_across_halves():
    # for w = 2 then 1: (a0 + a2) + (a1 + a3).  Adjacent pairing or a sequential sum gives 0 or 1.
    a = np.array([1e8, 1.0, -1e8, 1.0], dtype=F32)
    assert Q.tree_sum(a) == 2.0
    assert ((F32(1e8) + F32(1.0)) + F32(-1e8)) + F32(1.0) == 1.0  # a sequential sum differs


def test_tree_sum_exact_on_integers():
    rng = np.random.default_rng(0)
    for g in (32, 64, 128):
        a = rng.integers(-1000, 1000, size=(50, g)).astype(F32)
        assert np.array_equal(Q.tree_sum(a), a.astype(np.int64).sum(axis=1).astype(F32))


# ----------------------------------------------------------------------------- outliers
def _tail_prob(g, tau):
    # studentized residual r = d / s (s unbiased): r^2 g / (g-1)^2 ~ Beta(1/2, (g-2)/2)
    x = tau * tau * g / (g - 1) ** 2
    return stats.beta.sf(x, 0.5, (g - 2) / 2)


@pytest.mark.parametrize("g,tau", [(32, 3.0), (64, 3.0), (64, 2.5)])
def test_outlier_rate_closed_form(g, tau):
    rng = np.random.default_rng(10 + g)
    x = rng.standard_normal((200000, g)).astype(F32)
    rate = Q.outlier_mask(x, tau).mean()
    p = _tail_prob(g, tau)
    n = x.size
    sd = np.sqrt(p * (1 - p) / n)
    assert abs(rate - p) < 5 * sd, (rate, p)


def test_outlier_closed_form_values_quoted():
    # the survey's numbers for tau = 3 (sanity of the closed form itself)
    assert abs(_tail_prob(32, 3.0) - 1.1837e-3) < 1e-6
    assert abs(_tail_prob(64, 3.0) - 1.8992e-3) < 1e-6


@pytest.mark.parametrize("g,tau,cap", [(32, 3.0, 3), (64, 3.0, 6), (32, 3.5, 2), (64, 3.5, 5)])
def test_outlier_hard_cap(g, tau, cap):
    # m outliers need m * tau^2 * Q2 / (g-1) < Q2, so m <= ceil((g-1)/tau^2) - 1
    rng = np.random.default_rng(g)
    x = rng.standard_normal((20000, g)).astype(F32)
    # heavy tails and planted spikes push towards the cap
    k = rng.integers(0, cap + 3, size=20000)
    for i in range(20000):
        pos = rng.choice(g, size=k[i], replace=False)
        x[i, pos] += (rng.choice([-1, 1], size=k[i]) * rng.uniform(20, 200, size=k[i])).astype(F32)
    cnt = Q.outlier_mask(x, tau).sum(axis=1)
    assert cnt.max() <= cap
    # a balanced pattern of m = 2*floor(cap/2) spikes +-A (mean 0) reaches m: (g-1) > tau^2 m
    m = 2 * (cap // 2)
    y = np.zeros((1, g), dtype=F32)
    y[0, :m] = np.tile([50.0, -50.0], m // 2)
    assert Q.outlier_mask(y, tau).sum() == m


def test_samuelson_bound_and_constant_group():
    rng = np.random.default_rng(5)
    x = (rng.standard_t(1.5, size=(20000, 32)) * 10).astype(F32)
    # max |x - mean| / s <= (g-1)/sqrt(g) = 5.48 for g = 32: tau = 5.6 can never flag
    assert not Q.outlier_mask(x, 5.6).any()
    assert Q.outlier_mask(x, 3.0).any()
    assert not Q.outlier_mask(np.full((3, 64), 7.25, dtype=F32), 3.0).any()


def test_outlier_rule_matches_fp64_listing_rule():
    # the listing: mean over the head-group, unbiased std, strict |x - mean| > tau * std
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((30000, 64)) * rng.lognormal(0, 1, (30000, 1))).astype(F32)
    x[rng.random(x.shape) < 0.01] *= 9
    got = Q.outlier_mask(x, 3.0)
    xd = x.astype(np.float64)
    mu = xd.mean(axis=1, keepdims=True)
    sd = xd.std(axis=1, ddof=1, keepdims=True)
    z = np.abs(xd - mu) / sd
    ref = z > 3.0
    clear = np.abs(z - 3.0) > 1e-5
    assert np.array_equal(got[clear], ref[clear])
    assert (~clear).mean() < 1e-3


def test_outlier_strict_inequality_constructed_equality():
    # g = 64, tau = 2: six +4, six -4, seven +2, seven -2, two +1, two -1, 34 zeros.
    # mean 0, Q2 = 12*16 + 14*4 + 4 = 252, and for the +-4 entries 63 * 16 = 1008 = 4 * 252:
    # exact equality, so the strict test flags nothing; tau = 1.99 flags the twelve +-4.
    x = np.zeros((1, 64), dtype=F32)
    vals = [4] * 6 + [-4] * 6 + [2] * 7 + [-2] * 7 + [1, 1, -1, -1]
    x[0, :len(vals)] = vals
    assert not Q.outlier_mask(x, 2.0).any()
    assert Q.outlier_mask(x, 1.99).sum() == 12


def test_outlier_mask_scale_invariance():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5000, 64)).astype(F32)
    m = Q.outlier_mask(x, 3.0)
    for k in (-3, 5):
        assert np.array_equal(Q.outlier_mask((x * F32(2.0 ** k)).astype(F32), 3.0), m)


# ----------------------------------------------------------------------------- INT4
def test_int4_exact_on_grid():
    rng = np.random.default_rng(8)
    R = 500
    z = F.fp16_round(rng.uniform(-5, 5, R).astype(F32))
    s = F.fp16_round(rng.uniform(0.01, 0.5, R).astype(F32))
    k = rng.integers(0, 16, size=(R, 128))
    k[:, 0], k[:, 1] = 0, 15
    for gi in range(4):
        k[:, 32 * gi], k[:, 32 * gi + 1] = 0, 15
    x = (z[:, None].astype(np.float64) + k * s[:, None].astype(np.float64)).astype(F32)
    exact = x.astype(np.float64) == z[:, None] + k * s[:, None].astype(np.float64)
    rows = exact.all(axis=1)
    spec = Q.QuantSpec("int4", 32, "none")
    q = Q.quantize_rows(x[rows], spec)
    d = Q.dequantize_rows(q, spec)
    # S = (max-min)/15 must come back exactly as s for grid data
    assert np.array_equal(q.codes, k[rows].astype(np.uint8))
    assert np.array_equal(d, x[rows].astype(np.float64))


def test_int4_roundtrip_bound_and_monotone():
    rng = np.random.default_rng(9)
    spec = Q.QuantSpec("int4", 32, "fp16")
    for off, sc in [(0, 1), (100, 0.3), (-1000, 30), (0, 1e-3)]:
        x = (off + sc * rng.standard_normal((2000, 128))).astype(F32)
        q = Q.quantize_rows(x, spec)
        d = Q.dequantize_rows(q, spec)
        xg = x.reshape(-1, 32).astype(np.float64)
        keep = ~q.mask.reshape(-1, 32)
        mn = np.where(keep, xg, np.inf).min(1)
        mx = np.where(keep, xg, -np.inf).max(1)
        sz = F.fp16_from_bits(q.meta.view(np.uint16).reshape(-1, 2))
        s_exact = (mx - mn) / 15
        bound = 0.5 * sz[:, 0] + 15 * np.abs(s_exact - sz[:, 0]) + np.abs(mn - sz[:, 1])
        err = np.abs(d.reshape(-1, 32) - xg)
        lim = bound[:, None] + 2.0 ** -20 * np.maximum(np.abs(xg), np.abs(sz[:, 1:2]))
        assert np.all((err <= lim)[keep])
        codes = q.codes.reshape(-1, 32).astype(int)
        # codes are monotone in x within a group (non-outliers)
        for i in range(0, len(xg), 97):
            o = np.argsort(xg[i][keep[i]], kind="stable")
            assert np.all(np.diff(codes[i][keep[i]][o]) >= 0)
        # min -> 0 and max -> 15 wherever the fp16 rounding of zero and scale moves the ends by
        # less than half a step
        safe = (np.abs(mn - sz[:, 1]) + 15 * np.abs(s_exact - sz[:, 0])) < 0.45 * sz[:, 0]
        assert safe.mean() > 0.5
        cmax = np.where(keep, codes, -1).max(1)
        cmin = np.where(keep, codes, 99).min(1)
        assert np.all(cmax[safe] == 15) and np.all(cmin[safe] == 0)
        # outlier values are the original values rounded to fp16
        assert np.array_equal(d[q.mask], F.fp16_round(x[q.mask]).astype(np.float64))


def test_int4_matches_pages_zero_point_form_fp64():
    # Q = Round(Clamp(X/Scale + ZeroPoint, 0, 15)) with ZeroPoint = -zero/Scale, in fp64
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((3000, 128)) * 2 + 1).astype(F32)
    spec = Q.QuantSpec("int4", 32, "fp16")
    q = Q.quantize_rows(x, spec)
    sz = F.fp16_from_bits(q.meta.view(np.uint16).reshape(-1, 2))
    xg = np.where(q.mask, 0, x).reshape(-1, 32).astype(np.float64)
    y = xg / sz[:, :1] - sz[:, 1:] / sz[:, :1]
    ref = np.rint(np.clip(y, 0, 15))
    frac = np.abs(np.abs(y - np.floor(y)) - 0.5)
    clear = frac > 1e-4
    assert np.array_equal(q.codes.reshape(-1, 32)[clear], ref[clear])


# ----------------------------------------------------------------------------- FP4
def test_fp4_roundtrip_bound():
    rng = np.random.default_rng(11)
    spec = Q.QuantSpec("fp4", 32, "fp16")
    x = (rng.standard_normal((4000, 128)) * rng.lognormal(0, 1, (4000, 1))).astype(F32)
    q = Q.quantize_rows(x, spec)
    d = Q.dequantize_rows(q, spec)
    s8 = F.e4m3_decode(q.meta.reshape(-1))  # [R*4]
    xg = x.reshape(-1, 32).astype(np.float64)
    dg = d.reshape(-1, 32)
    keep = ~q.mask.reshape(-1, 32)
    y = np.abs(xg) / s8[:, None]
    step = np.where(y <= 2, 0.25, np.where(y <= 4, 0.5, 1.0))
    lim = s8[:, None] * step + 2.0 ** -23 * np.abs(xg)
    assert np.all((np.abs(dg - xg) <= lim)[keep])
    # scale: E4M3 of absmax/6 over non-outliers; the max maps next to 6
    a = np.where(keep, np.abs(xg), 0).max(1)
    assert np.array_equal(q.meta.reshape(-1), F.e4m3_encode((a / 6).astype(F32)))


def test_fp4_tiny_group_all_zero():
    x = np.full((1, 32), 6 * 2.0 ** -11, dtype=F32)  # absmax/6 = 2^-11 < half of 2^-9
    q = Q.quantize_rows(x, Q.QuantSpec("fp4", 32, "none"))
    assert q.meta[0, 0] == 0 and not q.codes.any()


# ----------------------------------------------------------------------------- FP8 row
def test_fp8row_roundtrip():
    rng = np.random.default_rng(12)
    spec = Q.QuantSpec("fp8row", 0, "none")
    x = (rng.standard_normal((3000, 128)) * rng.lognormal(0, 2, (3000, 1))).astype(F32)
    q = Q.quantize_rows(x, spec)
    d = Q.dequantize_rows(q, spec)
    s = q.meta.view(np.float32).reshape(-1).astype(np.float64)
    a = np.abs(x).max(1)
    assert np.allclose(s, a / 448, rtol=2 ** -23)
    err = np.abs(d - x)
    lim = np.maximum(np.abs(x) * 2.0 ** -4, s[:, None] * 2.0 ** -10) * (1 + 2 ** -20)
    assert np.all(err <= lim)
    z = Q.quantize_rows(np.zeros((1, 128), F32), spec)
    assert z.meta.view(np.float32)[0] == 1.0 and not z.codes.any()


# ----------------------------------------------------------------------------- 2-bit
def test_c2_seeds_are_quartile_bin_midpoints():
    x = np.arange(64, dtype=F32)[None, :]
    q = Q.quantize_rows(x, Q.QuantSpec("c2", 64, "none", lloyd_iters=0))
    cent = F.fp16_from_bits(q.meta.view(np.uint16).reshape(4))
    assert cent.tolist() == [8.0, 24.0, 40.0, 56.0]
    # with 4 outliers removed n = 60: ranks floor(7.5), floor(22.5), floor(37.5), floor(52.5)
    x = np.arange(64, dtype=F32)
    x[[3, 20, 40, 60]] = [5000, -5000, 4000, -4000]
    q = Q.quantize_rows(x[None, :], Q.QuantSpec("c2", 64, "e4m3", sigma=1.0, lloyd_iters=0))
    keep = np.sort(x[~q.mask[0]])
    assert len(keep) == 60
    cent = F.fp16_from_bits(q.meta.view(np.uint16).reshape(4))
    assert cent.tolist() == [float(keep[7]), float(keep[22]), float(keep[37]), float(keep[52])]


def test_c2_four_equal_population_values_exact():
    rng = np.random.default_rng(13)
    for _ in range(200):
        vals = np.sort(F.fp16_round(rng.uniform(-3, 3, 4).astype(F32)))
        if len(np.unique(vals)) < 4:
            continue
        x = rng.permutation(np.repeat(vals, 16)).astype(F32)[None, :]
        q = Q.quantize_rows(x, Q.QuantSpec("c2", 64, "none"))
        assert np.array_equal(Q.dequantize_rows(q, Q.QuantSpec("c2", 64, "none"))[0],
                              x[0].astype(np.float64))


def _lloyd_fp64(x, iters):
    """Independent float64 Lloyd (plain loops) with the same seeding and tie rules."""
    v = sorted(x)
    n = len(v)
    c = [v[((2 * j + 1) * n) // 8] for j in range(4)]
    for _ in range(iters):
        sums, cnts = [0.0] * 4, [0] * 4
        for xi in x:
            d = [abs(xi - cj) for cj in c]
            a = d.index(min(d))
            sums[a] += xi
            cnts[a] += 1
        c = [sums[j] / cnts[j] if cnts[j] else c[j] for j in range(4)]
    return np.array(c)


def test_c2_lloyd_matches_independent_fp64():
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((300, 64)) * rng.lognormal(0, 1, (300, 1))).astype(F32)
    spec = Q.QuantSpec("c2", 64, "none")
    q = Q.quantize_rows(x, spec)
    cent = F.fp16_from_bits(q.meta.view(np.uint16).reshape(300, 4))
    ref = np.array([_lloyd_fp64([float(t) for t in row], 8) for row in x])
    close = np.all(np.abs(cent - ref) <= 2.0 ** -10 * np.maximum(np.abs(ref), 1e-3) * 2, axis=1)
    assert close.mean() > 0.98


def _lloyd_fp64_margin(x, iters):
    """The float64 Lloyd above, also returning the smallest gap between an element's nearest
    and second-nearest centroid over every assignment it makes (the seeds' and each iteration's)
    and the final assignment's."""
    v = sorted(x)
    n = len(v)
    c = [v[((2 * j + 1) * n) // 8] for j in range(4)]
    gap = float("inf")
    for it in range(iters + 1):
        sums, cnts = [0.0] * 4, [0] * 4
        for xi in x:
            d = sorted((abs(xi - cj), j) for j, cj in enumerate(c))
            gap = min(gap, d[1][0] - d[0][0])
            a = min(range(4), key=lambda j: (abs(xi - c[j]), j))
            sums[a] += xi
            cnts[a] += 1
        if it == iters:
            break
        c = [sums[j] / cnts[j] if cnts[j] else c[j] for j in range(4)]
    return np.array(c), gap


@pytest.mark.parametrize("iters", [1, 2, 8])
def test_c2_lloyd_equals_fp64_where_no_assignment_is_close(iters):
    """Where no element lies within a small margin of two centroids at any iteration, float32
    and float64 Lloyd make the same assignments, so their centroids differ only by the
    rounding of the float32 sums: the stored fp16 centroids must equal the float64 centroids
    rounded to fp16, except for a value within that rounding of an fp16 rounding boundary."""
    rng = np.random.default_rng(140 + iters)
    x = (rng.standard_normal((400, 64)) * rng.lognormal(0, 1, (400, 1))).astype(F32)
    spec = Q.QuantSpec("c2", 64, "none", lloyd_iters=iters)
    q = Q.quantize_rows(x, spec)
    cent = F.fp16_from_bits(q.meta.view(np.uint16).reshape(400, 4)).astype(np.float64)
    checked = 0
    for r in range(400):
        row = [float(t) for t in x[r]]
        ref, gap = _lloyd_fp64_margin(row, iters)
        scale = max(abs(t) for t in row)
        if gap <= 1e-4 * scale:
            continue
        want = F.fp16_round(ref.astype(F32)).astype(np.float64)
        for j in range(4):
            if cent[r, j] == want[j]:
                continue
            # a float64 centroid this close to an fp16 rounding boundary may round either way
            ulp = np.spacing(np.float16(want[j])).astype(np.float64)
            lo, hi = sorted((cent[r, j], want[j]))
            mid = (lo + hi) / 2
            assert hi - lo <= ulp * 1.0001 and abs(ref[j] - mid) <= 1e-5 * abs(ref[j]), \
                (r, j, cent[r, j], want[j], ref[j])
        checked += 1
    assert checked >= 300, checked


def test_c2_sse_vs_bruteforce_optimum_and_monotone():
    rng = np.random.default_rng(15)
    spec_it = [Q.QuantSpec("c2", 64, "none", lloyd_iters=i) for i in range(9)]
    for trial in range(20):
        x = rng.standard_normal(64).astype(F32)
        xs = np.sort(x.astype(np.float64))
        # brute force: best split of the sorted data into 4 contiguous non-empty intervals
        pre = np.concatenate([[0], np.cumsum(xs)])
        pre2 = np.concatenate([[0], np.cumsum(xs * xs)])

        def sse(i, j):
            n = j - i
            s = pre[j] - pre[i]
            return pre2[j] - pre2[i] - s * s / n

        best = min(sse(0, a) + sse(a, b) + sse(b, c) + sse(c, 64)
                   for a, b, c in itertools.combinations(range(1, 64), 3))
        prev = np.inf
        for it in range(9):
            q = Q.quantize_rows(x[None, :], spec_it[it])
            d = Q.dequantize_rows(q, spec_it[it])[0]
            e = np.sum((d - x) ** 2)
            assert e >= best * (1 - 1e-3)   # fp16 centroids can sit a hair off the optimum
            assert e <= prev * (1 + 1e-3) + 1e-6
            prev = e
        cent = F.fp16_from_bits(q.meta.view(np.uint16).reshape(4))
        assert np.all(np.diff(cent) >= 0)


def test_c2_fit_excludes_outliers_and_codes_zero_at_outliers():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((500, 128)).astype(F32)
    x[:, 5] = 300.0
    x[:, 100] = -250.0
    spec = Q.QuantSpec("c2", 64, "e4m3")
    q = Q.quantize_rows(x, spec)
    assert q.mask[:, 5].all() and q.mask[:, 100].all()
    cent = F.fp16_from_bits(q.meta.view(np.uint16).reshape(500, 2, 4))
    assert np.abs(cent).max() < 10
    # outlier slots hold the code of 0.0 under the group's codebook
    for r in range(0, 500, 50):
        for c in (5, 100):
            gcent = cent[r, c // 64]
            assert q.codes[r, c] == int(np.argmin(np.abs(gcent)))
    d = Q.dequantize_rows(q, spec)
    assert np.all(d[:, 5] == 288.0) and np.all(d[:, 100] == -256.0)  # E4M3 of 300 / -250


def test_c2_scale_invariance():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((200, 128)).astype(F32)
    spec = Q.QuantSpec("c2", 64, "e4m3")
    q0 = Q.quantize_rows(x, spec)
    q1 = Q.quantize_rows((x * F32(4.0)).astype(F32), spec)
    assert np.array_equal(q0.codes, q1.codes) and np.array_equal(q0.mask, q1.mask)
    c0 = F.fp16_from_bits(q0.meta.view(np.uint16))
    c1 = F.fp16_from_bits(q1.meta.view(np.uint16))
    assert np.array_equal(c0 * 4, c1)


def test_int4_zero_minimum_is_positive_zero():
    x = np.zeros((1, 32), dtype=F32)
    x[0, 3] = -0.0
    x[0, 5] = 1.5
    q = Q.quantize_rows(x, Q.QuantSpec("int4", 32, "none"))
    z_bits = q.meta.view(np.uint16)[0, 1]
    assert z_bits == 0x0000


# ----------------------------------------------------------------------------- format variants
# Uniform 2-bit ([P1] listing: linspace(min, max, 4) of the residuals, argmin) and symmetric INT4
# ([P4] listing quantize_kv_cache_fp4: absmax / 7 clamped at 1e-5, round, clamp to [-8, 7]).
def test_u2_equally_spaced_values_are_exact():
    # values 0, 1, 2, 3 in any order: the linspace is exactly the 4 values, every code is its value
    rng = np.random.default_rng(21)
    x = rng.permutation(np.repeat(np.arange(4, dtype=F32), 16))[None, :].astype(F32)
    x = np.concatenate([x, x * F32(-0.5) + F32(10.0)], axis=1)   # second group: 10, 9.5, 9, 8.5
    spec = Q.QuantSpec("u2", 64, "none")
    q = Q.quantize_rows(x, spec)
    assert np.array_equal(q.codes[0, :64], x[0, :64].astype(np.uint8))
    assert np.array_equal(Q.dequantize_rows(q, spec)[0], x[0].astype(np.float64))
    cent = F.fp16_from_bits(q.meta.view(np.uint16).reshape(2, 4))
    assert cent[0].tolist() == [0.0, 1.0, 2.0, 3.0] and cent[1].tolist() == [8.5, 9.0, 9.5, 10.0]


def test_u2_ends_are_min_and_max_of_the_zero_filled_residuals():
    # the listing zero-fills outlier slots before taking min / max: with all non-outliers in
    # [1, 2] and one outlier, the low end is 0, not 1
    rng = np.random.default_rng(22)
    x = rng.uniform(1.0, 2.0, 64).astype(F32)
    x[17] = 500.0
    spec = Q.QuantSpec("u2", 64, "fp16", sigma=3.0)
    q = Q.quantize_rows(x[None, :], spec)
    assert q.mask[0].tolist() == [i == 17 for i in range(64)]
    cent = F.fp16_from_bits(q.meta.view(np.uint16).reshape(4))
    kept = x[~q.mask[0]]
    assert cent[0] == 0.0 and cent[3] == F.fp16_round(F32(kept.max()))
    # without outlier isolation the ends are the plain min and max
    q = Q.quantize_rows(x[None, :], Q.QuantSpec("u2", 64, "none"))
    cent = F.fp16_from_bits(q.meta.view(np.uint16).reshape(4))
    assert cent[0] == F.fp16_round(F32(x.min())) and cent[3] == F.fp16_round(F32(500.0))


def test_u2_centroids_match_torch_linspace():
    # library routine: the four uniform centroids are torch.linspace(min, max, 4) in float32 (the
    # listing's call), rounded to fp16.  Random (min, max) pairs over many magnitudes, both signs,
    # equal ends; each group holds its min and max and 62 values between them.
    import torch
    rng = np.random.default_rng(24)
    n = 4000
    a = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 4, n)).astype(F32)
    b = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 4, n)).astype(F32)
    mn, mx = np.minimum(a, b), np.maximum(a, b)
    mx[:50] = mn[:50]
    mid = (mn[:, None] + (mx - mn)[:, None] * rng.uniform(0, 1, (n, 62))).astype(F32)
    mid = np.clip(mid, mn[:, None], mx[:, None]).astype(F32)
    x = np.concatenate([mx[:, None], mid[:, :31], mn[:, None], mid[:, 31:]], axis=1).astype(F32)
    q = Q.quantize_rows(np.concatenate([x, x], axis=1), Q.QuantSpec("u2", 64, "none"))
    got = q.meta.view(np.uint16).reshape(n, 2, 4)[:, 0]
    ref = np.stack([torch.linspace(float(lo), float(hi), 4, dtype=torch.float32).numpy()
                    for lo, hi in zip(mn, mx)]).astype(F32)
    assert np.array_equal(got, F.fp16_bits(F.fp16_round(ref)))


def test_u2_codes_are_nearest_centroids():
    # invariant on random groups: each code's centroid is no farther than any other, and strictly
    # nearer than every lower index (first index on ties); interior points within fp16 rounding
    # of the exact thirds
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((40, 128)) * rng.uniform(0.01, 50, (40, 1))).astype(F32)
    spec = Q.QuantSpec("u2", 64, "none")
    q = Q.quantize_rows(x, spec)
    cent = F.fp16_from_bits(q.meta.view(np.uint16).reshape(40, 2, 4)).astype(np.float64)
    for r in range(40):
        for gi in range(2):
            c = cent[r, gi]
            lo, hi = float(x[r, 64 * gi:64 * gi + 64].min()), float(x[r, 64 * gi:64 * gi + 64].max())
            for k, frac in enumerate((0.0, 1 / 3, 2 / 3, 1.0)):
                assert abs(c[k] - (lo + frac * (hi - lo))) <= 2 ** -10 * max(abs(lo), abs(hi)) + 1e-30
            for j in range(64):
                v = float(x[r, 64 * gi + j])
                code = int(q.codes[r, 64 * gi + j])
                d = [abs(np.float32(v) - np.float32(ck)) for ck in c]
                assert all(d[code] <= dk for dk in d)
                assert all(d[code] < d[k] for k in range(code))


def test_int4s_integer_grid_and_ties_to_even():
    # absmax 7 gives S = 1: integers map to themselves (+8); halves round to even; -7.5 rounds
    # to -8 (kept), 7.5 would round to 8 and clamp, but absmax 7 keeps it out of the group
    g = np.array([-7, -6, -5, -4, -3, -2, -1, 0, 1, 2, 3, 4, 5, 6, 7, 0.5, 1.5, 2.5, -0.5, -1.5,
                  -2.5, 6.5, -6.5, 3.25, -3.75, 0, 0, 0, 0, 0, 0, 0], dtype=F32)
    x = np.tile(g, 4)[None, :]
    spec = Q.QuantSpec("int4s", 32, "none")
    q = Q.quantize_rows(x, spec)
    want = np.array([-7, -6, -5, -4, -3, -2, -1, 0, 1, 2, 3, 4, 5, 6, 7, 0, 2, 2, 0, -2, -2, 6, -6,
                     3, -4, 0, 0, 0, 0, 0, 0, 0]) + 8
    assert np.array_equal(q.codes[0], np.tile(want, 4))
    sz = F.fp16_from_bits(q.meta.view(np.uint16).reshape(4, 2))
    assert sz[:, 0].tolist() == [1.0] * 4 and sz[:, 1].tolist() == [-8.0] * 4
    assert np.array_equal(Q.dequantize_rows(q, spec)[0], np.tile(want - 8, 4).astype(np.float64))


def test_int4s_clamp_and_bounds():
    rng = np.random.default_rng(24)
    spec = Q.QuantSpec("int4s", 64, "none")
    # all-zero group: the scale clamps at 1e-5 (as fp16), every code is 8, the value 0
    q = Q.quantize_rows(np.zeros((1, 128), F32), spec)
    sz = F.fp16_from_bits(q.meta.view(np.uint16).reshape(2, 2))
    assert sz[0, 0] == F.fp16_round(F32(1e-5)) and np.all(q.codes == 8)
    assert not Q.dequantize_rows(q, spec).any()
    # random groups: the absmax element maps to +-7, every value is within S/2 of its
    # reconstruction, and the codes of -x are 16 - codes of x
    x = (rng.standard_normal((30, 128)) * rng.uniform(0.1, 100, (30, 1))).astype(F32)
    q, qn = Q.quantize_rows(x, spec), Q.quantize_rows(-x, spec)
    S = F.fp16_from_bits(q.meta.view(np.uint16).reshape(30, 2, 2))[..., 0].astype(np.float64)
    d = Q.dequantize_rows(q, spec)
    for r in range(30):
        for gi in range(2):
            seg = slice(64 * gi, 64 * gi + 64)
            a = np.argmax(np.abs(x[r, seg]))
            assert abs(int(q.codes[r, seg][a]) - 8) == 7
            assert np.all(np.abs(d[r, seg] - x[r, seg]) <= S[r, gi] / 2 * (1 + 2 ** -20))
    assert np.array_equal(qn.codes.astype(int), 16 - q.codes.astype(int))


# ----------------------------------------------------------------------------- channel mask
# [P4] "Key Production Engineering Takeaways" item 2: a static mask of the top channels by
# absolute magnitude kept at high precision.
def test_channel_mask_records_exactly_the_masked_channels():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((20, 128)).astype(F32)
    x[:, 77] *= 300.0
    for fmt, g, out in [("int4", 32, "fp16"), ("c2", 64, "fp16"), ("fp4", 32, "e4m3")]:
        spec = Q.QuantSpec(fmt, g, out, channels=(3, 77))
        q = Q.quantize_rows(x, spec)
        assert np.array_equal(np.nonzero(q.mask.any(axis=0))[0], [3, 77]) and q.mask[:, [3, 77]].all()
        d = Q.dequantize_rows(q, spec)
        want = F.fp16_round(x[:, [3, 77]]) if out == "fp16" else F.e4m3_decode(F.e4m3_encode(x[:, [3, 77]]))
        assert np.array_equal(d[:, [3, 77]], want.astype(np.float64))
        # the fit ignores the masked channels: other values there change no other code or metadata
        y = x.copy()
        y[:, [3, 77]] = rng.standard_normal((20, 2)).astype(F32) * 1e4
        qy = Q.quantize_rows(y, spec)
        keep = np.ones(128, bool)
        keep[[3, 77]] = False
        assert np.array_equal(qy.codes[:, keep], q.codes[:, keep]) and np.array_equal(qy.meta, q.meta)


def test_top_channels_finds_the_scaled_channels():
    from workloads import CONFIGS
    from workloads import generate as G
    w = CONFIGS["int4_b1_s1k"]   # 4 channels per (KV head, K or V) scaled x20
    for h in range(w.H):
        for kind in (G.K, G.V):
            heavy = tuple(int(c) for c in np.nonzero(G._head_constants(w, h, kind) == 20.0)[0])
            assert Q.top_channels(G.kv_rows(w, 0, h, kind, 0, 256), 4) == heavy
    # ties go to the lower channels; k larger than the distinct maxima
    z = np.ones((4, 128), F32)
    z[:, 9] = 2.0
    assert Q.top_channels(z, 3) == (0, 1, 9)


def test_calibrated_mask_matches_top_channels():
    # the workloads' calibration (what a caller does once) picks the oracle's top channels
    from workloads import CONFIGS
    from workloads import device as WD
    from workloads import generate as G
    for name, k in [("int4_b1_s1k", 4), ("c2_b64_s32k", 2)]:
        w = WD.variant(CONFIGS[name], chan_mask=k)
        for h in range(min(w.H, 3)):
            for kind in (G.K, G.V):
                assert G.mask_channels(w, h, kind) == Q.top_channels(G.kv_rows(w, 0, h, kind, 0, 256), k)


# ----------------------------------------------------------------------------- INT3
# [P3] "Sub-Byte KV-Cache Quantization": asymmetric 3-bit packed codes.
def test_int3_packing_is_one_little_endian_bit_stream():
    codes = np.array([1, 2, 3, 4, 5, 6, 7, 0] * 16, dtype=np.uint8)
    packed = Q.pack_codes(codes[None, :], 3)[0]
    assert packed.shape == (48,)
    stream = sum(int(c) << (3 * i) for i, c in enumerate(codes))       # channel i at bit 3 i
    assert bytes(packed) == stream.to_bytes(48, "little")
    assert list(packed[:3]) == [0xD1, 0x58, 0x1F]
    rng = np.random.default_rng(41)
    c = rng.integers(0, 8, (5, 128)).astype(np.uint8)
    assert np.array_equal(Q.unpack_codes(Q.pack_codes(c, 3), 3, 128), c)


def test_int3_grid_and_bound():
    # min 0, max 7: S = 1, zero = 0, every integer is its own code
    x = np.tile(np.arange(8, dtype=F32), 16)[None, :]
    spec = Q.QuantSpec("int3", 32, "none")
    q = Q.quantize_rows(x, spec)
    assert np.array_equal(q.codes[0], x[0].astype(np.uint8))
    sz = F.fp16_from_bits(q.meta.view(np.uint16).reshape(4, 2))
    assert sz[:, 0].tolist() == [1.0] * 4 and sz[:, 1].tolist() == [0.0] * 4
    # random groups: reconstruction within half a step (plus the fp16 rounding of S and zero)
    rng = np.random.default_rng(42)
    x = (rng.standard_normal((20, 128)) * rng.uniform(0.1, 10, (20, 1))).astype(F32)
    for g in (32, 64):
        spec = Q.QuantSpec("int3", g, "none")
        q = Q.quantize_rows(x, spec)
        d = Q.dequantize_rows(q, spec)
        S = F.fp16_from_bits(q.meta.view(np.uint16).reshape(20, 128 // g, 2))[..., 0]
        lim = np.repeat(S, g, axis=1) * 0.5 + np.abs(x) * 2.0 ** -10 + 1e-6
        assert np.all(np.abs(d - x) <= lim) and q.codes.max() <= 7


def test_int_fits_beyond_the_fp16_range_give_code_zero():
    # min -1e6, max 1e6: S and zero both round to +-inf in fp16, every quotient is inf / inf;
    # the codes are 0 (no value is taken as the bottom of the clamp range), never an
    # out-of-range integer
    x = np.where(np.arange(128) % 2 == 0, 1e6, -1e6).astype(F32)[None, :]
    for fmt in ("int4", "int3"):
        q = Q.quantize_rows(x, Q.QuantSpec(fmt, 32, "none"))
        assert not q.codes.any()
