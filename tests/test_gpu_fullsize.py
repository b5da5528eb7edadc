"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times (the
workload's own split, default softmax scale) and split into one workgroup per 2048 tokens: the whole cache is built on the device,
then sampled (sequence, KV head) pairs are checked against the oracle - the packed rows and
outlier records of the first and last tokens of each sampled list bit for bit, and the decode
output of every query head of the pair within the 2e-3 max-abs bar."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch  # noqa: F401  (device memory for the cache)

from workloads import CONFIGS
from workloads import device as WD
from workloads import generate as G

from gpu_util import ATOL, log, oracle_attention, page_tiers_of, read_list, run_decode, specs
from oracle import cache as OC

pytestmark = pytest.mark.gpu

EDGE = 160   # tokens checked bit for bit at each end of a sampled list (multiple of 16)


def check_rows(dc, b, h, kv, ta, tb, dev):
    """Device rows [ta, tb) of list (b, h, kv) and their outlier records == the oracle's."""
    w = dc.w
    spec, spec8 = specs(w, h, kv)
    x = G.kv_rows(w, b, h, kv, ta, tb)
    tiers = page_tiers_of(dc, b)
    tp = None if tiers is None else tiers[ta // 16:(tb + 15) // 16]
    ref = OC.build_list(x, spec, tp, spec8)
    what = f"{w.name} b={b} h={h} kv={kv} rows {ta}..{tb}"
    if dev["tier1"] is None:
        assert np.array_equal(dev["packed"][ta:tb], ref.packed), what + ": codes"
        assert np.array_equal(dev["meta"][ta:tb], ref.meta), what + ": metadata"
    else:
        t1 = dev["tier1"][ta:tb]
        t2 = ~t1
        assert np.array_equal(dev["packed"][ta:tb][t2], ref.packed[t2]), what + ": tier-2 codes"
        assert np.array_equal(dev["meta"][ta:tb][t2], ref.meta[t2]), what + ": tier-2 metadata"
        assert np.array_equal(dev["packed8"][ta:tb][t1], ref.packed8[t1]), what + ": FP8 codes"
        assert np.array_equal(dev["meta8"][ta:tb][t1], ref.meta8[t1]), what + ": FP8 scales"
    tok = dev["idx"].astype(np.int64) >> 7
    sel = (tok >= ta) & (tok < tb)
    assert np.array_equal(dev["idx"][sel].astype(np.int64) - ta * w.D, ref.idx.astype(np.int64)), \
        what + ": outlier indices"
    assert np.array_equal(dev["vals"][sel], ref.vals), what + ": outlier values"


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_full_size_sampled(name):
    w = CONFIGS[name]
    log(f"[gpu] full-size {name}: building the cache")
    dc = WD.build(w)
    assert dc.cache.status() == 0
    log(f"[gpu] full-size {name}: decode with split {w.split_chunk or 'default'}")
    got = run_decode(dc, split_chunk=w.split_chunk)
    assert np.all(np.isfinite(got))
    # the same decode split into one workgroup per 2048 tokens of all lists (many more cut lists)
    log(f"[gpu] full-size {name}: decode with split 2048")
    got2 = run_decode(dc, split_chunk=2048)
    rng = np.random.default_rng(1234)
    lens = dc.seq_lens_host
    pairs = {(int(np.argmax(lens)), int(rng.integers(w.H))), (int(rng.integers(w.B)), int(rng.integers(w.H)))}
    sm = 1.0 / math.sqrt(w.D)
    G_ = w.Hq // w.H
    for b, h in sorted(pairs):
        S = int(lens[b])
        for kv in (0, 1):
            dev = read_list(dc, b, h, kv)
            check_rows(dc, b, h, kv, 0, min(EDGE, S), dev)
            tail = max(0, (S - EDGE) // 16 * 16)
            check_rows(dc, b, h, kv, tail, S, dev)
        log(f"[gpu] full-size {name}: oracle attention b={b} h={h} S={S}")
        ref = oracle_attention(dc, b, range(h * G_, (h + 1) * G_), sm)
        for hq, o in ref.items():
            err = np.abs(got[b, hq] - o).max()
            assert err <= ATOL, f"{name} b={b} hq={hq}: max-abs {err}"
            err2 = np.abs(got2[b, hq] - o).max()
            assert err2 <= ATOL, f"{name} b={b} hq={hq} split 2048: max-abs {err2}"
