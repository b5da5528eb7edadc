"""GPU regression tests of the list truncation that starts every append at a position p > 0:
the records of tokens < p are kept, the others are dropped before the new rows' records are
written.  The 16-token block before p can hold far more records than a tau = 3 workload ever
produces: with tau = 1.3 (about 20 records per 128-channel row, about 310 per block) and with a
32-channel static mask (512 records per block).  Both are built through appends that start
inside a list (a second fill call at token 2048, then a one-token re-append of the last token
as a decode step does), compared bit for bit with the oracle, and decoded within 2e-3."""

import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import decode_attention_sub_amd as K  # noqa: E402
from oracle import cache as OC  # noqa: E402
from oracle import quantize as OQ  # noqa: E402
from workloads import CONFIGS  # noqa: E402
from workloads import device as WD  # noqa: E402
from workloads import generate as G  # noqa: E402

from gpu_util import (ATOL, assert_list_equal, log, oracle_attention, read_list,  # noqa: E402
                      run_decode)


def _append(p, cache, rows_k, rows_v, pos, counts):
    """rows_*: float32 [B, H, n, D] host arrays; pos, counts: per-sequence ints."""
    B = rows_k.shape[0]
    K.kvq_quantize_append(p, cache, torch.from_numpy(np.ascontiguousarray(rows_k)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(rows_v)).cuda(),
                          torch.tensor(pos, dtype=torch.int32, device="cuda"),
                          torch.tensor(counts, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert cache.status() == 0, K.kvq_status_string(cache.status())
    assert B == len(pos)


def _reappend_last(w, p, cache, S):
    """Replace token S - 1 of every list by a fresh row (the bench's decode-step append)."""
    nk = np.stack([[G.new_rows(w, b, h, G.NEW_K, 0) for h in range(w.H)] for b in range(w.B)])
    nv = np.stack([[G.new_rows(w, b, h, G.NEW_V, 0) for h in range(w.H)] for b in range(w.B)])
    _append(p, cache, nk, nv, [S - 1] * w.B, [1] * w.B)
    return nk, nv


def _check_decode(dc, what):
    w = dc.w
    sm = 1.0 / math.sqrt(w.D)
    for split in (0, 512):
        log(f"[gpu] truncation decode {what} split={split}")
        got = run_decode(dc, split_chunk=split, sm_scale=sm)
        for b in range(w.B):
            for hq, o in oracle_attention(dc, b, range(w.Hq), sm).items():
                err = np.abs(got[b, hq] - o).max()
                assert err <= ATOL, f"{what} b={b} hq={hq} split={split}: max-abs {err}"


def test_dense_outliers_across_fill_chunks():
    """tau = 1.3 on the spiky 2-bit data: the second fill call starts at token 2048 inside the
    list, then the last token is re-appended."""
    w = WD.variant(CONFIGS["c2_b16_s8k"], B=2, H=2, Hq=8, S=2100, sigma=1.3)
    log(f"[gpu] truncation: building {w}")
    dc = WD.build(w)
    assert dc.cache.status() == 0
    spec = OQ.QuantSpec(w.fmt, w.group, w.outlier, w.sigma, w.lloyd_iters)
    rows = {(b, h, kv): G.kv_rows(w, b, h, kv, 0, w.S)
            for b in range(w.B) for h in range(w.H) for kv in (0, 1)}
    per_block = min(OC.build_list(x[2032:2048], spec).count for x in rows.values())
    assert per_block > 256, f"a block before the second fill holds only {per_block} records"
    for (b, h, kv), x in rows.items():
        assert_list_equal(read_list(dc, b, h, kv), OC.build_list(x, spec), f"fill b={b} h={h} kv={kv}")
    nk, nv = _reappend_last(w, dc.params, dc.cache, w.S)
    for (b, h, kv), x in rows.items():
        new = (nk if kv == 0 else nv)[b, h]
        ref = OC.build_list(np.concatenate([x[:w.S - 1], new]), spec)
        assert_list_equal(read_list(dc, b, h, kv), ref, f"re-append b={b} h={h} kv={kv}")
    _check_decode(dc, "c2 tau=1.3")


def test_wide_channel_mask_across_fill_chunks():
    """A 32-channel static mask on INT4 rows (512 records per 16-token block), appended in two
    calls (tokens 0..2047, then 2048..2099) and re-appended at the last token."""
    w = WD.variant(CONFIGS["int4_b1_s1k"], B=1, H=2, Hq=8, S=2100)
    chans = tuple(range(1, 128, 4))
    S_cap = w.S
    p = WD.make_params(w, S_cap)
    words = np.zeros((2, w.H, 4), dtype=np.uint32)
    for c in chans:
        words[:, :, c // 32] |= np.uint32(1) << np.uint32(c % 32)
    mask = torch.from_numpy(words.view(np.int32)).cuda()
    cache = K.KVCache.allocate(p, len(chans) * S_cap, chan_mask=mask)
    rows = {(b, h, kv): G.kv_rows(w, b, h, kv, 0, w.S)
            for b in range(w.B) for h in range(w.H) for kv in (0, 1)}

    def stack(kv, t0, t1):
        return np.stack([[rows[(b, h, kv)][t0:t1] for h in range(w.H)] for b in range(w.B)])

    log("[gpu] truncation: 32-channel mask, two fill calls")
    for t0, t1 in ((0, 2048), (2048, w.S)):
        _append(p, cache, stack(0, t0, t1), stack(1, t0, t1), [t0] * w.B, [t1 - t0] * w.B)
    lens = np.full(w.B, w.S, dtype=np.int32)
    q_host = np.stack([G.queries(w, b) for b in range(w.B)])
    q = torch.from_numpy(q_host.view(np.int16)).cuda().view(torch.bfloat16)
    dc = WD.DeviceCache(w, p, cache, lens, torch.from_numpy(lens).cuda(), None, None, q_host, q)
    spec = OQ.QuantSpec(w.fmt, w.group, w.outlier, w.sigma, w.lloyd_iters, channels=chans)
    for (b, h, kv), x in rows.items():
        assert_list_equal(read_list(dc, b, h, kv), OC.build_list(x, spec), f"fill b={b} h={h} kv={kv}")
    nk, nv = _reappend_last(w, p, cache, w.S)
    for (b, h, kv), x in rows.items():
        new = (nk if kv == 0 else nv)[b, h]
        ref = OC.build_list(np.concatenate([x[:w.S - 1], new]), spec)
        assert ref.count == len(chans) * w.S
        assert_list_equal(read_list(dc, b, h, kv), ref, f"re-append b={b} h={h} kv={kv}")
    _check_decode(dc, "int4 32-channel mask")
