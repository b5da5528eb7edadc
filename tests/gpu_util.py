"""Helpers for the GPU parity tests: read one list of a device cache back to the host, build the
oracle's version of the same list from the same seeded rows, compare bit-exactly, and compute
the oracle's float64 attention over the device cache's own bytes."""

from __future__ import annotations

import sys

import numpy as np
import torch

import decode_attention_sub_amd as K
from oracle import attention as OA
from oracle import cache as OC
from oracle import quantize as OQ
from workloads import generate as G
from workloads.device import read_list  # noqa: F401

ATOL = 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def specs(w, h: int = 0, kv: int = 0):
    """Oracle specs of list (h, kv) of workload w (a static channel mask differs per list)."""
    chans = G.mask_channels(w, h, kv) if w.chan_mask else ()
    spec = OQ.QuantSpec(w.fmt, w.group, w.outlier, w.sigma, w.lloyd_iters, channels=chans)
    spec8 = OQ.QuantSpec("fp8row", 0, "none") if w.paged else None
    return spec, spec8


def oracle_list(w, b: int, h: int, kv: int, S: int, tier1_pages=None):
    x = G.kv_rows(w, b, h, kv, 0, S)
    spec, spec8 = specs(w, h, kv)
    return OC.build_list(x, spec, tier1_pages, spec8)


def assert_list_equal(got, ref, what=""):
    tier1 = got["tier1"]
    if tier1 is None:
        assert np.array_equal(got["packed"], ref.packed), f"{what}: packed codes differ"
        assert np.array_equal(got["meta"], ref.meta), f"{what}: metadata differs"
    else:
        t2 = ~tier1
        assert np.array_equal(got["packed"][t2], ref.packed[t2]), f"{what}: tier-2 codes differ"
        assert np.array_equal(got["meta"][t2], ref.meta[t2]), f"{what}: tier-2 metadata differs"
        assert np.array_equal(got["packed8"][tier1], ref.packed8[tier1]), f"{what}: FP8 codes differ"
        assert np.array_equal(got["meta8"][tier1], ref.meta8[tier1]), f"{what}: FP8 scales differ"
    assert got["count"] == ref.count, f"{what}: outlier count {got['count']} != {ref.count}"
    assert np.array_equal(got["idx"], ref.idx), f"{what}: outlier indices differ"
    assert np.array_equal(got["vals"], ref.vals), f"{what}: outlier values differ"
    assert np.array_equal(got["block_start"], ref.block_start), f"{what}: block starts differ"


def page_tiers_of(dc, b):
    if not dc.w.paged:
        return None
    S = int(dc.seq_lens_host[b])
    ent = dc.block_table_host[b].view(np.uint32)[: (S + 15) // 16]
    return (ent >> 31) == 1


def dequant_from_device(dc, b: int, h: int):
    """float64 K, V [S, D] of (b, h) decoded by the oracle from the device cache bytes."""
    w = dc.w
    res = []
    for kv in (0, 1):
        spec, spec8 = specs(w, h, kv)
        g = read_list(dc, b, h, kv)
        codes = OQ.unpack_codes(g["packed"], OQ.CODE_BITS[w.fmt], w.D)
        codes8 = g.get("packed8")
        res.append(OC.dequantize_list(codes, g["meta"], g["idx"], g["vals"], spec, w.D,
                                      g["tier1"], codes8, g.get("meta8"), spec8))
    return res


def oracle_attention(dc, b: int, hqs, sm_scale):
    w = dc.w
    out = {}
    by_kv = {}
    for hq in hqs:
        by_kv.setdefault(OA.gqa_kv_head(hq, w.Hq, w.H), []).append(hq)
    for h, heads in by_kv.items():
        Kd, Vd = dequant_from_device(dc, b, h)
        qf = OA.bf16_to_f64(dc.q_host[b])
        for hq in heads:
            out[hq] = OA.attention_one(qf[hq], Kd, Vd, sm_scale)
    return out


def run_decode(dc, split_chunk=0, sm_scale=None):
    w, p = dc.w, dc.params
    ws = K.kvq_workspace_bytes(p, split_chunk)
    work = torch.empty(max(ws // 4, 1), dtype=torch.float32, device="cuda") if ws else None
    out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device="cuda")
    K.kvq_decode_attention(p, dc.cache, dc.q, dc.seq_lens, out, work, dc.block_table,
                           sm_scale=sm_scale, split_chunk=split_chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy()
