"""GPU parity: the HIP quantize-append kernel against the oracle bit for bit (codes, metadata,
outlier lists, block starts), and the HIP decode attention against the oracle's float64
attention on the same dequantized values (max-abs <= 2e-3), at sizes the oracle finishes in
seconds that still span several 64-token steps, several split-K chunks and a ragged tail."""

import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from workloads import CONFIGS  # noqa: E402
from workloads import device as WD  # noqa: E402

from gpu_util import (ATOL, assert_list_equal, log, oracle_attention, oracle_list,  # noqa: E402
                      page_tiers_of, read_list, run_decode)

SMALL = {
    # INT4 g32 + fp16 outliers with the x20 channels, GQA 4, ragged S
    "int4_small": WD.variant(CONFIGS["int4_b1_s1k"], B=2, S=777),
    # 2-bit g64 + E4M3 outliers with Laplace spikes, GQA 4
    "c2_small": WD.variant(CONFIGS["c2_b16_s8k"], B=2, H=2, Hq=8, S=1000),
    # 2-bit, LogNormal key channels, GQA 8
    "c2_g8_small": WD.variant(CONFIGS["c2_b64_s32k"], B=2, H=2, Hq=16, S=1100),
    # FP4 g32 + fp16 outliers, GQA 8
    "fp4_small": WD.variant(CONFIGS["fp4_b4_s128k"], B=2, H=2, Hq=16, S=3000),
    # FP4 with groups of 64 and INT4 with groups of 64 (generic kernel)
    "fp4_g64_small": WD.variant(CONFIGS["fp4_b4_s128k"], B=1, H=2, Hq=8, S=900, group=64),
    "int4_g64_small": WD.variant(CONFIGS["int4_b1_s1k"], B=1, S=500, group=64),
    # 2-bit with GQA 16 (every MFMA row used) and with MHA (one row)
    "c2_g16_small": WD.variant(CONFIGS["c2_b64_s32k"], B=1, H=1, Hq=16, S=1500),
    "c2_mha_small": WD.variant(CONFIGS["c2_b16_s8k"], B=2, H=3, Hq=3, S=333),
    # tau = 1.5: crowded steps with more than 128 records per list (the kernel's slow path)
    "c2_dense_outliers": WD.variant(CONFIGS["c2_b16_s8k"], B=1, H=2, Hq=8, S=700, sigma=1.5),
    "fp4_dense_outliers": WD.variant(CONFIGS["fp4_b4_s128k"], B=1, H=1, Hq=8, S=650, sigma=1.5),
    # format variants on the same kernels: uniform 2-bit codebook (stored as 2-bit centroids,
    # MFMA decoder) and symmetric INT4 (stored as INT4, generic decoder), with and without
    # outlier lists
    "u2_small": WD.variant(CONFIGS["c2_b16_s8k"], B=2, H=2, Hq=8, S=900, fmt="u2"),
    "int4s_small": WD.variant(CONFIGS["int4_b1_s1k"], B=2, S=650, fmt="int4s"),
    "int4s_g64_noout": WD.variant(CONFIGS["int4_b1_s1k"], B=1, H=2, Hq=4, S=300, fmt="int4s",
                                  group=64, outlier="none"),
    # asymmetric 3-bit codes packed as one bit stream (generic decoder), groups of 32 and 64
    "int3_small": WD.variant(CONFIGS["int4_b1_s1k"], B=2, S=600, fmt="int3"),
    "int3_g64_e4m3": WD.variant(CONFIGS["int4_b1_s1k"], B=1, H=2, Hq=8, S=333, fmt="int3",
                                group=64, outlier="e4m3"),
    # static channel mask (top channels by magnitude kept as fp16 records in every row): INT4 on
    # the data with 4 channels x20 per list, 2-bit on the LogNormal-channel keys
    "int4_chanmask": WD.variant(CONFIGS["int4_b1_s1k"], B=2, S=600, chan_mask=4),
    "c2_chanmask": WD.variant(CONFIGS["c2_b64_s32k"], B=2, H=2, Hq=16, S=700, chan_mask=2,
                              outlier="fp16"),
    "int3_chanmask": WD.variant(CONFIGS["int4_b1_s1k"], B=1, S=400, fmt="int3", chan_mask=4),
    # tiered paged cache, variable lengths
    "tiered_small": WD.variant(CONFIGS["tiered_b32_paged"], B=3, H=2, Hq=8, S=3000,
                               S_range=(90, 3000), fp8_page_frac=0.3),
    # tiered paged cache with GQA 16 and mostly FP8 pages
    "tiered_g16_small": WD.variant(CONFIGS["tiered_b32_paged"], B=2, H=1, Hq=16, S=1500,
                                   S_range=(40, 1500), fp8_page_frac=0.7),
}


@pytest.fixture(scope="module", params=sorted(SMALL))
def small(request):
    w = SMALL[request.param]
    log(f"[gpu] building {request.param} {w}")
    dc = WD.build(w)
    assert dc.cache.status() == 0
    return request.param, dc


def test_quantize_bit_exact(small):
    name, dc = small
    w = dc.w
    for b in range(w.B):
        for h in range(w.H):
            for kv in (0, 1):
                S = int(dc.seq_lens_host[b])
                got = read_list(dc, b, h, kv)
                ref = oracle_list(w, b, h, kv, S, page_tiers_of(dc, b))
                assert_list_equal(got, ref, f"{name} b={b} h={h} kv={kv}")


@pytest.mark.parametrize("split", [0, 128, 512, 16384])
def test_decode_matches_oracle(small, split):
    name, dc = small
    w = dc.w
    if dc.w.paged and split == 0:
        split = 256
    log(f"[gpu] decode {name} split={split}")
    sm = 1.0 / math.sqrt(w.D)
    got = run_decode(dc, split_chunk=split, sm_scale=sm)
    for b in range(w.B):
        ref = oracle_attention(dc, b, range(w.Hq), sm)
        for hq, o in ref.items():
            err = np.abs(got[b, hq] - o).max()
            assert err <= ATOL, f"{name} b={b} hq={hq} split={split}: max-abs {err}"


@pytest.mark.parametrize("sm", [-0.07, 0.0, 0.4])
def test_decode_softmax_scale(sm):
    """Negative, zero and large softmax scales (the kernel folds the sign into the queries)."""
    for name in ("c2_small", "c2_g16_small", "fp4_small"):
        w = SMALL[name]
        log(f"[gpu] decode {name} sm_scale={sm}")
        dc = WD.build(w)
        got = run_decode(dc, split_chunk=0, sm_scale=sm)
        for b in range(w.B):
            ref = oracle_attention(dc, b, range(w.Hq), sm)
            for hq, o in ref.items():
                err = np.abs(got[b, hq] - o).max()
                assert err <= ATOL, f"{name} b={b} hq={hq} sm={sm}: max-abs {err}"


def test_decode_deterministic(small):
    name, dc = small
    a = run_decode(dc, split_chunk=256)
    b = run_decode(dc, split_chunk=256)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["c2_small", "fp4_small", "tiered_small", "int4_small", "int3_small"])
def test_decode_workspace_contents_do_not_matter(name):
    """Lists cut between workgroups are merged by the last workgroup to finish a part (MFMA
    decoder), counted on arrival words in the workspace that carry a per-call tag; split-K chunks
    of the generic decoder are merged by a second kernel: whatever the workspace holds (random
    bytes, or the words of earlier calls with another split), the result is the same, bit for
    bit."""
    import decode_attention_sub_amd as K
    w = SMALL[name]
    dc = WD.build(w)
    p = dc.params
    ref = run_decode(dc, split_chunk=256)
    nbytes = max(K.kvq_workspace_bytes(p, s) for s in (0, 128, 256))
    work = torch.empty(nbytes // 4 + 1, dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(7)

    def decode(split):
        out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device="cuda")
        K.kvq_decode_attention(p, dc.cache, dc.q, dc.seq_lens, out, work, dc.block_table,
                               split_chunk=split)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    work.random_(generator=gen)                      # random bytes
    assert np.array_equal(decode(256), ref)
    assert np.array_equal(decode(256), ref)          # the words of the call before
    decode(128)                                      # other splits leave other words
    decode(0)
    assert np.array_equal(decode(256), ref)
    assert dc.cache.status() == 0


def test_bulk_equals_incremental():
    """Appending S tokens in one call equals S one-token appends, bit for bit."""
    import decode_attention_sub_amd as K
    from workloads import generate as G
    w = WD.variant(CONFIGS["c2_b16_s8k"], B=2, H=2, Hq=8, S=70)
    bulk = WD.build(w)
    p = bulk.params
    inc = K.KVCache.allocate(p, bulk.cache.outl_capacity)
    for t in range(w.S):
        k = np.stack([[G.kv_rows(w, b, h, 0, t, t + 1) for h in range(w.H)] for b in range(w.B)])
        v = np.stack([[G.kv_rows(w, b, h, 1, t, t + 1) for h in range(w.H)] for b in range(w.B)])
        pos = torch.full((w.B,), t, dtype=torch.int32, device="cuda")
        cnt = torch.ones(w.B, dtype=torch.int32, device="cuda")
        K.kvq_quantize_append(p, inc, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                              pos, cnt)
    torch.cuda.synchronize()
    for key in ("codes0", "codes1", "meta0", "meta1", "count", "bstart"):
        assert torch.equal(bulk.cache.tensors[key], inc.tensors[key]), key
    dci = WD.DeviceCache(w, p, inc, bulk.seq_lens_host, bulk.seq_lens, None, None, bulk.q_host,
                         bulk.q)
    for b in range(w.B):
        for h in range(w.H):
            for kv in (0, 1):
                g1, g2 = read_list(bulk, b, h, kv), read_list(dci, b, h, kv)
                assert np.array_equal(g1["idx"], g2["idx"]) and np.array_equal(g1["vals"], g2["vals"])


def test_reappend_truncates_lists():
    """Re-appending from position p replaces tokens >= p: lists end up as if built directly."""
    import decode_attention_sub_amd as K
    from workloads import generate as G
    w = WD.variant(CONFIGS["c2_b16_s8k"], B=2, H=2, Hq=8, S=200)
    dc = WD.build(w)
    p = dc.params
    # overwrite tokens 150..199 with the values of tokens 37..86 of another sequence
    t0, n = 150, 50
    k = np.stack([[G.kv_rows(w, 1 - b, h, 0, 37, 37 + n) for h in range(w.H)] for b in range(w.B)])
    v = np.stack([[G.kv_rows(w, 1 - b, h, 1, 37, 37 + n) for h in range(w.H)] for b in range(w.B)])
    pos = torch.full((w.B,), t0, dtype=torch.int32, device="cuda")
    cnt = torch.full((w.B,), n, dtype=torch.int32, device="cuda")
    K.kvq_quantize_append(p, dc.cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), pos, cnt)
    torch.cuda.synchronize()
    from oracle import cache as OC
    from gpu_util import specs
    spec, _ = specs(w)
    for b in range(w.B):
        for h in range(w.H):
            for kv in (0, 1):
                x = np.concatenate([G.kv_rows(w, b, h, kv, 0, t0), G.kv_rows(w, 1 - b, h, kv, 37, 37 + n)])
                ref = OC.build_list(x, spec)
                assert_list_equal(read_list(dc, b, h, kv), ref, f"b={b} h={h} kv={kv}")


def test_capacity_overflow_reports_status():
    """A tiny outlier capacity makes the kernel drop records and report KVQ_ERR_CAPACITY."""
    import decode_attention_sub_amd as K
    from workloads import generate as G
    w = WD.variant(CONFIGS["c2_b16_s8k"], B=1, H=1, Hq=4, S=300)
    p = WD.make_params(w, w.S)
    cache = K.KVCache.allocate(p, 3)
    k = torch.from_numpy(G.kv_rows(w, 0, 0, 0, 0, w.S)[None, None]).cuda()
    v = torch.from_numpy(G.kv_rows(w, 0, 0, 1, 0, w.S)[None, None]).cuda()
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    cnt = torch.full((1,), w.S, dtype=torch.int32, device="cuda")
    K.kvq_quantize_append(p, cache, k, v, zero, cnt)
    torch.cuda.synchronize()
    assert cache.status() == K.KVQ_ERR_CAPACITY
    assert int(cache.tensors["count"][0].item()) == 3


def test_out_of_range_position_reports_status():
    import decode_attention_sub_amd as K
    w = WD.variant(CONFIGS["c2_b16_s8k"], B=1, H=1, Hq=4, S=64)
    p = WD.make_params(w, 64)
    cache = K.KVCache.allocate(p, 100)
    k = torch.zeros((1, 1, 8, 128), dtype=torch.float32, device="cuda")
    pos = torch.full((1,), 60, dtype=torch.int32, device="cuda")
    cnt = torch.full((1,), 8, dtype=torch.int32, device="cuda")
    K.kvq_quantize_append(p, cache, k, k, pos, cnt)
    torch.cuda.synchronize()
    assert cache.status() == K.KVQ_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["c2_g8_small", "int4_g64_small", "tiered_small"])
def test_invalid_seq_len_reports_status(name):
    """A sequence length of 0 or past the capacity is reported through the status word; that
    sequence is skipped and every other sequence's output is the one of a valid call, up to the
    order of float32 sums (the MFMA decoder shares the steps of all valid lists among its
    workgroups, so the points where lists are cut depend on every length)."""
    import dataclasses
    import decode_attention_sub_amd as K
    w = SMALL[name]
    dc = WD.build(w)
    S_cap = dc.params.max_seq_len
    for split in (0, 128):
        good = run_decode(dc, split_chunk=split)
        assert dc.cache.status() == 0
        for bad in (0, S_cap + 1):
            lens = dc.seq_lens_host.copy()
            lens[0] = bad
            dcb = dataclasses.replace(dc, seq_lens_host=lens, seq_lens=torch.from_numpy(lens).cuda())
            log(f"[gpu] decode {name} with seq_len {bad} split={split}")
            got = run_decode(dcb, split_chunk=split)
            assert dc.cache.status() == K.KVQ_ERR_INVALID_ARG
            dc.cache.tensors["status"].zero_()
            assert np.isnan(got[0]).all(), "the rejected sequence's output was written"
            assert np.allclose(got[1:], good[1:], rtol=1e-4, atol=1e-5)


def test_zero_count_append_leaves_sequence_untouched():
    """counts[b] = 0 appends nothing to sequence b (codes, metadata, lists, block starts)."""
    import decode_attention_sub_amd as K
    from workloads import generate as G
    w = WD.variant(CONFIGS["c2_b16_s8k"], B=2, H=2, Hq=8, S=100)
    dc = WD.build(w)
    p = dc.params
    before = {k: t.clone() for k, t in dc.cache.tensors.items() if t is not None}
    n = 20
    k = np.stack([[G.kv_rows(w, 1 - b, h, 0, 0, n) for h in range(w.H)] for b in range(w.B)])
    v = np.stack([[G.kv_rows(w, 1 - b, h, 1, 0, n) for h in range(w.H)] for b in range(w.B)])
    pos = torch.tensor([40, 40], dtype=torch.int32, device="cuda")
    cnt = torch.tensor([n, 0], dtype=torch.int32, device="cuda")
    K.kvq_quantize_append(p, dc.cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), pos, cnt)
    torch.cuda.synchronize()
    assert dc.cache.status() == 0
    from oracle import cache as OC
    from gpu_util import specs

    def share(t, b):   # sequence b's part of a buffer laid out [B, ...]
        return t.reshape(w.B, -1)[b]
    for key in ("codes0", "codes1", "meta0", "meta1", "count", "bstart"):
        assert torch.equal(share(dc.cache.tensors[key], 1), share(before[key], 1)), key
    assert not torch.equal(share(dc.cache.tensors["codes0"], 0), share(before["codes0"], 0))
    for h in range(w.H):
        for kv in (0, 1):
            spec, _ = specs(w, h, kv)
            ref = OC.build_list(G.kv_rows(w, 1, h, kv, 0, w.S), spec)
            assert_list_equal(read_list(dc, 1, h, kv), ref, f"h={h} kv={kv}")


def test_paged_bad_slot_reports_status():
    """A block-table entry naming a slot outside its pool is reported by the decoder (the rows
    of that page read as zeros; nothing is read outside the pools)."""
    import decode_attention_sub_amd as K
    w = SMALL["tiered_small"]
    dc = WD.build(w)
    p = dc.params
    for entry in (p.num_pages + 5, (1 << 31) | (p.num_pages_fp8 + 3)):
        bt = dc.block_table_host.copy()
        bt[0, 1] = np.uint32(entry).view(np.int32)
        dc.cache.tensors["status"].zero_()
        dcb = WD.DeviceCache(w, p, dc.cache, dc.seq_lens_host, dc.seq_lens, bt,
                             torch.from_numpy(bt).cuda(), dc.q_host, dc.q)
        for split in (0, 128):
            log(f"[gpu] decode with bad block-table entry {entry:#x} split={split}")
            dc.cache.tensors["status"].zero_()
            run_decode(dcb, split_chunk=split)
            assert dc.cache.status() == K.KVQ_ERR_INVALID_ARG


# Many (sequence, KV head) units with short chunks: the launcher packs several chunks into one
# workgroup (4 chunks of 3 waves for 2-bit, 2 chunks of 6 waves for FP4 g32) and the merge sums
# 12 / 10 chunk partials.
PACKED = {
    "c2_packed": (WD.variant(CONFIGS["c2_b16_s8k"], B=32, Hq=32, H=8, S=1500), 128),
    "fp4_packed": (WD.variant(CONFIGS["fp4_b4_s128k"], B=8, Hq=64, H=8, S=2500, split_chunk=256), 256),
}


@pytest.mark.parametrize("name", sorted(PACKED))
def test_decode_packed_chunks(name):
    w, split = PACKED[name]
    log(f"[gpu] packed chunks {name}: building the cache")
    dc = WD.build(w)
    assert dc.cache.status() == 0
    got = run_decode(dc, split_chunk=split)
    sm = 1.0 / math.sqrt(w.D)
    for b in (0, w.B // 2 + 1, w.B - 1):
        ref = oracle_attention(dc, b, range(w.Hq), sm)
        for hq, o in ref.items():
            err = np.abs(got[b, hq] - o).max()
            assert err <= ATOL, f"{name} b={b} hq={hq} split={split}: max-abs {err}"


PREFIX = {
    # decode over a prefix of each list: lengths around the 16-token blocks and 32-token steps,
    # with the lists' later tokens and outlier records present in the cache
    "c2_g8": WD.variant(CONFIGS["c2_b64_s32k"], B=8, H=2, Hq=16, S=300),
    "c2_g16": WD.variant(CONFIGS["c2_b64_s32k"], B=8, H=1, Hq=16, S=300),
    "u2_g4": WD.variant(CONFIGS["c2_b16_s8k"], B=8, H=2, Hq=8, S=300, fmt="u2"),
    "fp4_g8": WD.variant(CONFIGS["fp4_b4_s128k"], B=8, H=2, Hq=16, S=300),
    "int4_g4": WD.variant(CONFIGS["int4_b1_s1k"], B=8, S=300),
    "int3_g4": WD.variant(CONFIGS["int4_b1_s1k"], B=8, S=300, fmt="int3"),
}


@pytest.mark.parametrize("name", sorted(PREFIX))
def test_decode_prefix_lengths(name):
    import dataclasses
    from oracle import attention as OA
    from gpu_util import dequant_from_device
    w = PREFIX[name]
    log(f"[gpu] prefix decode {name}")
    dc = WD.build(w)
    lens = np.array([1, 2, 15, 16, 17, 31, 33, 300], dtype=np.int32)[:w.B]
    full = {(b, h): dequant_from_device(dc, b, h) for b in range(w.B) for h in range(w.H)}
    dcp = dataclasses.replace(dc, seq_lens_host=lens, seq_lens=torch.from_numpy(lens).cuda())
    sm = 1.0 / math.sqrt(w.D)
    G_ = w.Hq // w.H
    for split in (0, 64, 128):
        got = run_decode(dcp, split_chunk=split, sm_scale=sm)
        for b in range(w.B):
            qf = OA.bf16_to_f64(dc.q_host[b])
            for hq in range(w.Hq):
                Kd, Vd = full[(b, hq // G_)]
                ref = OA.attention_one(qf[hq], Kd[:lens[b]], Vd[:lens[b]], sm)
                err = np.abs(got[b, hq] - ref).max()
                assert err <= ATOL, f"{name} b={b} S={lens[b]} hq={hq} split={split}: max-abs {err}"


def _special_rows(n_rep: int = 2):
    """Rows that stress the fits: zeros, a constant, one spike, alternating signs, fp32
    subnormals, large values, a value past the E4M3 range, fp16 rounding ties."""
    rng = np.random.default_rng(99)
    D = 128
    rows = [np.zeros(D), np.full(D, 3.5), np.where(np.arange(D) == 7, 1000.0, 0.0),
            np.where(np.arange(D) % 2 == 0, 1.0, -1.0), rng.standard_normal(D) * 1e-40,
            rng.standard_normal(D) * 2e4, np.where(np.arange(D) == 100, 1e6, rng.standard_normal(D)),
            (rng.integers(-64, 64, D) + 0.5) * 2.0 ** -10,
            np.concatenate([np.full(64, -2.0), np.full(64, 5.0)])]
    x = np.stack(rows * n_rep).astype(np.float32)
    return x


@pytest.mark.parametrize("fmt,group,outlier", [("c2", 64, "e4m3"), ("c2", 64, "none"),
                                               ("u2", 64, "fp16"), ("int4", 32, "fp16"),
                                               ("int4s", 64, "e4m3"), ("fp4", 32, "fp16"),
                                               ("int3", 32, "fp16"), ("int3", 64, "none"),
                                               ("int4", 64, "none")])
def test_quantize_special_rows(fmt, group, outlier):
    """Degenerate and extreme rows, appended in one call, are packed bit for bit like the
    oracle's."""
    import decode_attention_sub_amd as K
    from oracle import cache as OC
    from oracle import quantize as OQ
    x = _special_rows()
    if fmt in ("int3", "int4") and outlier == "none":
        # scale and zero both beyond the fp16 range: every quotient is inf / inf, code 0
        x = np.concatenate([x, np.where(np.arange(128) % 2 == 0, 1e6, -1e6)[None].astype(np.float32)])
    n = x.shape[0]
    w = WD.variant(CONFIGS["c2_b16_s8k"], B=1, H=1, Hq=4, S=n, fmt=fmt, group=group, outlier=outlier)
    p = WD.make_params(w, 64)
    cache = K.KVCache.allocate(p, 4096)
    k = torch.from_numpy(x[None, None]).cuda()
    v = torch.from_numpy(-x[None, None]).cuda()
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    cnt = torch.full((1,), n, dtype=torch.int32, device="cuda")
    K.kvq_quantize_append(p, cache, k, v, zero, cnt)
    torch.cuda.synchronize()
    assert cache.status() == 0
    lens = np.array([n], dtype=np.int32)
    dc = WD.DeviceCache(w, p, cache, lens, torch.from_numpy(lens).cuda(), None, None, None, None)
    spec = OQ.QuantSpec(fmt, group, outlier, w.sigma, w.lloyd_iters)
    for kv, rows in ((0, x), (1, -x)):
        assert_list_equal(read_list(dc, 0, 0, kv), OC.build_list(rows, spec), f"{fmt} {outlier} kv={kv}")
