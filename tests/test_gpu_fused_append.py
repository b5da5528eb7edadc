"""GPU parity of the fused append + decode (kvq_append_decode) against the oracle.

The call appends one new token per sequence at position seq_lens[b] - 1 (the list is cut back to
the records of earlier tokens, as an append there does) and decodes over seq_lens.  Checked:
  * every list's bytes (codes, metadata, outlier records, count, block starts) equal the oracle's
    list of the same rows with row seq_lens[b] - 1 replaced by the new token (bit-exact);
  * the output is within 2e-3 of the oracle's float64 attention over the cache's own bytes;
  * the output agrees with the two separate calls (append, then decode) on a copy of the cache,
    and two fused calls from the same cache state give the same bits.
Cases span 2-bit and FP4 caches, E4M3 / fp16 / no outliers, a static channel mask, the uniform
codebook, up to 8 and 16 query heads per KV head, new tokens at positions 0, mid-step and at a
step boundary, and default and fine work splits (lists cut between many workgroups)."""

import math

import numpy as np
import pytest
import torch

import decode_attention_sub_amd as K
from gpu_util import ATOL, assert_list_equal, log, oracle_attention, read_list, specs
from oracle import cache as OC
from workloads import CONFIGS
from workloads import device as WD
from workloads import generate as G

pytestmark = pytest.mark.gpu


def clone_cache(c):
    """A second device cache holding the same bytes as cache c."""
    t = c.tensors
    mask = t["chan_mask"]
    c2 = K.KVCache.allocate(c.params, c.outl_capacity, "cuda",
                            chan_mask=None if mask is None else mask.clone())
    for k, v in t.items():
        if v is not None and k != "chan_mask":
            c2.tensors[k].copy_(v)
    return c2


def new_rows(w, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((w.B, w.H, w.D)).astype(np.float32)
    v = rng.standard_normal((w.B, w.H, w.D)).astype(np.float32)
    # a few large channels so that the new rows hold outlier records
    k[..., 3] *= 12.0
    v[..., 77] *= -15.0
    return k, v


def run_fused(dc, cache, k_new, v_new, lens_t, split_chunk):
    w, p = dc.w, dc.params
    ws = K.kvq_workspace_bytes(p, split_chunk)
    work = torch.empty(max(ws // 4, 1), dtype=torch.float32, device="cuda") if ws else None
    out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device="cuda")
    K.kvq_append_decode(p, cache, k_new, v_new, dc.q, lens_t, out, work, split_chunk=split_chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def run_separate(dc, cache, k_new, v_new, lens_t, split_chunk):
    w, p = dc.w, dc.params
    pos = (lens_t - 1).to(torch.int32)
    cnt = torch.ones(w.B, dtype=torch.int32, device="cuda")
    K.kvq_quantize_append(p, cache, k_new.view(w.B, w.H, 1, w.D), v_new.view(w.B, w.H, 1, w.D),
                          pos, cnt)
    ws = K.kvq_workspace_bytes(p, split_chunk)
    work = torch.empty(max(ws // 4, 1), dtype=torch.float32, device="cuda") if ws else None
    out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device="cuda")
    K.kvq_decode_attention(p, cache, dc.q, lens_t, out, work, split_chunk=split_chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # name, base workload, overrides, new-token positions + 1 per sequence, split chunks
    ("c2_e4m3_g8", "c2_b64_s32k", dict(B=4, H=2, Hq=16, S=700), [1, 33, 64, 700], [0, 128]),
    ("c2_e4m3_g16", "c2_b64_s32k", dict(B=3, H=2, Hq=32, S=300), [300, 2, 97], [0, 64]),
    ("c2_fp16", "c2_b64_s32k", dict(B=2, H=2, Hq=8, S=260, outlier="fp16"), [260, 129], [0]),
    ("c2_none", "c2_b64_s32k", dict(B=2, H=2, Hq=8, S=200, outlier="none"), [200, 31], [0]),
    ("c2_mask", "c2_b64_s32k", dict(B=2, H=2, Hq=16, S=300, chan_mask=4), [300, 17], [0, 64]),
    ("u2", "c2_b64_s32k", dict(B=2, H=2, Hq=16, S=300, fmt="u2"), [300, 40], [0]),
    ("fp4_fp16_g8", "fp4_b4_s128k", dict(B=3, H=2, Hq=16, S=900), [900, 1, 450], [0, 256]),
    ("fp4_g16", "fp4_b4_s128k", dict(B=2, H=2, Hq=32, S=300), [300, 65], [0]),
]


@pytest.mark.parametrize("name,base,over,lens,splits", CASES, ids=[c[0] for c in CASES])
def test_fused_append_decode(name, base, over, lens, splits):
    w = WD.variant(CONFIGS[base], **over)
    log(f"fused append+decode {name}: {over} lens {lens} splits {splits}")
    dc = WD.build(w)
    lens = np.array(lens, dtype=np.int32)
    lens_t = torch.from_numpy(lens).cuda()
    kh, vh = new_rows(w, 77)
    k_new = torch.from_numpy(kh).cuda()
    v_new = torch.from_numpy(vh).cuda()
    sm = 1.0 / math.sqrt(w.D)
    base_cache = clone_cache(dc.cache)
    for split in splits:
        cache_f = clone_cache(dc.cache) if split != splits[-1] else dc.cache
        cache_s = clone_cache(base_cache)
        cache_r = clone_cache(base_cache)
        got = run_fused(dc, cache_f, k_new, v_new, lens_t, split)
        ref_sep = run_separate(dc, cache_s, k_new, v_new, lens_t, split)
        again = run_fused(dc, cache_r, k_new, v_new, lens_t, split)
        assert int(cache_f.tensors["status"].item()) == 0, "fused call reported an error"
        assert np.array_equal(got.view(np.uint32), again.view(np.uint32)), f"{name}: not deterministic"
        assert np.abs(got - ref_sep).max() <= ATOL, f"{name} split {split}: fused vs separate"
        # the lists: the oracle's rows with the new token at lens[b] - 1
        view = WD.DeviceCache(w, dc.params, cache_f, lens, lens_t, None, None, dc.q_host, dc.q)
        for b in range(w.B):
            S = int(lens[b])
            for h in range(w.H):
                for kv in (0, 1):
                    x = G.kv_rows(w, b, h, kv, 0, S)
                    x[S - 1] = (kh if kv == 0 else vh)[b, h]
                    spec, _ = specs(w, h, kv)
                    ref = OC.build_list(x, spec)
                    assert_list_equal(read_list(view, b, h, kv), ref,
                                      f"{name} split {split} b={b} h={h} kv={kv}")
        worst = 0.0
        for b in range(w.B):
            for hq, o in oracle_attention(view, b, range(w.Hq), sm).items():
                worst = max(worst, float(np.abs(got[b, hq] - o).max()))
        log(f"  split {split}: lists bit-exact, attention max-abs {worst:.2e}")
        assert worst <= ATOL, f"{name} split {split}: attention error {worst}"


def test_fused_invalid_length_appends_nothing():
    w = WD.variant(CONFIGS["c2_b64_s32k"], B=3, H=2, Hq=16, S=200)
    dc = WD.build(w)
    before = {k: v.clone() for k, v in dc.cache.tensors.items() if v is not None}
    lens = torch.tensor([200, 0, 120], dtype=torch.int32, device="cuda")
    kh, vh = new_rows(w, 5)
    out = torch.full((w.B, w.Hq, w.D), 7.0, dtype=torch.float32, device="cuda")
    ws = K.kvq_workspace_bytes(dc.params, 0)
    work = torch.empty(max(ws // 4, 1), dtype=torch.float32, device="cuda")
    K.kvq_append_decode(dc.params, dc.cache, torch.from_numpy(kh).cuda(), torch.from_numpy(vh).cuda(),
                        dc.q, lens, out, work)
    torch.cuda.synchronize()
    assert dc.cache.status() == K.KVQ_ERR_INVALID_ARG
    assert torch.all(out[1] == 7.0), "the rejected sequence's output was written"
    assert torch.isfinite(out[0]).all() and torch.isfinite(out[2]).all()
    # sequence 1's lists are untouched
    cap = dc.cache.outl_capacity
    for kv in (0, 1):
        for h in range(w.H):
            lid = (1 * w.H + h) * 2 + kv
            assert dc.cache.tensors["count"][lid] == before["count"][lid]
            a = dc.cache.tensors[f"idx{kv}"].view(w.B, w.H, cap)[1, h]
            assert torch.equal(a, before[f"idx{kv}"].view(w.B, w.H, cap)[1, h])


def test_fused_rejects_unsupported_caches():
    w = WD.variant(CONFIGS["int4_b1_s1k"], S=64)
    dc = WD.build(w)
    k = torch.zeros((w.B, w.H, w.D), dtype=torch.float32, device="cuda")
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    with pytest.raises(K.KvqError) as e:
        K.kvq_append_decode(dc.params, dc.cache, k, k, dc.q, dc.seq_lens, out)
    assert e.value.status == K.KVQ_ERR_UNSUPPORTED


FULL = ["c2_b16_s8k", "c2_b64_s32k", "fp4_b4_s128k"]


@pytest.mark.parametrize("name", FULL)
def test_fused_full_size_sampled(name):
    """The fused call at the workload's full size (the launch bench.py --fused times): the new
    rows and the tail of sampled lists bit for bit, and the sampled (sequence, KV head) pairs'
    attention within the bar of the oracle over the cache's bytes."""
    w = CONFIGS[name]
    log(f"[gpu] fused full-size {name}: building the cache")
    dc = WD.build(w)
    assert dc.cache.status() == 0
    kh, vh = new_rows(w, 99)
    lens_t = dc.seq_lens
    log(f"[gpu] fused full-size {name}: append + decode")
    got = run_fused(dc, dc.cache, torch.from_numpy(kh).cuda(), torch.from_numpy(vh).cuda(), lens_t,
                    w.split_chunk)
    assert dc.cache.status() == 0
    assert np.all(np.isfinite(got))
    lens = dc.seq_lens_host
    rng = np.random.default_rng(4321)
    pairs = {(w.B - 1, w.H - 1), (int(rng.integers(w.B)), int(rng.integers(w.H)))}
    sm = 1.0 / math.sqrt(w.D)
    G_ = w.Hq // w.H
    for b, h in sorted(pairs):
        S = int(lens[b])
        ta = max(0, (S - 160) // 16 * 16)
        for kv in (0, 1):
            x = G.kv_rows(w, b, h, kv, ta, S)
            x[-1] = (kh if kv == 0 else vh)[b, h]
            spec, _ = specs(w, h, kv)
            ref = OC.build_list(x, spec)
            dev = read_list(dc, b, h, kv)
            what = f"{name} b={b} h={h} kv={kv} rows {ta}..{S}"
            assert np.array_equal(dev["packed"][ta:S], ref.packed), what + ": codes"
            assert np.array_equal(dev["meta"][ta:S], ref.meta), what + ": metadata"
            tok = dev["idx"].astype(np.int64) >> 7
            sel = (tok >= ta) & (tok < S)
            assert np.array_equal(dev["idx"][sel].astype(np.int64) - ta * w.D, ref.idx.astype(np.int64)), \
                what + ": outlier indices"
            assert np.array_equal(dev["vals"][sel], ref.vals), what + ": outlier values"
        log(f"[gpu] fused full-size {name}: oracle attention b={b} h={h} S={S}")
        for hq, o in oracle_attention(dc, b, range(h * G_, (h + 1) * G_), sm).items():
            err = np.abs(got[b, hq] - o).max()
            assert err <= ATOL, f"{name} b={b} hq={hq}: max-abs {err}"
