"""Build a device cache for a workload by streaming the seeded rows through the library's
quantize-append entry point.  Holds no method arithmetic: it generates inputs, sizes buffers
and calls ``kvq_quantize_append``."""

from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

from . import generate as G
from .configs import Workload

FILL_CHUNK = 2048


def max_outliers_per_row(D: int, g: int, tau: float) -> int:
    """Capacity bound: m outliers in a group of g need m * tau^2 < g - 1 (one spare per group
    for rounding at exact equality)."""
    per_group = max(math.ceil((g - 1) / (tau * tau)) - 1, 0) + 1
    return (D // g) * min(per_group, g)


@dataclasses.dataclass
class DeviceCache:
    w: Workload
    params: object
    cache: object
    seq_lens_host: np.ndarray
    seq_lens: object            # torch int32 [B]
    block_table_host: Optional[np.ndarray]
    block_table: object         # torch int32 [B, max_pages] or None
    q_host: np.ndarray          # uint16 bf16 bits [B, Hq, D]
    q: object                   # torch bf16 [B, Hq, D]


def make_params(w: Workload, S_cap: int, n2: int = 0, n1: int = 0, max_pages: int = 0):
    import decode_attention_sub_amd as K
    if w.paged:
        return K.make_params(w.B, w.Hq, w.H, S_cap, w.fmt, w.group, w.outlier, w.sigma,
                             w.lloyd_iters, page_size=w.page_size, num_pages=n2,
                             num_pages_fp8=n1, max_pages_per_seq=max_pages)
    return K.make_params(w.B, w.Hq, w.H, S_cap, w.fmt, w.group, w.outlier, w.sigma, w.lloyd_iters)


def _rows_for(w: Workload, kind: int, t0: int, n: int, lens: np.ndarray, pool) -> np.ndarray:
    out = np.zeros((w.B, w.H, n, w.D), dtype=np.float32)

    def one(bh):
        b, h = bh
        m = int(min(n, max(int(lens[b]) - t0, 0)))
        if m > 0:
            out[b, h, :m] = G.kv_rows(w, b, h, kind, t0, t0 + m)

    list(pool.map(one, [(b, h) for b in range(w.B) for h in range(w.H)]))
    return out


def build(w: Workload, S_cap: Optional[int] = None, device: str = "cuda",
          threads: int = 16, extra_capacity_tokens: int = 0, log=None,
          spare_pages: int = 0) -> DeviceCache:
    """Allocate and fill the cache of workload ``w`` (all B sequences, every token).
    spare_pages (paged): free slots left at the end of the 2-bit pool (slots n2 .. n2 +
    spare_pages - 1), e.g. for pages moved there from the FP8 tier."""
    import torch
    import decode_attention_sub_amd as K

    lens = G.seq_lens(w)
    S_max = int(lens.max())
    S_cap = S_cap or (S_max + extra_capacity_tokens)
    bt_host = bt = None
    n2 = n1 = 0
    max_pages = 0
    if w.paged:
        max_pages = (S_cap + w.page_size - 1) // w.page_size
        tiers = G.page_tiers(w, np.minimum(lens + extra_capacity_tokens, S_cap))
        bt_host, n2, n1 = G.block_tables(w, tiers, max_pages)
        bt = torch.from_numpy(bt_host).to(device)
    p = make_params(w, S_cap, n2 + spare_pages, n1, max_pages)
    cap = max_outliers_per_row(w.D, w.group, w.sigma) * S_cap
    mask = None
    if w.chan_mask:
        assert w.chan_mask <= max_outliers_per_row(w.D, w.group, w.sigma)
        words = np.zeros((2, w.H, w.D // 32), dtype=np.uint32)
        for kv in (0, 1):
            for h in range(w.H):
                for c in G.mask_channels(w, h, kv):
                    words[kv, h, c // 32] |= np.uint32(1) << np.uint32(c % 32)
        mask = torch.from_numpy(words.view(np.int32)).to(device)
    cache = K.KVCache.allocate(p, cap, device, chan_mask=mask)
    lens_t = torch.from_numpy(lens).to(device)
    with ThreadPoolExecutor(threads) as pool:
        for t0 in range(0, S_max, FILL_CHUNK):
            n = min(FILL_CHUNK, S_max - t0)
            k = torch.from_numpy(_rows_for(w, G.K, t0, n, lens, pool)).to(device)
            v = torch.from_numpy(_rows_for(w, G.V, t0, n, lens, pool)).to(device)
            pos = torch.full((w.B,), t0, dtype=torch.int32, device=device)
            cnt = torch.clamp(lens_t - t0, 0, n).to(torch.int32)
            K.kvq_quantize_append(p, cache, k, v, pos, cnt, bt)
            if log:
                log(f"filled tokens {t0}..{t0 + n} of {S_max}")
    torch.cuda.synchronize()
    q_host = np.stack([G.queries(w, b) for b in range(w.B)])
    q = torch.from_numpy(q_host.view(np.int16)).to(device).view(torch.bfloat16)
    return DeviceCache(w, p, cache, lens, lens_t, bt_host, bt, q_host, q)


def variant(w: Workload, **kw) -> Workload:
    return dataclasses.replace(w, **kw)


def read_list(dc, b: int, h: int, kv: int):
    """Device cache -> host arrays of one (b, h, kv) list in logical token order: packed codes,
    metadata (FP8-tier rows separately for paged caches), outlier records and block starts."""
    import decode_attention_sub_amd as K
    w, p, t = dc.w, dc.params, dc.cache.tensors
    S = int(dc.seq_lens_host[b])
    sz = K.kvq_cache_sizes(p, dc.cache.outl_capacity)
    CB, MB = sz.code_bytes_per_row, sz.meta_bytes_per_row
    out = {}
    if not w.paged:
        codes = t[f"codes{kv}"].view(w.B, w.H, p.max_seq_len, CB)[b, h, :S].cpu().numpy()
        meta = t[f"meta{kv}"].view(w.B, w.H, p.max_seq_len, MB)[b, h, :S].cpu().numpy()
        out.update(packed=codes, meta=meta, tier1=None)
    else:
        ent = dc.block_table_host[b].view(np.uint32).astype(np.int64)[(np.arange(S) // 16)]
        tier1 = (ent >> 31) == 1
        slot = ent & 0x7FFFFFFF
        j = np.arange(S) % 16
        c2 = t[f"codes{kv}"].view(-1, w.H, 16, CB).cpu().numpy()
        m2 = t[f"meta{kv}"].view(-1, w.H, 16, MB).cpu().numpy()
        packed = np.zeros((S, CB), np.uint8)
        meta = np.zeros((S, MB), np.uint8)
        packed[~tier1] = c2[slot[~tier1], h, j[~tier1]]
        meta[~tier1] = m2[slot[~tier1], h, j[~tier1]]
        packed8 = np.zeros((S, w.D), np.uint8)
        meta8 = np.zeros((S, 4), np.uint8)
        if p.num_pages_fp8 > 0:
            c8 = t[f"codes8_{kv}"].view(-1, w.H, 16, w.D).cpu().numpy()
            s8 = t[f"scale8_{kv}"].view(-1, w.H, 16).cpu().numpy().view(np.uint8).reshape(-1, w.H, 16, 4)
            packed8[tier1] = c8[slot[tier1], h, j[tier1]]
            meta8[tier1] = s8[slot[tier1], h, j[tier1]]
        out.update(packed=packed, meta=meta, tier1=tier1, packed8=packed8, meta8=meta8)
    lid = (b * w.H + h) * 2 + kv
    cnt = int(t["count"][lid].item())
    cap = dc.cache.outl_capacity
    idx = t[f"idx{kv}"].view(w.B, w.H, cap)[b, h, :cnt].cpu().numpy().view(np.uint32)
    vb = 2 if w.outlier == "fp16" else 1
    raw = t[f"val{kv}"].view(w.B, w.H, cap * vb)[b, h, :cnt * vb].cpu().numpy()
    vals = raw.view(np.uint16) if vb == 2 else raw
    nblk_all = (p.max_seq_len + 15) // 16
    bstart = t["bstart"].view(w.B, w.H, 2, nblk_all)[b, h, kv, :(S + 15) // 16].cpu().numpy()
    out.update(idx=idx, vals=vals, count=cnt, block_start=bstart)
    return out
