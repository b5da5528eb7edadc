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
          threads: int = 16, extra_capacity_tokens: int = 0, log=None) -> DeviceCache:
    """Allocate and fill the cache of workload ``w`` (all B sequences, every token)."""
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
    p = make_params(w, S_cap, n2, n1, max_pages)
    cap = max_outliers_per_row(w.D, w.group, w.sigma) * S_cap
    cache = K.KVCache.allocate(p, cap, device)
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
