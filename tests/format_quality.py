"""Error against bytes of the cache formats (the format-variants comparison), on the CPU with the
oracle: for seeded slices of a workload, every format's bits per element (codes, metadata and the
outlier records actually kept), the relative RMS error of the dequantized K and V, and the error
of the decode-attention output against attention over the unquantized rows (float64).

    python tests/format_quality.py [workload] [slices] [tokens]

Test infrastructure: it calls the oracle and the seeded generators only."""

from __future__ import annotations

import dataclasses
import math
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from oracle import attention as OA          # noqa: E402
from oracle import cache as OC              # noqa: E402
from oracle import quantize as OQ           # noqa: E402
from workloads import CONFIGS               # noqa: E402
from workloads import generate as G         # noqa: E402

# (label, format, group, outlier dtype[, static mask channels]): the workloads' formats, the
# variants stored like them and the 3-bit codes
FORMATS = [
    ("2-bit centroids, Lloyd (c2)", "c2", 64, "e4m3"),
    ("2-bit uniform linspace (u2)", "u2", 64, "e4m3"),
    ("2-bit centroids, no outliers", "c2", 64, "none"),
    ("2-bit uniform, no outliers", "u2", 64, "none"),
    ("INT4 asymmetric g32 (int4)", "int4", 32, "fp16"),
    ("INT4 symmetric g32 (int4s)", "int4s", 32, "fp16"),
    ("INT4 symmetric g32, no outliers", "int4s", 32, "none"),
    ("FP4 E2M1 g32 (fp4)", "fp4", 32, "fp16"),
    ("INT3 asymmetric g32 (int3)", "int3", 32, "fp16"),
    ("2-bit centroids, 2-channel fp16 mask", "c2", 64, "fp16", 2),
    ("INT4 asymmetric g32, 4-channel fp16 mask", "int4", 32, "fp16", 4),
]


def measure(workload: str = "c2_b64_s32k", slices: int = 4, tokens: int = 2048, formats=FORMATS):
    w = CONFIGS[workload]
    D = w.D
    G_ = w.Hq // w.H
    sm = 1.0 / math.sqrt(D)
    rows = []
    picks = [(b % w.B, (3 * b + 1) % w.H) for b in range(slices)]
    data = []
    for b, h in picks:
        x = [G.kv_rows(w, b, h, kv, 0, tokens) for kv in (0, 1)]
        q = OA.bf16_to_f64(G.queries(w, b))[h * G_:(h + 1) * G_]
        ref = np.stack([OA.attention_one(q[i], x[0].astype(np.float64), x[1].astype(np.float64), sm)
                        for i in range(G_)])
        data.append((x, q, ref))
    for label, fmt, g, out, *mask in formats:
        wm = dataclasses.replace(w, chan_mask=mask[0]) if mask else w
        spec_of = {(h, kv): OQ.QuantSpec(fmt, g, out, w.sigma, w.lloyd_iters,
                                         channels=G.mask_channels(wm, h, kv) if mask else ())
                   for _, h in picks for kv in (0, 1)}
        bits = 0
        se = [0.0, 0.0]
        ss = [0.0, 0.0]
        amax = 0.0
        rel = []
        for (b, h), (x, q, ref) in zip(picks, data):
            deq = []
            for kv in (0, 1):
                spec = spec_of[(h, kv)]
                ls = OC.build_list(x[kv], spec)
                d = OC.dequantize_list(ls.codes, ls.meta, ls.idx, ls.vals, spec, D)
                deq.append(d)
                xv = x[kv].astype(np.float64)
                se[kv] += float(np.sum((d - xv) ** 2))
                ss[kv] += float(np.sum(xv ** 2))
                bits += 8 * (ls.packed.size + ls.meta.size)
                bits += 8 * ls.count * ({"none": 0, "fp16": 2, "e4m3": 1}[out] + 4)
            o = np.stack([OA.attention_one(q[i], deq[0], deq[1], sm) for i in range(G_)])
            amax = max(amax, float(np.max(np.abs(o - ref))))
            rel.append(float(np.sqrt(np.sum((o - ref) ** 2) / np.sum(ref ** 2))))
        n_el = 2 * len(data) * tokens * D
        rows.append(dict(label=label, fmt=fmt, group=g, outlier=out, mask=mask[0] if mask else 0,
                         bits_per_element=bits / n_el,
                         k_rel_rmse=math.sqrt(se[0] / ss[0]), v_rel_rmse=math.sqrt(se[1] / ss[1]),
                         attn_max_abs=amax, attn_rel_rms=float(np.mean(rel))))
    return rows


def main():
    wl = sys.argv[1] if len(sys.argv) > 1 else "c2_b64_s32k"
    n = int(sys.argv[2]) if len(sys.argv) > 2 else 4
    t = int(sys.argv[3]) if len(sys.argv) > 3 else 2048
    rows = measure(wl, n, t)
    print(f"workload {wl}: {n} (sequence, KV head) slices x {t} tokens, K and V")
    print("| Format | bits / element | K rel. RMSE | V rel. RMSE | attention max-abs err | attention rel. RMS err |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['label']} | {r['bits_per_element']:.3f} | {r['k_rel_rmse']:.4f} | {r['v_rel_rmse']:.4f} "
              f"| {r['attn_max_abs']:.4f} | {r['attn_rel_rms']:.4f} |")


if __name__ == "__main__":
    main()
