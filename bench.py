"""Benchmark of the quantized-KV decode step on one MI355X.

One step = quantize-append of one new token per sequence (re-appending the last position, so the
context stays at S) and fused dequantize + decode attention over S tokens: an append launch and
a decode launch, or with ``--fused`` one launch that does both (kvq_append_decode; contiguous
2-bit and FP4 caches).  Inputs are seeded synthetic data resident in HBM before timing starts.

Prints one JSON line.  ``value`` is algorithmic KV bytes moved per second by the whole step;
``roofline`` reports the decode launch alone (its bytes, with the appended rows' bytes when the
launch also appends, / its average launch time measured with HIP events on the stream it runs
on) against the 8 TB/s HBM peak; ``cpu_baseline`` is the oracle timed on a bounded sample of
the same step on the host cores.

    python bench.py [--gpus 1] [--steps 100] [--warmup 40] [--workload c2_b64_s32k] [--flush auto]

Workloads whose decode moves less than 768 MB would otherwise be read partly from the 256 MB
Infinity Cache and the L2s on the next step; for them (``--flush auto``) every step starts by
streaming a 1 GiB buffer through the caches, outside the timed step, and the step time is the
sum of the per-step event intervals.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn KV bytes/s and % of HBM peak; us/step at B=64,S=32k 2-bit"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def fp8_pages(dc, seq_lens: np.ndarray) -> int:
    """Pages of the sequences' live token ranges that the block table puts in the FP8 tier."""
    tiers = (dc.block_table_host.view(np.uint32) >> 31) == 1
    return sum(int(tiers[b, :(int(s) + 15) // 16].sum()) for b, s in enumerate(seq_lens))


def algorithmic_bytes(dc, n_outliers: int, seq_lens: np.ndarray) -> int:
    """Bytes the decode must move: codes + per-group metadata of every row, outlier records
    (value + 4-byte index) actually present, the bf16 query read and the fp32 output written,
    plus the block table of a paged cache."""
    import decode_attention_sub_amd as K
    w, p = dc.w, dc.params
    sz = K.kvq_cache_sizes(p, 1)
    tokens = int(seq_lens.sum())
    vb = 2 if w.outlier == "fp16" else 1
    if w.paged:
        tok8 = fp8_pages(dc, seq_lens) * 16  # whole pages (the last page of a sequence may be partial)
        tok8 = min(tok8, tokens)
        kv = 2 * w.H * ((tokens - tok8) * (sz.code_bytes_per_row + sz.meta_bytes_per_row)
                        + tok8 * (w.D + 4))
        table = sum((int(s) + 15) // 16 for s in seq_lens) * 4
    else:
        kv = 2 * w.H * tokens * (sz.code_bytes_per_row + sz.meta_bytes_per_row)
        table = 0
    return kv + n_outliers * (vb + 4) + w.B * w.Hq * w.D * (2 + 4) + table


KERNEL_SOURCES = ["decode_attention_sub_amd/csrc/decode_mfma.hip",
                  "decode_attention_sub_amd/csrc/kvq_device.h",
                  "decode_attention_sub_amd/csrc/kvq_launch.h"]


def measured_counters(workload: str) -> dict:
    """HBM bytes and busy fractions per decode launch from the committed counter record of this
    workload: {"traffic": bytes, "mfma_busy": fraction, "valu_busy": fraction}, each None when the
    record lacks it, and all None when there is no record or the decode kernel's sources have
    changed since it was taken.

    mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * 1024 SIMDs): the share of SIMD
    cycles with a matrix instruction in flight.  valu_busy = 4 * SQ_ACTIVE_INST_VALU /
    (GRBM_GUI_ACTIVE * 1024): the share of SIMD cycles issuing vector ALU instructions
    (SQ_ACTIVE_INST_VALU counts in units of four cycles)."""
    import hashlib
    none = {"traffic": None, "mfma_busy": None, "valu_busy": None}
    path = os.path.join(ROOT, "profiles", f"decode_mfma_{workload}_counters.txt")
    if not os.path.exists(path):
        return none
    rec = {}
    for ln in open(path):
        if ln.startswith("#") or ":" not in ln:
            continue
        k, v = ln.split(":", 1)
        rec[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if rec.get("workload") != workload or rec.get("kernel_sources_sha256") != h.hexdigest():
        return none
    out = dict(none)
    if "traffic_bytes_per_launch" in rec:
        out["traffic"] = int(rec["traffic_bytes_per_launch"])
    for k in ("mfma_busy", "valu_busy"):
        if k in rec:
            out[k] = float(rec[k])
    return out


def read_ceiling_gbs(device="cuda") -> float:
    import torch
    import decode_attention_sub_amd as K
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=device)
    buf.fill_(1)
    sink = torch.empty(1024 * 256, dtype=torch.int32, device=device)
    K.kvq_probe_read(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        K.kvq_probe_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = 5 * buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    return gbs


def _oracle_worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)   # one thread per worker process: cores = worker processes


def _oracle_slice(task):
    """The oracle's work for one (sequence, KV head) group of one step: float32 quantization of
    the new token's K and V rows, float64 dequantization of both lists, float64 attention of the
    group's query heads.  Returns (seconds, algorithmic bytes)."""
    from oracle import attention as OA
    from oracle import cache as OC
    from oracle import quantize as OQ
    spec, spec8, D, lists, x_new, qf, sm, vb = task
    t0 = time.perf_counter()
    for x in x_new:
        OQ.quantize_rows(x, spec)
    KV = []
    for g in lists:
        codes = OQ.unpack_codes(g["packed"], OQ.CODE_BITS[spec.fmt], D)
        KV.append(OC.dequantize_list(codes, g["meta"], g["idx"], g["vals"], spec, D,
                                     g["tier1"], g.get("packed8"), g.get("meta8"), spec8))
    for q in qf:
        OA.attention_one(q, KV[0], KV[1], sm)
    dt = time.perf_counter() - t0
    S = lists[0]["packed"].shape[0]
    n_out = len(lists[0]["idx"]) + len(lists[1]["idx"])
    row = lists[0]["packed"].shape[1] + lists[0]["meta"].shape[1]
    return dt, 2 * S * row + n_out * (vb + 4) + len(qf) * D * 6


def cpu_baseline(dc, single_budget_s: float = 8.0, max_groups: int = 256):
    """The oracle (float32 quantization of the new token, float64 dequantization and attention),
    as it stands, on a sample of (sequence, KV head) groups of the same step, in the metric's
    unit (GB/s of algorithmic bytes).  The groups run in parallel worker processes, one per
    host core available to this process (at most 16), each single-threaded; a second figure
    runs groups one after another on a single core."""
    import multiprocessing as mp
    from oracle import attention as OA
    from oracle import quantize as OQ
    from workloads import generate as G
    from workloads.device import read_list

    w = dc.w
    spec = OQ.QuantSpec(w.fmt, w.group, w.outlier, w.sigma, w.lloyd_iters)
    spec8 = OQ.QuantSpec("fp8row", 0, "none") if w.paged else None
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    rng = np.random.default_rng(0)
    rng.shuffle(pairs)
    pairs = pairs[:max_groups]
    G_ = w.Hq // w.H
    sm = 1.0 / math.sqrt(w.D)
    vb = 2 if w.outlier == "fp16" else 1
    tasks = []
    for b, h in pairs:   # device bytes are read back before any timing
        lists = [read_list(dc, b, h, kv) for kv in (0, 1)]
        x_new = [G.new_rows(w, b, h, G.NEW_K + kv, 0) for kv in (0, 1)]
        qf = OA.bf16_to_f64(dc.q_host[b])[h * G_:(h + 1) * G_]
        tasks.append((spec, spec8, w.D, lists, x_new, qf, sm, vb))
    host_cpus = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = host_cpus
    workers = max(1, min(avail, 16))
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_oracle_worker_init) as pool:
        pool.map(_oracle_slice, tasks[:workers], chunksize=1)   # warm the workers
        t0 = time.perf_counter()
        res = pool.map(_oracle_slice, tasks, chunksize=1)
        wall = time.perf_counter() - t0
    par_bytes = sum(r[1] for r in res)
    with ctx.Pool(1, initializer=_oracle_worker_init) as pool:
        pool.map(_oracle_slice, tasks[:1])
        one_t, one_b, n_one = 0.0, 0, 0
        for dt, nb in pool.imap(_oracle_slice, tasks, chunksize=1):
            one_t += dt
            one_b += nb
            n_one += 1
            if one_t >= single_budget_s:
                break
    return {"value": round(par_bytes / wall / 1e9, 6), "unit": "GB/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{len(tasks)} of {w.B * w.H} (sequence, KV head) groups of one step "
                      f"({len(tasks) * G_} query heads over their full context) in {workers} "
                      f"single-threaded worker processes, {wall:.1f} s wall, "
                      f"{sum(r[0] for r in res):.1f} s of oracle time; host has {host_cpus} CPUs, "
                      f"{avail} available to the process",
            "single_core": {"value": round(one_b / one_t / 1e9, 6), "unit": "GB/s", "cores": 1,
                            "sample": f"{n_one} groups one after another, {one_t:.1f} s"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--ramp-s", type=float, default=0.3,
                    help="seconds of back-to-back steps before the warmup steps, so the shader "
                         "clock has ramped up whatever --warmup is (not timed, not counted)")
    ap.add_argument("--workload", default="c2_b64_s32k")
    ap.add_argument("--split", type=int, default=-1, help="split-K chunk (default: workload's)")
    ap.add_argument("--fmt", default=None,
                    help="other format on the workload's shapes and data: u2 for 2-bit workloads "
                         "(uniform codebook, same storage), int4s (symmetric fit, same storage) or "
                         "int3 (3-bit codes) for INT4 ones")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chan-mask", type=int, default=0,
                    help="keep this many calibrated top channels per (KV head, K or V) as outlier "
                         "records in every row (static channel mask) instead of the tau test")
    ap.add_argument("--flush", choices=("auto", "on", "off"), default="auto",
                    help="stream 1 GiB through the caches before every step (auto: when the "
                         "decode moves less than 768 MB)")
    ap.add_argument("--retier-every", type=int, default=0,
                    help="paged workloads: every N-th timed step decodes with page masses and "
                         "moves the cold FP8 pages to the 2-bit tier (after one initial conversion, "
                         "timed on its own)")
    ap.add_argument("--retier-keep", type=float, default=0.15,
                    help="fraction of each sequence's pages (by attention mass) kept in FP8")
    ap.add_argument("--prologue", action="store_true",
                    help="each step runs the fused attention prologue (RMSNorm, Q/K/V projection of "
                         "width Hq*D with seeded bf16 weights, KV-cache write of the new token) in "
                         "place of the append, and decodes with the queries it produced")
    ap.add_argument("--fused", action="store_true",
                    help="one launch per step that appends and decodes (kvq_append_decode; "
                         "contiguous 2-bit and FP4 g32 caches, without --prologue or "
                         "--retier-every) instead of an append launch and a decode launch")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (reference for byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the decode path is "
              "sharded by (sequence, KV head) and needs no exchange between GPUs", file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_attention_sub_amd as K
    from workloads import CONFIGS
    from workloads import device as WD
    from workloads import generate as G

    w = CONFIGS[args.workload]
    if args.fmt:
        base = {"u2": "c2", "int4s": "int4", "int3": "int4"}.get(args.fmt)
        if base != w.fmt:
            sys.exit(f"--fmt {args.fmt}: not an alternative to the workload's format {w.fmt}")
        w = WD.variant(w, fmt=args.fmt)
    if args.chan_mask:
        w = WD.variant(w, chan_mask=args.chan_mask)
    torch.cuda.set_device(0)
    ceiling = read_ceiling_gbs()
    log(f"measured read ceiling {ceiling:.0f} GB/s")
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        K.kvq_probe_copy(src, dst)
        torch.cuda.synchronize()
        del src, dst
    t0 = time.time()
    spare = 0
    if args.retier_every:
        if not w.paged:
            sys.exit("--retier-every needs a paged workload")
        spare = int(sum(int(t.sum()) for t in G.page_tiers(w, G.seq_lens(w))))   # FP8 pages
    dc = WD.build(w, log=log if w.S >= 32768 else None, spare_pages=spare)
    log(f"cache built in {time.time() - t0:.1f} s")
    p, cache = dc.params, dc.cache
    split = w.split_chunk if args.split < 0 else args.split
    ws = K.kvq_workspace_bytes(p, split)
    work = torch.empty(max(ws // 4, 1), dtype=torch.float32, device="cuda") if ws else None
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lens = dc.seq_lens
    pos = (lens - 1).to(torch.int32)
    ones = torch.ones(w.B, dtype=torch.int32, device="cuda")
    n_total = args.warmup + args.steps
    new_k, new_v = [], []
    for s in range(n_total):
        k = np.stack([[G.new_rows(w, b, h, G.NEW_K, s)[0] for h in range(w.H)] for b in range(w.B)])
        v = np.stack([[G.new_rows(w, b, h, G.NEW_V, s)[0] for h in range(w.H)] for b in range(w.B)])
        new_k.append(torch.from_numpy(k[:, :, None, :]).cuda())
        new_v.append(torch.from_numpy(v[:, :, None, :]).cuda())
    q_dec = dc.q
    if args.prologue:
        d_model = G.model_width(w)
        log(f"prologue: generating the {(w.Hq + 2 * w.H) * w.D} x {d_model} projection")
        W_row = torch.from_numpy(G.projection(w, d_model).view(np.int16)).cuda()
        W_dev = torch.empty_like(W_row)
        K.kvq_prologue_pack_weights(p, W_row, W_dev)   # once, as at model load
        del W_row
        gain_dev = torch.from_numpy(G.norm_gain(w, d_model).view(np.int16)).cuda()
        n_hid = min(n_total, 8)
        hid = [torch.from_numpy(G.hidden_states(w, s, d_model).view(np.int16)).cuda() for s in range(n_hid)]
        pws = torch.zeros(K.kvq_prologue_workspace_bytes(p, d_model) // 4 + 1, dtype=torch.int32,
                          device="cuda")
        q_dec = torch.empty((w.B, w.Hq, w.D), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    fused = args.fused
    if fused and (args.prologue or args.retier_every or w.paged
                  or not (w.fmt in ("c2", "u2") or (w.fmt == "fp4" and w.group == 32))):
        sys.exit("--fused needs a contiguous 2-bit or FP4 g32 cache, without --prologue or "
                 "--retier-every")
    n_est = int(cache.tensors["count"].sum().item())
    flush = args.flush == "on" or (args.flush == "auto" and
                                    algorithmic_bytes(dc, n_est, dc.seq_lens_host) < (768 << 20))
    if flush:
        fbuf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        fbuf.fill_(1)
        fsink = torch.empty(1024 * 256, dtype=torch.int32, device="cuda")
        log("streaming 1 GiB through the caches before every step")

    retier = None
    if args.retier_every:
        # The FP8 pages of the built cache are a Bernoulli draw; one initial conversion moves the
        # cold ones to spare 2-bit slots (timed on its own).  Later calls, every N-th timed step,
        # refresh the ranking; each takes its own slice of the remaining free slots.
        mws = K.kvq_mass_workspace_bytes(p, split)
        mwork = torch.zeros(mws // 4 + 1, dtype=torch.float32, device="cuda")
        mass = torch.zeros((w.B, p.max_pages_per_seq), dtype=torch.float32, device="cuda")
        free_all = list(range(p.num_pages - spare, p.num_pages))
        n_moved = torch.zeros(1, dtype=torch.int32, device="cuda")

        def retier_call(free_list):
            n_free = len(free_list)
            rws = K.kvq_retier_workspace_bytes(p, n_free)
            rwork = torch.empty(rws // 4 + 1, dtype=torch.int32, device="cuda")
            free_t = torch.tensor(free_list, dtype=torch.int32, device="cuda") if n_free else None
            freed = torch.empty(max(1, min(n_free, p.num_pages_fp8)), dtype=torch.int32, device="cuda")
            return rwork, free_t, freed

        fp8_before = fp8_pages(dc, dc.seq_lens_host)
        ini = retier_call(free_all)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        K.kvq_decode_attention_mass(p, cache, dc.q, lens, out, mass, mwork, dc.block_table,
                                    split_chunk=split)
        K.kvq_retier(p, cache, dc.block_table, lens, mass, args.retier_keep, ini[1], ini[2],
                     n_moved, ini[0])
        e1.record(stream)
        torch.cuda.synchronize()
        moved0 = int(n_moved.item())
        dc.block_table_host[:] = dc.block_table.cpu().numpy()
        remaining = free_all[moved0:]
        n_calls = 2 * ((args.steps + args.retier_every - 1) // args.retier_every) + 1
        per = max(1, len(remaining) // n_calls) if remaining else 0
        calls = [retier_call(remaining[i * per:(i + 1) * per]) for i in range(n_calls)]
        retier = {"every": args.retier_every, "keep_frac": args.retier_keep,
                  "fp8_pages_before": fp8_before, "initial_pages_moved": moved0,
                  "initial_us": round(e0.elapsed_time(e1) * 1e3, 1),
                  "fp8_pages_after": fp8_pages(dc, dc.seq_lens_host),
                  "free_slots_per_call": per}
        log(f"initial re-tier: {moved0} of {fp8_before} FP8 pages moved in "
            f"{retier['initial_us']} us")
        call_i = [0]
        rt_ev = []

    def step(s, ev=None, do_retier=False):
        if flush:
            K.kvq_probe_read(fbuf, fsink)
        if ev is not None:
            ev[2].record(stream)
        if fused:   # one launch: the append of every sequence's token S - 1 and the decode
            if ev is not None:
                ev[0].record(stream)
            K.kvq_append_decode(p, cache, new_k[s], new_v[s], q_dec, lens, out, work,
                                split_chunk=split)
            if ev is not None:
                ev[1].record(stream)
            return
        if args.prologue:
            K.kvq_attention_prologue(p, cache, hid[s % n_hid], gain_dev, W_dev, 1e-5, pos, q_dec, pws,
                                     block_table=dc.block_table)
        else:
            K.kvq_quantize_append(p, cache, new_k[s], new_v[s], pos, ones, dc.block_table)
        if ev is not None:
            ev[0].record(stream)
        if do_retier:
            K.kvq_decode_attention_mass(p, cache, dc.q, lens, out, mass, mwork, dc.block_table,
                                        split_chunk=split)
            if ev is not None:
                ev[1].record(stream)
            c = calls[min(call_i[0], len(calls) - 1)]
            call_i[0] += 1
            K.kvq_retier(p, cache, dc.block_table, lens, mass, args.retier_keep, c[1], c[2],
                         n_moved, c[0])
            if ev is not None:
                r_ev = torch.cuda.Event(enable_timing=True)
                r_ev.record(stream)
                rt_ev.append((ev[1], r_ev))
            return
        K.kvq_decode_attention(p, cache, q_dec, lens, out, work, dc.block_table, split_chunk=split)
        if ev is not None:
            ev[1].record(stream)

    def retier_now(i):
        return retier is not None and (i + 1) % args.retier_every == 0

    # clock ramp: the shader clock climbs over the first few dozen back-to-back decodes
    t_ramp = time.perf_counter()
    n_ramp = 0
    while time.perf_counter() - t_ramp < args.ramp_s:
        for _ in range(5):
            step(n_ramp % n_total)
            n_ramp += 1
        torch.cuda.synchronize()
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    # Two timed passes over the same K steps (new tokens of the later steps of the pass
    # before).  The first has no event inside the loop and gives the step time; the second
    # brackets every append and every decode with events and gives the decode kernel's time.
    # With flushing, the step time is the sum of the per-step intervals of the second pass.
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, None, retier_now(i))
    g1.record(stream)
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + i, evs[i], retier_now(i))
    torch.cuda.synchronize()
    ms_step = (float(np.sum([e[2].elapsed_time(e[1]) for e in evs])) if flush
               else g0.elapsed_time(g1)) / args.steps
    plain = [i for i in range(args.steps) if not retier_now(i)]   # steps without re-tiering
    dec_all = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in plain])
    dec_ms = float(np.mean(dec_all))
    if retier is not None:
        mass_ms = [evs[i][0].elapsed_time(evs[i][1]) for i in range(args.steps) if retier_now(i)]
        retier["us_mass_decode"] = round(float(np.mean(mass_ms)) * 1e3, 2) if mass_ms else None
        retier["us_per_retier"] = (round(float(np.mean([a.elapsed_time(b) for a, b in rt_ev])) * 1e3, 2)
                                   if rt_ev else None)
        dc.block_table_host[:] = dc.block_table.cpu().numpy()   # the byte count uses the tiers now
    status = cache.status()
    if status != 0:
        raise RuntimeError(f"device status {status}: {K.kvq_status_string(status)}")

    n_out = int(cache.tensors["count"].sum().item())
    lens_h = dc.seq_lens_host
    dec_bytes = algorithmic_bytes(dc, n_out, lens_h)
    app_bytes = w.B * w.H * 2 * (w.D * 4 + K.kvq_cache_sizes(p, 1).code_bytes_per_row
                                 + K.kvq_cache_sizes(p, 1).meta_bytes_per_row)
    if args.prologue:
        # the projection's weights, the hidden states, the gain and q written, and the new rows'
        # codes and metadata (as for the append, without its float32 inputs)
        sz = K.kvq_cache_sizes(p, 1)
        pro_bytes = ((w.Hq + 2 * w.H) * w.D * d_model * 2 + w.B * d_model * 2 + d_model * 2
                     + w.B * w.Hq * w.D * 2 + w.B * w.H * 2 * (sz.code_bytes_per_row + sz.meta_bytes_per_row))
        pro_all = np.array([evs[i][2].elapsed_time(evs[i][0]) for i in plain])
        pro_ms = float(np.mean(pro_all))
        pro_flop = 2.0 * w.B * d_model * (w.Hq + 2 * w.H) * w.D
        app_bytes = pro_bytes
    step_bytes = dec_bytes + app_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    # the timed kernel: the decode, or in a fused step the launch that also appends
    kern_bytes = dec_bytes + (app_bytes if fused else 0)
    achieved = kern_bytes / (dec_ms * 1e-3) / 1e9
    elems = 2 * w.H * int(lens_h.sum()) * w.D
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if w.fmt in ("c2", "fp4", "u2") else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "H": w.H, "D": w.D,
                   "S": int(lens_h.max()), "format": w.fmt, "group": w.group,
                   "outliers": w.outlier, "tau": w.sigma, "split_chunk": split if split else "default",
                   "layers": 1, "cache_flush_per_step": flush, "channel_mask": w.chan_mask,
                   "clock_ramp_steps": n_ramp,
                   "step": "fused append+decode launch" if fused else "append launch + decode launch"},
        "us_per_step_decode": round(dec_ms * 1e3, 2),
        "us_decode_p10_p50_p90": [round(float(np.percentile(dec_all, q)) * 1e3, 2) for q in (10, 50, 90)],
        "us_per_step": round(ms_step * 1e3, 2),
        "pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "pct_read_ceiling": round(100 * achieved / ceiling, 2),
        "read_ceiling_GBs": round(ceiling, 1),
        "tokens_heads_per_s": round(int(lens_h.sum()) * w.H / (dec_ms * 1e-3), 1),
        "outliers": n_out, "outlier_fraction": round(n_out / elems, 6),
        "decode_bytes": dec_bytes,
        "kernel_bytes": kern_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     **measured_counters(w.name)},
    }
    if retier is not None:
        res["retier"] = retier
    if args.prologue:
        res["prologue"] = {
            "d_model": d_model, "us": round(pro_ms * 1e3, 2),
            "us_p10_p50_p90": [round(float(np.percentile(pro_all, q)) * 1e3, 2) for q in (10, 50, 90)],
            "bytes": pro_bytes, "GBs": round(pro_bytes / (pro_ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(pro_bytes / (pro_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tflops_bf16": round(pro_flop / (pro_ms * 1e-3) / 1e12, 2),
            "frac_mfma_bf16": round(pro_flop / (pro_ms * 1e-3) / 1e12 / 2500.0, 4)}
    if not args.no_cpu_baseline:
        log("timing the oracle on a sample of the step")
        res["cpu_baseline"] = cpu_baseline(dc)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
