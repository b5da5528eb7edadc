"""GPU parity of the fused attention prologue (RMSNorm, joint Q/K/V projection, KV-cache write)
against the oracle.

* The projected rows (the kernel's float32 side output) against the oracle's float64 prologue,
  element by element within a bound derived from the kernel's arithmetic: every operand
  a_i = bf16(h_i g_i) is h_i g_i rounded once (relative error <= 2^-9), the products are exact
  and summed in float32 (error <= d 2^-24 sum |a_i W_ji|), and the row scale 1 / sqrt(sum h^2 /
  d + eps) carries a few float32 roundings of its own.  With a unit gain every operand is exact
  (a_i = h_i) and only the float32 sums remain.  The root-mean-square error is also held to a
  small multiple of what independent operand roundings give.
* q in bfloat16 equals the nearest-even rounding of the float32 projected row, bit for bit.
* The cache after the call equals, bit for bit, the oracle's lists with the kernel's own float32
  K and V rows appended at each sequence's position (floating point decides the codes, so both
  sides quantize the same float32 rows); a negative position leaves the sequence untouched.
* A decode with the new queries over the updated cache is within 2e-3 of the oracle.
* A second call gives identical results (the arrival counters return to zero; the sums do not
  depend on which workgroup finishes last)."""

import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import decode_attention_sub_amd as K  # noqa: E402
from oracle import cache as OC  # noqa: E402
from oracle import prologue as OP  # noqa: E402
from workloads import CONFIGS  # noqa: E402
from workloads import device as WD  # noqa: E402
from workloads import generate as G  # noqa: E402

from gpu_util import ATOL, assert_list_equal, log, oracle_attention, read_list, run_decode, specs  # noqa: E402

EPS = 1e-5
CASES = {
    # contiguous 2-bit cache, one row block, d_model 512 (4 stages of 128 columns)
    "c2": (WD.variant(CONFIGS["c2_b16_s8k"], B=3, H=2, Hq=8, S=300), 512, False),
    # 70 sequences: two row blocks, the second ragged (6 rows); 16 query heads per KV head
    "c2_rows": (WD.variant(CONFIGS["c2_b16_s8k"], B=70, H=1, Hq=16, S=40), 1024, False),
    # a unit gain: every bf16 operand is exact
    "c2_unit_gain": (WD.variant(CONFIGS["c2_b16_s8k"], B=2, H=2, Hq=4, S=100), 768, True),
    # INT4 groups of 32 with fp16 outliers
    "int4": (WD.variant(CONFIGS["int4_b1_s1k"], B=2, H=2, Hq=8, S=200), 512, False),
    # FP4 groups of 32 (E4M3 block scales)
    "fp4": (WD.variant(CONFIGS["fp4_b4_s128k"], B=2, H=2, Hq=8, S=200), 512, False),
    # paged cache with FP8 pages: the new row lands on an FP8 or a 2-bit page
    "tiered": (WD.variant(CONFIGS["tiered_b32_paged"], B=4, H=2, Hq=8, S=300, S_range=(90, 300),
                          fp8_page_frac=0.5), 640, False),
}


def _inputs(w, d, unit_gain):
    h = G.hidden_states(w, 0, d)
    g = G.f32_to_bf16_bits(np.ones(d, dtype=np.float32)) if unit_gain else G.norm_gain(w, d)
    W = G.projection(w, d)
    return h, g, W


def _run(dc, d, h, g, W, positions, ws=None):
    w, p = dc.w, dc.params
    dev = "cuda"
    ht = torch.from_numpy(h.view(np.int16)).to(dev)
    gt = torch.from_numpy(g.view(np.int16)).to(dev)
    Wr = torch.from_numpy(W.view(np.int16)).to(dev)
    Wt = torch.empty_like(Wr)
    K.kvq_prologue_pack_weights(p, Wr, Wt)
    pos = torch.tensor(positions, dtype=torch.int32, device=dev)
    q = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=dev)
    proj = torch.full((w.B, (w.Hq + 2 * w.H) * w.D), float("nan"), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.zeros(K.kvq_prologue_workspace_bytes(p, d) // 4 + 1, dtype=torch.int32, device=dev)
    K.kvq_attention_prologue(p, dc.cache, ht, gt, Wt, EPS, pos, q, ws, block_table=dc.block_table,
                             proj_out=proj)
    torch.cuda.synchronize()
    return q.cpu().numpy().view(np.uint16), proj.cpu().numpy(), ws


def _check_projection(w, d, h, g, W, proj, unit_gain):
    q_ref, k_ref, v_ref = OP.prologue(h, g, W, EPS, w.Hq, w.H, w.D)
    ref = np.concatenate([q_ref.reshape(w.B, -1), k_ref.reshape(w.B, -1), v_ref.reshape(w.B, -1)], 1)
    hf = OP.bf16_to_f64(h)
    gf = OP.bf16_to_f64(g)
    Wf = OP.bf16_to_f64(W)
    r = 1.0 / np.sqrt(np.mean(hf * hf, axis=1) + EPS)                  # [B]
    S1 = np.abs(hf * gf) @ np.abs(Wf).T                                # [B, n] sum |h g W|
    u = 2.0 ** -24
    op = 0.0 if unit_gain else 2.0 ** -9
    bound = (r[:, None] * S1 * (op + d * u * (1 + op)) * 1.01 + np.abs(ref) * (d + 8) * u) + 1e-30
    err = np.abs(proj.astype(np.float64) - ref)
    worst = np.max(err / bound)
    assert worst <= 1.0, f"projection error {worst:.3f} x its bound"
    # independent roundings: rms error about r * 2^-9 / sqrt(3) * sqrt(sum (h g W)^2)
    if not unit_gain:
        S2 = np.sqrt((hf * gf) ** 2 @ (Wf ** 2).T)
        expect = np.sqrt(np.mean((r[:, None] * S2 * 2.0 ** -9 / math.sqrt(3.0)) ** 2))
        rms = np.sqrt(np.mean(err ** 2))
        assert rms <= 2.0 * expect, f"rms error {rms:.3g} vs {expect:.3g} expected"
    return ref


@pytest.mark.parametrize("name", sorted(CASES))
def test_prologue_matches_oracle(name):
    w, d, unit_gain = CASES[name]
    log(f"[gpu] prologue {name}: B={w.B} Hq={w.Hq} H={w.H} d={d} fmt={w.fmt} paged={w.paged}")
    dc = WD.build(w, extra_capacity_tokens=1)
    assert dc.cache.status() == 0
    h, g, W = _inputs(w, d, unit_gain)
    lens = dc.seq_lens_host.copy()
    positions = [int(s) for s in lens]
    if w.B > 2:
        positions[1] = -1            # no cache write for this sequence
    q, proj, ws = _run(dc, d, h, g, W, positions)
    assert dc.cache.status() == 0, K.kvq_status_string(dc.cache.status())
    _check_projection(w, d, h, g, W, proj, unit_gain)
    # q: nearest-even bf16 of the float32 rows
    nq = w.Hq * w.D
    assert np.array_equal(q.reshape(w.B, -1), G.f32_to_bf16_bits(proj[:, :nq]))
    # cache lists: the oracle's with the kernel's float32 rows appended
    for b in range(w.B):
        S = int(lens[b])
        t = positions[b]
        n_tok = S + 1 if t >= 0 else S
        if w.paged:
            ent = dc.block_table_host[b].view(np.uint32)[: (n_tok + 15) // 16]
            tiers = (ent >> 31) == 1
        else:
            tiers = None
        for hk in range(w.H):
            for kv in (0, 1):
                spec, spec8 = specs(w, hk, kv)
                x = G.kv_rows(w, b, hk, kv, 0, S)
                if t >= 0:
                    col = (w.Hq + kv * w.H + hk) * w.D
                    x = np.concatenate([x, proj[b, col:col + w.D][None, :]]).astype(np.float32)
                ref = OC.build_list(x, spec, tiers, spec8)
                dc.seq_lens_host[b] = n_tok
                got = read_list(dc, b, hk, kv)
                dc.seq_lens_host[b] = S
                assert_list_equal(got, ref, f"{name} b={b} h={hk} kv={kv}")
    # a second call on the same workspace: identical results
    q2, proj2, _ = _run(dc, d, h, g, W, [-1] * w.B, ws)
    assert np.array_equal(q2, q) and np.array_equal(proj2, proj)
    assert dc.cache.status() == 0
    # decode with the new queries over the updated cache
    new_lens = np.array([int(s) + 1 if t >= 0 else int(s) for s, t in zip(lens, positions)], dtype=np.int32)
    dc.seq_lens_host[:] = new_lens
    dc.seq_lens.copy_(torch.from_numpy(new_lens))
    dc.q_host[:] = q.reshape(w.B, w.Hq, w.D)
    dc.q.copy_(torch.from_numpy(q.reshape(w.B, w.Hq, w.D).view(np.int16)).view(torch.bfloat16))
    sm = 1.0 / math.sqrt(w.D)
    got = run_decode(dc, sm_scale=sm)
    for b in range(w.B):
        for hq, o in oracle_attention(dc, b, range(w.Hq), sm).items():
            err = np.abs(got[b, hq] - o).max()
            assert err <= ATOL, f"{name} decode after the prologue b={b} hq={hq}: {err}"


def _pack_reference(W):
    """The block order of the packed weights, by index arithmetic on the host: block (cg, ks) of
    16 output rows x 32 inputs, its 16-byte unit 16 q + j = W[16 cg + j][32 ks + 8 q: +8]."""
    n, d = W.shape
    blocks = W.reshape(n // 16, 16, d // 32, 4, 8)        # [cg][j][ks][q][8]
    return np.ascontiguousarray(blocks.transpose(0, 2, 3, 1, 4)).reshape(-1)   # [cg][ks][q][j][8]


def test_packed_weights_layout():
    w = WD.variant(CONFIGS["c2_b16_s8k"], B=1, H=2, Hq=8, S=64)
    p = WD.make_params(w, 64)
    d = 384
    W = G.projection(w, d)
    Wr = torch.from_numpy(W.view(np.int16)).cuda()
    Wp = torch.empty_like(Wr)
    K.kvq_prologue_pack_weights(p, Wr, Wp)
    torch.cuda.synchronize()
    got = Wp.cpu().numpy().view(np.uint16).reshape(-1)
    assert np.array_equal(got, _pack_reference(W))
    # one hand-checked unit: block (cg 1, ks 2), unit 16 * 3 + 5 = W[16 + 5][64 + 24 .. 64 + 31]
    nks = d // 32
    u = ((1 * nks + 2) * 64 + 16 * 3 + 5) * 8
    assert np.array_equal(got[u:u + 8], W[21, 88:96])


def test_prologue_rejects_bad_arguments():
    w = WD.variant(CONFIGS["c2_b16_s8k"], B=2, H=2, Hq=8, S=64)
    p = WD.make_params(w, 64)
    with pytest.raises(K.KvqError):
        K.kvq_prologue_workspace_bytes(p, 100)        # d_model not a multiple of 128
    with pytest.raises(K.KvqError):
        K.kvq_prologue_workspace_bytes(p, 0)
