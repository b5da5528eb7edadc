"""kvq_decode_attention_noalloc (the allocation-free variant for callers that cannot allocate)
against kvq_decode_attention on the same inputs, through the C ABI: two calls in a row, the
second on a smaller problem (fewer sequences, fewer chunks), each output equal bit for bit to
the workspace entry point's output with the same split; a request whose partials exceed the
scratch array is rejected before any launch."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import decode_attention_sub_amd as K  # noqa: E402
from workloads import CONFIGS  # noqa: E402
from workloads import device as WD  # noqa: E402

from gpu_util import log, run_decode  # noqa: E402


def _noalloc(dc, split):
    w = dc.w
    out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device="cuda")
    K.kvq_decode_attention_noalloc(dc.params, dc.cache, dc.q, dc.seq_lens, out, dc.block_table,
                                   split_chunk=split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name,split", [("c2", 128), ("fp4", 256), ("int4", 64),
                                        ("tiered", 256)])
def test_noalloc_matches_workspace_entry_point(name, split):
    big = {
        "c2": WD.variant(CONFIGS["c2_b64_s32k"], B=3, H=2, Hq=16, S=1500),
        "fp4": WD.variant(CONFIGS["fp4_b4_s128k"], B=3, H=2, Hq=16, S=2500),
        "int4": WD.variant(CONFIGS["int4_b1_s1k"], B=3, S=900),
        "tiered": WD.variant(CONFIGS["tiered_b32_paged"], B=3, H=2, Hq=8, S=2000,
                             S_range=(300, 2000), fp8_page_frac=0.3),
    }[name]
    small = WD.variant(big, B=1, S=big.S // 3,
                       S_range=None if big.S_range is None else (100, big.S // 3))
    for i, w in enumerate((big, small)):
        log(f"[gpu] noalloc {name} call {i} {w}")
        dc = WD.build(w)
        assert K.kvq_workspace_bytes(dc.params, split) > 0   # the partials go to the scratch
        ref = run_decode(dc, split_chunk=split)
        got = _noalloc(dc, split)
        assert dc.cache.status() == 0
        assert np.array_equal(got, ref), f"{name} call {i}: differs from kvq_decode_attention"


def test_noalloc_rejects_partials_beyond_scratch():
    w = WD.variant(CONFIGS["c2_b16_s8k"], B=2, H=2, Hq=8, S=200)
    dc = WD.build(w)
    p = WD.make_params(w, 1 << 20)   # the cache buffers are never touched: the call fails first
    p.batch = 64
    need = K.kvq_workspace_bytes(p, 64)
    assert need > K.NOALLOC_SCRATCH_BYTES
    with pytest.raises(K.KvqError) as e:
        out = torch.empty(1, dtype=torch.float32, device="cuda")
        K.kvq_decode_attention_noalloc(p, dc.cache, dc.q, dc.seq_lens, out, split_chunk=64)
    assert e.value.status == K.KVQ_ERR_WORKSPACE
