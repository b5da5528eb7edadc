"""CPU tests of the C ABI: the library loads, exports every function include/kvq.h declares,
and its host-side arithmetic and argument validation behave as documented (no GPU calls)."""

import os
import re

import pytest

import decode_attention_sub_amd as K
from oracle import kvbytes as KB

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|const char\*)\s+(kvq_\w+)\(", src, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(K._lib, n), n
    assert set(names) == set(K.EXPORTED)


def test_kv_bytes_matches_formula_and_oracle():
    p = K.make_params(64, 64, 8, 32768, "fp16", 64, "none")
    assert K.kvq_kv_bytes(p, 80, 1) == 327680
    assert K.kvq_kv_bytes(p, 1, 64 * 32768) == 8589934592
    for fmt, g, out in [("int4", 32, "fp16"), ("fp4", 32, "fp16"), ("c2", 64, "e4m3")]:
        p = K.make_params(4, 32, 8, 1000, fmt, g, out)
        for L, T, n in [(1, 1, 0), (80, 12345, 678), (3, 7, 1)]:
            assert K.kvq_kv_bytes(p, L, T, n) == KB.kv_bytes(fmt, L, 8, 128, T, g, n, out)


def test_cache_sizes_and_workspace():
    p = K.make_params(64, 64, 8, 32768, "c2", 64, "e4m3")
    s = K.kvq_cache_sizes(p, 100)
    assert (s.code_bytes_per_row, s.meta_bytes_per_row) == (32, 16)
    assert s.codes == 64 * 8 * 32768 * 32 and s.meta == 64 * 8 * 32768 * 16
    assert s.outl_idx == 64 * 8 * 100 * 4 and s.outl_val == 64 * 8 * 100
    assert s.outl_block_start == 64 * 8 * 2 * 2048 * 4
    # MFMA decoder: two partial slots of Hq / H = 8 query heads and a 32-byte merge descriptor
    # per workgroup; 256 workgroups by default, one per 2048 tokens of all lists with a split
    assert K.kvq_workspace_bytes(p) == 256 * (2 * 8 * 130 * 4 + 32)
    assert K.kvq_workspace_bytes(p, 2048) == (64 * 8 * 32768 // 2048) * (2 * 8 * 130 * 4 + 32)
    # default split of formats on the generic decoder: 64-token chunks for a short context
    pi = K.make_params(1, 8, 2, 1024, "int4", 32, "fp16")
    assert K.kvq_workspace_bytes(pi) == 1 * 8 * 16 * 130 * 4
    # FP4 g32 (MFMA decoder): 256 workgroups
    assert K.kvq_workspace_bytes(K.make_params(4, 64, 8, 131072, "fp4", 32, "fp16")) == 256 * (2 * 8 * 130 * 4 + 32)
    # few steps: at least 12 per workgroup (1 x 2 lists of 32 steps -> 6 workgroups)
    assert K.kvq_workspace_bytes(K.make_params(1, 8, 2, 1024, "c2", 64, "e4m3")) == 6 * (2 * 4 * 130 * 4 + 32)
    p4 = K.make_params(4, 64, 8, 131072, "fp4", 32, "fp16")
    s4 = K.kvq_cache_sizes(p4, 10)
    assert (s4.code_bytes_per_row, s4.meta_bytes_per_row) == (64, 4)
    pp = K.make_params(2, 8, 2, 100, "c2", 64, "e4m3", page_size=16, num_pages=9,
                       num_pages_fp8=4, max_pages_per_seq=7)
    sp = K.kvq_cache_sizes(pp, 10)
    assert sp.codes == 9 * 2 * 16 * 32 and sp.codes8 == 4 * 2 * 16 * 128 and sp.scale8 == 4 * 2 * 16 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), K.KVQ_ERR_UNSUPPORTED),
    (dict(Hq=12, H=8), K.KVQ_ERR_INVALID_ARG),
    (dict(Hq=64, H=2), K.KVQ_ERR_UNSUPPORTED),            # GQA group of 32
    (dict(group=48), K.KVQ_ERR_UNSUPPORTED),
    (dict(fmt="c2", group=32), K.KVQ_ERR_UNSUPPORTED),
    (dict(S_cap=0), K.KVQ_ERR_INVALID_ARG),
    (dict(sigma=0.0), K.KVQ_ERR_INVALID_ARG),
    (dict(sigma=float("nan")), K.KVQ_ERR_INVALID_ARG),
    (dict(fmt="fp16"), K.KVQ_ERR_UNSUPPORTED),
])
def test_invalid_params_rejected(kw, status):
    base = dict(B=2, Hq=8, H=2, S_cap=100, fmt="c2", group=64, outlier="e4m3", sigma=3.0, D=128)
    base.update(kw)
    p = K.make_params(base["B"], base["Hq"], base["H"], base["S_cap"], base["fmt"],
                      base["group"], base["outlier"], base["sigma"], D=base["D"])
    with pytest.raises(K.KvqError) as e:
        K.kvq_workspace_bytes(p)
    assert e.value.status == status


def test_paged_params_validation():
    bad = K.make_params(2, 8, 2, 100, "c2", 64, "e4m3", page_size=16, num_pages=9,
                        num_pages_fp8=4, max_pages_per_seq=6)          # 6 * 16 < 100
    with pytest.raises(K.KvqError):
        K.kvq_workspace_bytes(bad)
    bad = K.make_params(2, 8, 2, 100, "int4", 32, "fp16", page_size=16, num_pages=9,
                        max_pages_per_seq=7)                             # paged tier 2 is 2-bit only
    with pytest.raises(K.KvqError):
        K.kvq_workspace_bytes(bad)
    bad = K.make_params(2, 8, 2, 100, "c2", 64, "e4m3", page_size=32, max_pages_per_seq=7)
    with pytest.raises(K.KvqError):
        K.kvq_workspace_bytes(bad)


def test_split_chunk_must_be_multiple_of_64():
    p = K.make_params(2, 8, 2, 1000, "c2", 64, "e4m3")
    assert K.kvq_workspace_bytes(p, 128) == (2 * 2 * 1000 + 127) // 128 * (2 * 4 * 130 * 4 + 32)
    with pytest.raises(K.KvqError):
        K.kvq_workspace_bytes(p, 100)


def test_null_pointers_rejected_before_launch():
    p = K.make_params(2, 8, 2, 100, "c2", 64, "e4m3")
    c = K.kvq_cache()
    st = K._lib.kvq_decode_attention(K.C.byref(p), K.C.byref(c), None, None, None, 0.1, 0,
                                     None, None, 0, None)
    assert st == K.KVQ_ERR_INVALID_ARG
    st = K._lib.kvq_quantize_append(K.C.byref(p), K.C.byref(c), None, None, 1, None, None, None,
                                    None)
    assert st == K.KVQ_ERR_INVALID_ARG


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert K.kvq_status_string(s) != "unknown status"


def test_format_variants_size_and_check_like_their_base():
    # uniform 2-bit is laid out as CENTROID2, symmetric INT4 as INT4_ASYM
    for var, base, g, out in [("u2", "c2", 64, "e4m3"), ("int4s", "int4", 32, "fp16"),
                              ("int4s", "int4", 64, "none")]:
        pv = K.make_params(4, 32, 8, 1000, var, g, out)
        pb = K.make_params(4, 32, 8, 1000, base, g, out)
        sv, sb = K.kvq_cache_sizes(pv, 50), K.kvq_cache_sizes(pb, 50)
        assert (sv.code_bytes_per_row, sv.meta_bytes_per_row, sv.codes, sv.meta, sv.outl_val) == \
               (sb.code_bytes_per_row, sb.meta_bytes_per_row, sb.codes, sb.meta, sb.outl_val)
        assert K.kvq_workspace_bytes(pv) == K.kvq_workspace_bytes(pb)
        for L, T, n in [(1, 1, 0), (80, 12345, 678 if out != "none" else 0)]:
            assert K.kvq_kv_bytes(pv, L, T, n) == KB.kv_bytes(var, L, 8, 128, T, g, n, out)
    with pytest.raises(K.KvqError) as e:                       # uniform 2-bit: groups of 64 only
        K.kvq_workspace_bytes(K.make_params(2, 8, 2, 100, "u2", 32, "e4m3"))
    assert e.value.status == K.KVQ_ERR_UNSUPPORTED
    with pytest.raises(K.KvqError) as e:                       # variants: contiguous caches only
        K.kvq_workspace_bytes(K.make_params(2, 8, 2, 100, "u2", 64, "e4m3", page_size=16,
                                            num_pages=9, num_pages_fp8=4, max_pages_per_seq=7))
    assert e.value.status == K.KVQ_ERR_UNSUPPORTED


def test_int3_sizes_and_checks():
    # 3-bit codes: 48 bytes per 128-channel row, fp16 scale and zero per group; contiguous only
    for g, out in [(32, "e4m3"), (64, "fp16"), (32, "none")]:
        p = K.make_params(4, 32, 8, 1000, "int3", g, out)
        s = K.kvq_cache_sizes(p, 50)
        assert (s.code_bytes_per_row, s.meta_bytes_per_row) == (48, (128 // g) * 4)
        assert s.codes == 4 * 8 * 1000 * 48
        for L, T, n in [(1, 1, 0), (80, 12345, 678 if out != "none" else 0)]:
            assert K.kvq_kv_bytes(p, L, T, n) == KB.kv_bytes("int3", L, 8, 128, T, g, n, out)
        assert K.kvq_workspace_bytes(p) == K.kvq_workspace_bytes(K.make_params(4, 32, 8, 1000, "int4", g, out))
    with pytest.raises(K.KvqError) as e:
        K.kvq_workspace_bytes(K.make_params(2, 8, 2, 100, "int3", 16, "e4m3"))
    assert e.value.status == K.KVQ_ERR_UNSUPPORTED
    with pytest.raises(K.KvqError) as e:
        K.kvq_workspace_bytes(K.make_params(2, 8, 2, 100, "int3", 32, "e4m3", page_size=16,
                                            num_pages=9, num_pages_fp8=4, max_pages_per_seq=7))
    assert e.value.status == K.KVQ_ERR_UNSUPPORTED


def test_kv_bytes_rounds_packed_codes_up_to_whole_bytes():
    # 20 channels: 3-bit codes are 60 bits -> 8 bytes, 2-bit 40 bits -> 5, 4-bit 80 bits -> 10;
    # plus the per-group metadata of 5 groups of 4 (4 B INT3 / INT4, 8 B 2-bit)
    for fmt, row in (("int3", 8 + 5 * 4), ("c2", 5 + 5 * 8), ("int4", 10 + 5 * 4)):
        p = K.make_params(1, 2, 2, 16, fmt, 4, "none", D=20)
        assert K.kvq_kv_bytes(p, 1, 3) == 2 * 2 * 3 * row
        assert KB.kv_bytes(fmt, 1, 2, 20, 3, 4) == 2 * 2 * 3 * row
    p = K.make_params(1, 2, 2, 16, "int3", 7, "none", D=21)      # 63 bits -> 8 bytes
    assert K.kvq_kv_bytes(p, 1, 1) == 2 * 2 * (8 + 3 * 4)


def test_channel_mask_needs_an_outlier_dtype():
    import ctypes as C
    import numpy as np
    p = K.make_params(1, 4, 1, 64, "int4", 32, "none")
    c = K.kvq_cache()
    buf = (C.c_uint8 * 64)()
    for kv in range(2):
        c.codes[kv] = c.meta[kv] = C.cast(buf, C.c_void_p)
    c.outl_count = c.outl_block_start = C.cast(buf, C.c_void_p)
    mask = np.zeros(8, np.uint32)
    c.chan_mask = mask.ctypes.data
    st = K._lib.kvq_quantize_append(C.byref(p), C.byref(c), C.cast(buf, C.c_void_p), C.cast(buf, C.c_void_p),
                                    1, C.cast(buf, C.c_void_p), C.cast(buf, C.c_void_p), None, None)
    assert st == K.KVQ_ERR_INVALID_ARG


def _fake_cache(nbytes=256):
    """A kvq_cache whose pointers are host memory: only for calls that the host checks reject
    before any launch."""
    import ctypes as C
    buf = (C.c_uint8 * nbytes)()
    c = K.kvq_cache()
    ptr = C.cast(buf, C.c_void_p)
    for kv in range(2):
        c.codes[kv] = c.meta[kv] = c.outl_idx[kv] = c.outl_val[kv] = ptr
    c.outl_count = c.outl_block_start = c.status = ptr
    c.outl_capacity = 8
    return c, buf, ptr


def test_decode_host_checks_reject_before_launch():
    import ctypes as C
    c, buf, ptr = _fake_cache()
    p = K.make_params(2, 8, 2, 1000, "c2", 64, "e4m3")
    dec = K._lib.kvq_decode_attention
    # split into chunks of 128 tokens needs a workspace: none, then one byte too small
    need = K.kvq_workspace_bytes(p, 128)
    assert need > 0
    assert dec(C.byref(p), C.byref(c), ptr, ptr, None, C.c_float(0.1), 128, ptr, None, 0, None) \
        == K.KVQ_ERR_WORKSPACE
    assert dec(C.byref(p), C.byref(c), ptr, ptr, None, C.c_float(0.1), 128, ptr, ptr, need - 1, None) \
        == K.KVQ_ERR_WORKSPACE
    # split chunk not a multiple of 64, non-finite softmax scale, missing query / output
    assert dec(C.byref(p), C.byref(c), ptr, ptr, None, C.c_float(0.1), 100, ptr, ptr, need, None) \
        == K.KVQ_ERR_INVALID_ARG
    assert dec(C.byref(p), C.byref(c), ptr, ptr, None, C.c_float(float("inf")), 0, ptr, ptr, need, None) \
        == K.KVQ_ERR_INVALID_ARG
    assert dec(C.byref(p), C.byref(c), None, ptr, None, C.c_float(0.1), 0, ptr, ptr, need, None) \
        == K.KVQ_ERR_INVALID_ARG
    assert dec(C.byref(p), C.byref(c), ptr, ptr, None, C.c_float(0.1), 0, None, ptr, need, None) \
        == K.KVQ_ERR_INVALID_ARG
    # a paged cache needs its block table
    pp = K.make_params(2, 8, 2, 100, "c2", 64, "e4m3", page_size=16, num_pages=9,
                       num_pages_fp8=0, max_pages_per_seq=7)
    assert dec(C.byref(pp), C.byref(c), ptr, ptr, None, C.c_float(0.1), 0, ptr, ptr, 1 << 20, None) \
        == K.KVQ_ERR_INVALID_ARG


def test_append_host_checks_reject_before_launch():
    import ctypes as C
    c, buf, ptr = _fake_cache()
    p = K.make_params(2, 8, 2, 1000, "int4", 32, "fp16")
    app = K._lib.kvq_quantize_append
    assert app(C.byref(p), C.byref(c), ptr, ptr, 0, ptr, ptr, None, None) == K.KVQ_ERR_INVALID_ARG
    assert app(C.byref(p), C.byref(c), None, ptr, 1, ptr, ptr, None, None) == K.KVQ_ERR_INVALID_ARG
    c.outl_capacity = (1 << 28) + 1                            # record offsets are 32-bit
    assert app(C.byref(p), C.byref(c), ptr, ptr, 1, ptr, ptr, None, None) == K.KVQ_ERR_INVALID_ARG
