"""Python binding of libkvq.so (quantized-KV decode attention for MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of libkvq.so.  The
functions below carry the names of the C entry points declared in ``include/kvq.h``; PyTorch is
used for device memory and the current HIP stream.  Importing this package raises if the
library has not been built (``python decode_attention_sub_amd/build.py``); there is no CPU
fallback.
"""

from __future__ import annotations

import ctypes as C
import math
import os
from dataclasses import dataclass, field
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK, KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED = 0, -1, -2
KVQ_ERR_WORKSPACE, KVQ_ERR_HIP, KVQ_ERR_CAPACITY = -3, -4, -5
FMT = {"fp16": 0, "fp8row": 1, "int4": 2, "fp4": 3, "c2": 4, "bf16": 5, "u2": 6, "int4s": 7,
       "int3": 8}
OUTL = {"none": 0, "fp16": 1, "e4m3": 2}

EXPORTED = ("kvq_kv_bytes", "kvq_cache_sizes", "kvq_quantize_append", "kvq_workspace_bytes",
            "kvq_decode_attention", "kvq_decode_attention_noalloc", "kvq_append_decode",
            "kvq_mass_workspace_bytes",
            "kvq_decode_attention_mass", "kvq_retier_workspace_bytes", "kvq_retier",
            "kvq_prologue_workspace_bytes", "kvq_prologue_pack_weights", "kvq_attention_prologue",
            "kvq_probe_read", "kvq_probe_copy", "kvq_status_string")
NOALLOC_SCRATCH_BYTES = 32 << 20   # KVQ_NOALLOC_SCRATCH_BYTES


class kvq_params(C.Structure):
    _fields_ = [("batch", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("max_seq_len", C.c_int32), ("format", C.c_int32),
                ("group_size", C.c_int32), ("outlier_dtype", C.c_int32),
                ("outlier_sigma", C.c_float), ("lloyd_iters", C.c_int32),
                ("page_size", C.c_int32), ("num_pages", C.c_int32),
                ("num_pages_fp8", C.c_int32), ("max_pages_per_seq", C.c_int32)]


class kvq_cache(C.Structure):
    _fields_ = [("codes", C.c_void_p * 2), ("meta", C.c_void_p * 2), ("codes8", C.c_void_p * 2),
                ("scale8", C.c_void_p * 2), ("outl_idx", C.c_void_p * 2),
                ("outl_val", C.c_void_p * 2), ("outl_count", C.c_void_p),
                ("outl_block_start", C.c_void_p), ("outl_capacity", C.c_int64),
                ("status", C.c_void_p), ("chan_mask", C.c_void_p)]


class kvq_cache_sizes_t(C.Structure):
    _fields_ = [("codes", C.c_uint64), ("meta", C.c_uint64), ("codes8", C.c_uint64),
                ("scale8", C.c_uint64), ("outl_idx", C.c_uint64), ("outl_val", C.c_uint64),
                ("outl_count", C.c_uint64), ("outl_block_start", C.c_uint64),
                ("code_bytes_per_row", C.c_uint32), ("meta_bytes_per_row", C.c_uint32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with decode_attention_sub_amd/build.py")
    # torch ships its own HIP runtime and asks for it by a different name than this library does;
    # loading torch first makes the library bind to that same runtime.  Loaded the other way
    # round, the process holds two runtimes and torch's streams are foreign to the library.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    P, Pc, vp = C.POINTER(kvq_params), C.POINTER(kvq_cache), C.c_void_p
    sig = {
        "kvq_kv_bytes": (C.c_int32, [P, C.c_int32, C.c_int64, C.c_int64, C.POINTER(C.c_uint64)]),
        "kvq_cache_sizes": (C.c_int32, [P, C.c_int64, C.POINTER(kvq_cache_sizes_t)]),
        "kvq_quantize_append": (C.c_int32, [P, Pc, vp, vp, C.c_int32, vp, vp, vp, vp]),
        "kvq_workspace_bytes": (C.c_int32, [P, C.c_int32, C.POINTER(C.c_uint64)]),
        "kvq_decode_attention": (C.c_int32, [P, Pc, vp, vp, vp, C.c_float, C.c_int32, vp, vp,
                                             C.c_uint64, vp]),
        "kvq_decode_attention_noalloc": (C.c_int32, [P, Pc, vp, vp, vp, C.c_float, C.c_int32,
                                                     vp, vp]),
        "kvq_append_decode": (C.c_int32, [P, Pc, vp, vp, vp, vp, C.c_float, C.c_int32, vp, vp,
                                          C.c_uint64, vp]),
        "kvq_mass_workspace_bytes": (C.c_int32, [P, C.c_int32, C.POINTER(C.c_uint64)]),
        "kvq_decode_attention_mass": (C.c_int32, [P, Pc, vp, vp, vp, C.c_float, C.c_int32, vp, vp,
                                                  vp, C.c_uint64, vp]),
        "kvq_retier_workspace_bytes": (C.c_int32, [P, C.c_int32, C.POINTER(C.c_uint64)]),
        "kvq_retier": (C.c_int32, [P, Pc, vp, vp, vp, C.c_float, vp, C.c_int32, vp, vp, vp,
                                   C.c_uint64, vp]),
        "kvq_prologue_workspace_bytes": (C.c_int32, [P, C.c_int32, C.POINTER(C.c_uint64)]),
        "kvq_prologue_pack_weights": (C.c_int32, [P, C.c_int32, vp, vp, vp]),
        "kvq_attention_prologue": (C.c_int32, [P, Pc, vp, vp, vp, C.c_int32, C.c_float, vp, vp, vp,
                                               vp, vp, C.c_uint64, vp]),
        "kvq_probe_read": (C.c_int32, [vp, C.c_uint64, vp, vp]),
        "kvq_probe_copy": (C.c_int32, [vp, vp, C.c_uint64, vp]),
        "kvq_status_string": (C.c_char_p, [C.c_int32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {kvq_status_string(status)} ({status})")
        self.status = status


def _check(st: int, what: str):
    if st != KVQ_OK:
        raise KvqError(st, what)


def kvq_status_string(status: int) -> str:
    return _lib.kvq_status_string(status).decode()


def make_params(B, Hq, H, S_cap, fmt, group, outlier, sigma=3.0, lloyd_iters=8, D=128,
                page_size=0, num_pages=0, num_pages_fp8=0, max_pages_per_seq=0) -> kvq_params:
    return kvq_params(B, Hq, H, D, S_cap, FMT[fmt], group, OUTL[outlier], sigma, lloyd_iters,
                      page_size, num_pages, num_pages_fp8, max_pages_per_seq)


def kvq_kv_bytes(p: kvq_params, num_layers: int, num_tokens: int, num_outliers: int = 0) -> int:
    out = C.c_uint64()
    _check(_lib.kvq_kv_bytes(C.byref(p), num_layers, num_tokens, num_outliers, C.byref(out)),
           "kvq_kv_bytes")
    return out.value


def kvq_cache_sizes(p: kvq_params, outl_capacity: int) -> kvq_cache_sizes_t:
    out = kvq_cache_sizes_t()
    _check(_lib.kvq_cache_sizes(C.byref(p), outl_capacity, C.byref(out)), "kvq_cache_sizes")
    return out


def kvq_workspace_bytes(p: kvq_params, split_chunk: int = 0) -> int:
    out = C.c_uint64()
    _check(_lib.kvq_workspace_bytes(C.byref(p), split_chunk, C.byref(out)), "kvq_workspace_bytes")
    return out.value


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


@dataclass
class KVCache:
    """Device buffers of one cache layer (torch tensors as plain allocations) and the
    kvq_cache struct that points at them."""
    params: kvq_params
    outl_capacity: int
    tensors: dict = field(default_factory=dict)
    struct: kvq_cache = None

    @classmethod
    def allocate(cls, p: kvq_params, outl_capacity: int, device="cuda", chan_mask=None):
        """chan_mask: None, or a static channel mask as int32 [2, H, 4] (device) words."""
        import torch
        sz = kvq_cache_sizes(p, outl_capacity)
        u8 = dict(dtype=torch.uint8, device=device)
        t = {}
        for kv in (0, 1):
            t[f"codes{kv}"] = torch.empty(max(sz.codes, 1), **u8)
            t[f"meta{kv}"] = torch.empty(max(sz.meta, 1), **u8)
            t[f"codes8_{kv}"] = torch.empty(max(sz.codes8, 1), **u8) if p.page_size else None
            t[f"scale8_{kv}"] = (torch.empty(max(sz.scale8 // 4, 1), dtype=torch.float32,
                                             device=device) if p.page_size else None)
            t[f"idx{kv}"] = torch.empty(max(sz.outl_idx // 4, 1), dtype=torch.int32, device=device)
            t[f"val{kv}"] = torch.empty(max(sz.outl_val, 1), **u8)
        t["count"] = torch.zeros(sz.outl_count // 4, dtype=torch.int32, device=device)
        t["bstart"] = torch.zeros(sz.outl_block_start // 4, dtype=torch.int32, device=device)
        t["status"] = torch.zeros(1, dtype=torch.int32, device=device)
        if chan_mask is not None:
            assert chan_mask.dtype == torch.int32 and chan_mask.is_contiguous()
            assert tuple(chan_mask.shape) == (2, p.num_kv_heads, 4)
        t["chan_mask"] = chan_mask
        c = cls(p, outl_capacity, t)
        c.struct = kvq_cache(
            (C.c_void_p * 2)(_ptr(t["codes0"]), _ptr(t["codes1"])),
            (C.c_void_p * 2)(_ptr(t["meta0"]), _ptr(t["meta1"])),
            (C.c_void_p * 2)(_ptr(t["codes8_0"]), _ptr(t["codes8_1"])),
            (C.c_void_p * 2)(_ptr(t["scale8_0"]), _ptr(t["scale8_1"])),
            (C.c_void_p * 2)(_ptr(t["idx0"]), _ptr(t["idx1"])),
            (C.c_void_p * 2)(_ptr(t["val0"]), _ptr(t["val1"])),
            _ptr(t["count"]), _ptr(t["bstart"]), outl_capacity, _ptr(t["status"]),
            _ptr(chan_mask))
        return c

    def status(self) -> int:
        return int(self.tensors["status"].item())


def kvq_quantize_append(p: kvq_params, cache: KVCache, k_new, v_new, positions, counts,
                        block_table=None, stream=None):
    """k_new, v_new: float32 [B, H, max_new, D] (device, contiguous); positions, counts: int32
    [B] (device)."""
    assert k_new.is_contiguous() and v_new.is_contiguous()
    max_new = k_new.shape[2]
    _check(_lib.kvq_quantize_append(C.byref(p), C.byref(cache.struct), _ptr(k_new), _ptr(v_new),
                                    max_new, _ptr(positions), _ptr(counts), _ptr(block_table),
                                    _stream(stream)), "kvq_quantize_append")


def kvq_decode_attention(p: kvq_params, cache: KVCache, q_bf16, seq_lens, out, workspace=None,
                         block_table=None, sm_scale: Optional[float] = None, split_chunk: int = 0,
                         stream=None):
    """q_bf16: bfloat16 [B, Hq, D]; seq_lens: int32 [B]; out: float32 [B, Hq, D] (all device).
    sm_scale None passes NaN, which the library reads as its default 1/sqrt(head_dim)."""
    if sm_scale is None:
        sm_scale = math.nan
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.kvq_decode_attention(C.byref(p), C.byref(cache.struct), _ptr(q_bf16),
                                     _ptr(seq_lens), _ptr(block_table), sm_scale, split_chunk,
                                     _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)),
           "kvq_decode_attention")


def kvq_append_decode(p: kvq_params, cache: KVCache, k_new, v_new, q_bf16, seq_lens, out,
                      workspace=None, sm_scale: Optional[float] = None, split_chunk: int = 0,
                      stream=None):
    """One decode step with the append fused: k_new, v_new float32 [B, H, D] (device) are
    appended at token seq_lens[b] - 1, then attention over seq_lens as kvq_decode_attention."""
    if sm_scale is None:
        sm_scale = math.nan
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.kvq_append_decode(C.byref(p), C.byref(cache.struct), _ptr(k_new), _ptr(v_new),
                                  _ptr(q_bf16), _ptr(seq_lens), sm_scale, split_chunk, _ptr(out),
                                  _ptr(workspace), ws_bytes, _stream(stream)),
           "kvq_append_decode")


def kvq_decode_attention_noalloc(p: kvq_params, cache: KVCache, q_bf16, seq_lens, out,
                                 block_table=None, sm_scale: Optional[float] = None,
                                 split_chunk: int = 0, stream=None):
    """kvq_decode_attention without a workspace: the split-K partials live in the library's
    per-GPU scratch array (at most NOALLOC_SCRATCH_BYTES); nothing is allocated."""
    if sm_scale is None:
        sm_scale = math.nan
    _check(_lib.kvq_decode_attention_noalloc(C.byref(p), C.byref(cache.struct), _ptr(q_bf16),
                                             _ptr(seq_lens), _ptr(block_table), sm_scale,
                                             split_chunk, _ptr(out), _stream(stream)),
           "kvq_decode_attention_noalloc")


def kvq_mass_workspace_bytes(p: kvq_params, split_chunk: int = 0) -> int:
    out = C.c_uint64()
    _check(_lib.kvq_mass_workspace_bytes(C.byref(p), split_chunk, C.byref(out)),
           "kvq_mass_workspace_bytes")
    return out.value


def kvq_decode_attention_mass(p: kvq_params, cache: KVCache, q_bf16, seq_lens, out, page_mass,
                              workspace, block_table, sm_scale: Optional[float] = None,
                              split_chunk: int = 0, stream=None):
    """kvq_decode_attention of a paged cache that also writes page_mass: float32 [B,
    max_pages_per_seq] (device), the attention mass of every page."""
    if sm_scale is None:
        sm_scale = math.nan
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.kvq_decode_attention_mass(C.byref(p), C.byref(cache.struct), _ptr(q_bf16),
                                          _ptr(seq_lens), _ptr(block_table), sm_scale,
                                          split_chunk, _ptr(out), _ptr(page_mass),
                                          _ptr(workspace), ws_bytes, _stream(stream)),
           "kvq_decode_attention_mass")


def kvq_retier_workspace_bytes(p: kvq_params, n_free: int) -> int:
    out = C.c_uint64()
    _check(_lib.kvq_retier_workspace_bytes(C.byref(p), n_free, C.byref(out)),
           "kvq_retier_workspace_bytes")
    return out.value


def kvq_retier(p: kvq_params, cache: KVCache, block_table, seq_lens, page_mass, keep_frac: float,
               free_slots, freed_slots, n_moved, workspace, stream=None):
    """Move the cold FP8 pages to the 2-bit tier.  block_table int32 [B, max_pages] (device,
    rewritten); free_slots int32 [n_free] (device); freed_slots int32 (device, capacity
    min(n_free, num_pages_fp8)); n_moved int32 [1] (device)."""
    n_free = 0 if free_slots is None else free_slots.numel()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.kvq_retier(C.byref(p), C.byref(cache.struct), _ptr(block_table), _ptr(seq_lens),
                           _ptr(page_mass), keep_frac, _ptr(free_slots), n_free,
                           _ptr(freed_slots), _ptr(n_moved), _ptr(workspace), ws_bytes,
                           _stream(stream)), "kvq_retier")


def kvq_prologue_workspace_bytes(p: kvq_params, d_model: int) -> int:
    n = C.c_uint64(0)
    _check(_lib.kvq_prologue_workspace_bytes(C.byref(p), d_model, C.byref(n)),
           "kvq_prologue_workspace_bytes")
    return n.value


def kvq_prologue_pack_weights(p: kvq_params, weight_bf16, packed, stream=None):
    """weight_bf16: row-major [(Hq + 2H) * D, d] 16-bit tensor; packed: a distinct tensor of the
    same size receiving the block order kvq_attention_prologue reads (both device)."""
    d_model = weight_bf16.shape[-1]
    assert packed.numel() * packed.element_size() == weight_bf16.numel() * weight_bf16.element_size()
    _check(_lib.kvq_prologue_pack_weights(C.byref(p), d_model, _ptr(weight_bf16), _ptr(packed),
                                          _stream(stream)), "kvq_prologue_pack_weights")


def kvq_attention_prologue(p: kvq_params, cache: KVCache, hidden_bf16, gain_bf16, weight_packed,
                           eps: float, positions, q_out, workspace, block_table=None,
                           proj_out=None, stream=None):
    """hidden_bf16: bfloat16 [B, d]; gain_bf16: [d]; weight_packed: the projection packed by
    kvq_prologue_pack_weights; positions: int32 [B]; q_out: bfloat16 [B, Hq, D]; proj_out:
    optional float32 [B, (Hq + 2H) * D]; workspace: zero-filled before its first use (all
    device)."""
    d_model = hidden_bf16.shape[-1]
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.kvq_attention_prologue(C.byref(p), C.byref(cache.struct), _ptr(hidden_bf16),
                                       _ptr(gain_bf16), _ptr(weight_packed), d_model, float(eps),
                                       _ptr(positions), _ptr(block_table), _ptr(q_out),
                                       _ptr(proj_out), _ptr(workspace), ws_bytes, _stream(stream)),
           "kvq_attention_prologue")


def kvq_probe_read(src, sink, stream=None):
    _check(_lib.kvq_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                               _stream(stream)), "kvq_probe_read")


def kvq_probe_copy(src, dst, stream=None):
    _check(_lib.kvq_probe_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(),
                               _stream(stream)), "kvq_probe_copy")
