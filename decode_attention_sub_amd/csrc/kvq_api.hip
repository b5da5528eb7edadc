// C ABI of libkvq.so: argument validation, buffer sizing and kernel launches.
// The contract of every entry point is documented in include/kvq.h.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "kvq_device.h"
#include "kvq_launch.h"

using namespace kvq;

namespace {

constexpr int kDefaultPagedChunk = 4096;

bool is_quant_fmt(int f) { return f == FMT_INT4 || f == FMT_FP4 || f == FMT_C2 || f == FMT_INT3; }

// A format variant is checked, sized, stored and decoded as its base format; only the
// quantizer's fit differs.  Entry points work on a copy whose format is the base format.
struct Params {
  kvq_params p;
  int fit;
  explicit Params(const kvq_params* in) : p(in ? *in : kvq_params{}), fit(in ? fit_of(in->format) : 0) {
    p.format = storage_fmt(p.format);
  }
};

int32_t check_params(const kvq_params* p) {
  if (!p) return KVQ_ERR_INVALID_ARG;
  if (p->format == KVQ_FMT_UNIFORM2 || p->format == KVQ_FMT_INT4_SYM) {
    if (p->page_size != 0) return KVQ_ERR_UNSUPPORTED;
    const Params n(p);
    return check_params(&n.p);
  }
  if (p->batch < 1 || p->num_kv_heads < 1 || p->num_q_heads < 1 || p->max_seq_len < 1)
    return KVQ_ERR_INVALID_ARG;
  if (p->head_dim != kHeadDim) return KVQ_ERR_UNSUPPORTED;
  if (p->num_q_heads % p->num_kv_heads != 0) return KVQ_ERR_INVALID_ARG;
  const int G = p->num_q_heads / p->num_kv_heads;
  if (G > 16) return KVQ_ERR_UNSUPPORTED;
  if (!is_quant_fmt(p->format)) return KVQ_ERR_UNSUPPORTED;
  if (p->group_size != 32 && p->group_size != 64) return KVQ_ERR_UNSUPPORTED;
  if (p->format == FMT_C2 && p->group_size != 64) return KVQ_ERR_UNSUPPORTED;
  if (p->outlier_dtype < KVQ_OUTL_NONE || p->outlier_dtype > KVQ_OUTL_FP8_E4M3)
    return KVQ_ERR_INVALID_ARG;
  if (p->outlier_dtype != KVQ_OUTL_NONE && !(p->outlier_sigma > 0.0f && isfinite(p->outlier_sigma)))
    return KVQ_ERR_INVALID_ARG;
  if (p->format == FMT_C2 && (p->lloyd_iters < 0 || p->lloyd_iters > 64)) return KVQ_ERR_INVALID_ARG;
  if (p->page_size != 0 && p->page_size != kBlock) return KVQ_ERR_UNSUPPORTED;
  if (p->page_size) {
    if (p->format != FMT_C2) return KVQ_ERR_UNSUPPORTED;
    if (p->num_pages < 0 || p->num_pages_fp8 < 0 || p->max_pages_per_seq < 1) return KVQ_ERR_INVALID_ARG;
    if ((int64_t)p->max_pages_per_seq * kBlock < p->max_seq_len) return KVQ_ERR_INVALID_ARG;
  }
  if ((int64_t)p->max_seq_len * kHeadDim > 0xFFFFFFFFll) return KVQ_ERR_INVALID_ARG;  // uint32 index
  return KVQ_OK;
}

uint32_t code_bytes(const kvq_params* p) { return kHeadDim * code_bits(p->format) / 8; }
uint32_t meta_bytes(const kvq_params* p) {
  return (kHeadDim / p->group_size) * meta_bytes_per_group(p->format);
}

Layout make_layout(const kvq_params* p, int64_t outl_cap) {
  Layout L;
  L.B = p->batch;
  L.H = p->num_kv_heads;
  L.S_cap = p->max_seq_len;
  L.paged = p->page_size ? 1 : 0;
  L.max_pages = p->max_pages_per_seq;
  L.code_bytes = (int)code_bytes(p);
  L.meta_bytes = (int)meta_bytes(p);
  L.nblk = (p->max_seq_len + kBlock - 1) / kBlock;
  L.outl_cap = outl_cap;
  L.num_pages = p->page_size ? p->num_pages : 0;
  L.num_pages_fp8 = p->page_size ? p->num_pages_fp8 : 0;
  return L;
}

int32_t check_cache(const kvq_params* p, const kvq_cache* c) {
  if (!c) return KVQ_ERR_INVALID_ARG;
  for (int kv = 0; kv < 2; ++kv) {
    if (!c->codes[kv] || !c->meta[kv]) return KVQ_ERR_INVALID_ARG;
    if (p->page_size && p->num_pages_fp8 > 0 && (!c->codes8[kv] || !c->scale8[kv]))
      return KVQ_ERR_INVALID_ARG;
    if (p->outlier_dtype != KVQ_OUTL_NONE && (!c->outl_idx[kv] || !c->outl_val[kv]))
      return KVQ_ERR_INVALID_ARG;
  }
  if (!c->outl_count || !c->outl_block_start) return KVQ_ERR_INVALID_ARG;
  if (p->outlier_dtype != KVQ_OUTL_NONE && c->outl_capacity < 1) return KVQ_ERR_INVALID_ARG;
  if (c->chan_mask && p->outlier_dtype == KVQ_OUTL_NONE) return KVQ_ERR_INVALID_ARG;
  if (c->outl_capacity > (int64_t(1) << 28)) return KVQ_ERR_INVALID_ARG;  // 32-bit record offsets
  return KVQ_OK;
}

// Default split.  Formats on the MFMA decoder (2-bit, FP4 with groups of 32): enough
// (sequence, KV head, chunk) units for one workgroup per CU of an MI355X (256), never chunks
// shorter than 512 tokens (each wave keeps a run of steps).  Formats on the generic decoder
// (INT4, FP4 with groups of 64): its 4-wave workgroups take one 64-token step at a time, so
// short contexts are split down to 64-token chunks across ~1024 units (latency).
int resolve_chunk(const kvq_params* p, int32_t split_chunk) {
  if (split_chunk < 0) return -1;
  if (split_chunk == 0) {
    if (p->page_size) return kDefaultPagedChunk;
    const bool mfma = p->format == FMT_C2 || (p->format == FMT_FP4 && p->group_size == 32);
    const int64_t units = (int64_t)p->batch * p->num_kv_heads;
    const int64_t want = mfma ? 256 : 1024;
    const int64_t min_chunk = mfma ? 512 : 64;
    int64_t nchunks = units >= want ? 1 : (want + units - 1) / units;
    int64_t chunk = (p->max_seq_len + nchunks - 1) / nchunks;
    chunk = chunk < min_chunk ? min_chunk : chunk;
    return (int)(((chunk + 63) / 64) * 64);
  }
  if (split_chunk % 64) return -1;
  return split_chunk;
}


// Workgroups of the MFMA decoder, which share the 32-token steps of all lists evenly: one per CU
// of an MI355X (256, one resident workgroup each) by default, never fewer than 12 steps (one per
// wave) each at max_seq_len; with a split, about one per split_chunk tokens of all lists at
// max_seq_len (at most kMaxDecodeWGs).
constexpr int64_t kDecodeWGs = 256;
constexpr int64_t kMaxDecodeWGs = 16384;
bool mfma_format(const kvq_params* p) {
  return mfma_decodes(p->format, p->group_size, p->page_size != 0, p->num_pages, p->num_pages_fp8,
                      p->num_kv_heads);
}
int64_t decode_wgs(const kvq_params* p, int32_t split_chunk) {
  const int64_t lists = (int64_t)p->batch * p->num_kv_heads;
  const int64_t steps = lists * ((p->max_seq_len + 31) / 32);
  int64_t n = split_chunk > 0 ? (lists * p->max_seq_len + split_chunk - 1) / split_chunk
                              : std::min(kDecodeWGs, (steps + 11) / 12);
  return std::max<int64_t>(1, std::min({n, steps, kMaxDecodeWGs}));
}
// partials of the MFMA decoder: two (max, sum, output) slots of Hq / H query heads per
// workgroup, then 32 bytes per workgroup describing the cut list that ends in its range
uint64_t mfma_partial_bytes(const kvq_params* p, int32_t split_chunk) {
  if (!mfma_format(p)) return 0;
  const uint64_t n = (uint64_t)decode_wgs(p, split_chunk);
  return n * 2ull * (uint64_t)(p->num_q_heads / p->num_kv_heads) * (kHeadDim + 2) * 4ull + n * 32ull;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~255ull; }

// Attention prologue: workgroups per K / V tile and per Q tile (a tile is one head's 128 output
// columns for up to 64 batch rows): about 256 Q workgroups in all, four times finer slices of
// d_model for the K / V tiles (they finish first; the Q workgroups then quantize their rows).
// Workspace: control words (zero between calls), the finished K / V rows, the partial tiles.
struct PrologueShape {
  int splits_kv, splits_q, row_blocks, nwg;
  uint64_t control_bytes, rows_bytes, partial_bytes;
};
PrologueShape prologue_shape(const kvq_params* p, int32_t d_model) {
  PrologueShape s;
  const int nch = d_model / 128;
  s.row_blocks = (p->batch + kPrologueRows - 1) / kPrologueRows;
  const int64_t q_tiles = (int64_t)p->num_q_heads * s.row_blocks;
  s.splits_q = (int)std::max<int64_t>(1, std::min<int64_t>(nch, (256 + q_tiles - 1) / q_tiles));
  s.splits_kv = std::min(nch, 4 * s.splits_q);
  s.nwg = 2 * p->num_kv_heads * s.splits_kv + p->num_q_heads * s.splits_q;
  const uint64_t words = (uint64_t)s.row_blocks * (2 * p->num_kv_heads + p->num_q_heads) +
                         (uint64_t)s.row_blocks * 2 * p->num_kv_heads + s.row_blocks + 2;
  s.control_bytes = align256(words * 4ull);
  s.rows_bytes = align256((uint64_t)s.row_blocks * 2 * p->num_kv_heads * kPrologueRows * kHeadDim * 4ull);
  s.partial_bytes = (uint64_t)s.row_blocks * s.nwg * (kPrologueRows * kHeadDim + kPrologueRows) * 4ull;
  return s;
}
// workspace of a decode with page masses: the decode's own, then page and total log-sum-exps
uint64_t mass_ws_bytes(const kvq_params* p, uint64_t decode_bytes) {
  return align256(decode_bytes) +
         ((uint64_t)p->batch * p->num_q_heads * (uint64_t)(p->max_pages_per_seq + 1)) * 4ull;
}

// Scratch memory of kvq_decode_attention_noalloc: the split-K partials of callers that cannot
// allocate.  Each GPU the library runs on holds its own copy until the process ends; host code
// never uses the array's name as an address (it is a host-side stand-in): the device address is
// looked up once per device with hipGetSymbolAddress, with that device current, and kept here.
__device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array.
int32_t scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KVQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KVQ_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return KVQ_OK;
}

// A nonzero number that differs from call to call (it wraps after 2^32 - 1 calls): it tags the
// arrival counts that the MFMA decoder leaves in the workspace, so that counts of earlier calls
// (or any other content) read as zero and the workspace needs no clearing.
uint32_t next_nonce() {
  static std::atomic<uint32_t> counter{0};
  uint32_t n;
  do { n = counter.fetch_add(1, std::memory_order_relaxed) + 1; } while (n == 0);
  return n;
}

// Validation and launches of a decode.  workspace == nullptr with use_scratch: the split-K
// partials go to this device's scratch array (kvq_decode_attention_noalloc).  k_new / v_new
// (kvq_append_decode): the decode also appends each sequence's last token.
int32_t decode_impl(const kvq_params* pin, const kvq_cache* cache, const void* q_bf16,
                    const int32_t* seq_lens, const int32_t* block_table, float sm_scale,
                    int32_t split_chunk, float* out, void* workspace, uint64_t ws_bytes,
                    bool use_scratch, void* stream, float* page_mass = nullptr,
                    const float* k_new = nullptr, const float* v_new = nullptr) {
  int32_t st = check_params(pin);
  if (st) return st;
  const Params n(pin);
  const kvq_params* p = &n.p;
  st = check_cache(p, cache);
  if (st) return st;
  if (isnan(sm_scale)) sm_scale = 1.0f / sqrtf((float)p->head_dim);   // the default scale
  if (!q_bf16 || !seq_lens || !out || !isfinite(sm_scale)) return KVQ_ERR_INVALID_ARG;
  if (p->page_size && !block_table) return KVQ_ERR_INVALID_ARG;
  if ((k_new != nullptr) != (v_new != nullptr)) return KVQ_ERR_INVALID_ARG;
  if (k_new && (p->page_size || !mfma_format(p))) return KVQ_ERR_UNSUPPORTED;
  const int chunk = resolve_chunk(p, split_chunk);
  if (chunk < 0) return KVQ_ERR_INVALID_ARG;
  uint64_t need = 0;
  kvq_workspace_bytes(p, split_chunk, &need);
  uint64_t need_mass = need;
  if (page_mass) {   // per-page and per-head log-sum-exps after the partials
    if (!p->page_size) return KVQ_ERR_UNSUPPORTED;
    need_mass = mass_ws_bytes(p, need);
    if (!workspace || ws_bytes < need_mass || ((uintptr_t)workspace & 15)) return KVQ_ERR_WORKSPACE;
  }
  if (use_scratch && need) {
    if (need > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
    st = scratch_ptr(&workspace);
    if (st) return st;
    ws_bytes = KVQ_NOALLOC_SCRATCH_BYTES;
  }
  if (need && (!workspace || ws_bytes < need || ((uintptr_t)workspace & 15))) return KVQ_ERR_WORKSPACE;
  DecodeLaunch d;
  d.L = make_layout(p, cache->outl_capacity);
  d.cache = *cache;
  d.q = (const uint16_t*)q_bf16;
  d.seq_lens = seq_lens;
  d.block_table = p->page_size ? block_table : nullptr;
  d.out = out;
  d.Hq = p->num_q_heads;
  d.fmt = p->format;
  d.group = p->group_size;
  d.outl = p->outlier_dtype;
  d.chunk = chunk;
  d.n_chunks = (p->max_seq_len + chunk - 1) / chunk;
  d.partials = need ? (float*)workspace : nullptr;
  d.nwg = (int)decode_wgs(p, split_chunk);
  d.nonce = next_nonce();
  d.page_lse = nullptr;
  d.total_lse = nullptr;
  if (page_mass) {
    d.page_lse = (float*)((uint8_t*)workspace + align256(need));
    d.total_lse = d.page_lse + (size_t)p->batch * p->num_q_heads * p->max_pages_per_seq;
  }
  d.scale_log2 = sm_scale * 1.4426950408889634f;
  d.k_new = k_new;
  d.v_new = v_new;
  d.tau2 = p->outlier_sigma * p->outlier_sigma;
  d.fit = n.fit;
  d.lloyd = p->lloyd_iters;
  hipStream_t s = (hipStream_t)stream;
  bool handled = false;
  if (launch_decode_mfma(d, s, &handled) != hipSuccess) return KVQ_ERR_HIP;
  if (!handled && page_mass) return KVQ_ERR_UNSUPPORTED;   // nothing launched
  if (!handled && launch_decode_generic(d, s) != hipSuccess) return KVQ_ERR_HIP;
  if (!handled && d.n_chunks > 1 && launch_lse_merge(d, s) != hipSuccess) return KVQ_ERR_HIP;
  if (page_mass) {
    MassLaunch m;
    m.page_lse = d.page_lse;
    m.total_lse = d.total_lse;
    m.seq_lens = seq_lens;
    m.mass = page_mass;
    m.B = p->batch;
    m.Hq = p->num_q_heads;
    m.max_pages = p->max_pages_per_seq;
    m.S_cap = p->max_seq_len;
    if (launch_mass_normalize(m, s) != hipSuccess) return KVQ_ERR_HIP;
  }
  return KVQ_OK;
}

}  // namespace

extern "C" {

int32_t kvq_kv_bytes(const kvq_params* pin, int32_t num_layers, int64_t num_tokens,
                     int64_t num_outliers, uint64_t* out_bytes) {
  const Params n(pin);
  const kvq_params* p = pin ? &n.p : nullptr;
  if (!p || !out_bytes || num_layers < 0 || num_tokens < 0 || num_outliers < 0 ||
      p->num_kv_heads < 1 || p->head_dim < 1)
    return KVQ_ERR_INVALID_ARG;
  const uint64_t LH = 2ull * (uint64_t)num_layers * (uint64_t)p->num_kv_heads * (uint64_t)num_tokens;
  if (p->format == KVQ_FMT_FP16 || p->format == KVQ_FMT_BF16) {
    *out_bytes = LH * (uint64_t)p->head_dim * 2ull;
    return KVQ_OK;
  }
  uint64_t row;
  if (p->format == FMT_FP8ROW) {
    row = (uint64_t)p->head_dim + 4ull;
  } else {
    if (!is_quant_fmt(p->format) || p->group_size < 1 || p->head_dim % p->group_size)
      return KVQ_ERR_INVALID_ARG;
    row = ((uint64_t)p->head_dim * code_bits(p->format) + 7) / 8 +   // whole bytes per row
          (uint64_t)(p->head_dim / p->group_size) * meta_bytes_per_group(p->format);
  }
  uint64_t vb = p->outlier_dtype == KVQ_OUTL_FP16 ? 2 : (p->outlier_dtype == KVQ_OUTL_FP8_E4M3 ? 1 : 0);
  *out_bytes = LH * row + (uint64_t)num_outliers * (vb ? vb + 4ull : 0ull);
  return KVQ_OK;
}

int32_t kvq_cache_sizes(const kvq_params* pin, int64_t outl_capacity, kvq_cache_sizes_t* out) {
  int32_t st = check_params(pin);
  if (st) return st;
  const Params n(pin);
  const kvq_params* p = &n.p;
  if (!out || outl_capacity < 0) return KVQ_ERR_INVALID_ARG;
  memset(out, 0, sizeof(*out));
  out->code_bytes_per_row = code_bytes(p);
  out->meta_bytes_per_row = meta_bytes(p);
  const uint64_t BH = (uint64_t)p->batch * p->num_kv_heads;
  if (p->page_size) {
    const uint64_t rows = (uint64_t)p->num_pages * p->num_kv_heads * kBlock;
    const uint64_t rows8 = (uint64_t)p->num_pages_fp8 * p->num_kv_heads * kBlock;
    out->codes = rows * out->code_bytes_per_row;
    out->meta = rows * out->meta_bytes_per_row;
    out->codes8 = rows8 * kHeadDim;
    out->scale8 = rows8 * 4;
  } else {
    const uint64_t rows = BH * (uint64_t)p->max_seq_len;
    out->codes = rows * out->code_bytes_per_row;
    out->meta = rows * out->meta_bytes_per_row;
  }
  const uint64_t vb = p->outlier_dtype == KVQ_OUTL_FP16 ? 2 : 1;
  out->outl_idx = BH * (uint64_t)outl_capacity * 4;
  out->outl_val = (BH * (uint64_t)outl_capacity * vb + 3) & ~3ull;  // whole 32-bit words
  out->outl_count = BH * 2 * 4;
  out->outl_block_start = BH * 2 * (uint64_t)((p->max_seq_len + kBlock - 1) / kBlock) * 4;
  return KVQ_OK;
}

int32_t kvq_quantize_append(const kvq_params* pin, const kvq_cache* cache, const float* k_new,
                            const float* v_new, int32_t max_new, const int32_t* positions,
                            const int32_t* counts, const int32_t* block_table, void* stream) {
  int32_t st = check_params(pin);
  if (st) return st;
  const Params n(pin);
  const kvq_params* p = &n.p;
  st = check_cache(p, cache);
  if (st) return st;
  if (!k_new || !v_new || !positions || !counts || max_new < 1) return KVQ_ERR_INVALID_ARG;
  if (p->page_size && !block_table) return KVQ_ERR_INVALID_ARG;
  QuantizeLaunch q;
  q.L = make_layout(p, cache->outl_capacity);
  q.cache = *cache;
  q.k_new = k_new;
  q.v_new = v_new;
  q.positions = positions;
  q.counts = counts;
  q.block_table = p->page_size ? block_table : nullptr;
  q.max_new = max_new;
  q.outl = p->outlier_dtype;
  q.tau2 = p->outlier_sigma * p->outlier_sigma;
  q.lloyd = p->lloyd_iters;
  q.fmt = p->format;
  q.group = p->group_size;
  q.fit = n.fit;
  if (launch_quantize_append(q, (hipStream_t)stream) != hipSuccess) return KVQ_ERR_HIP;
  return KVQ_OK;
}

int32_t kvq_workspace_bytes(const kvq_params* pin, int32_t split_chunk, uint64_t* out_bytes) {
  int32_t st = check_params(pin);
  if (st) return st;
  const Params n(pin);
  const kvq_params* p = &n.p;
  if (!out_bytes) return KVQ_ERR_INVALID_ARG;
  const int chunk = resolve_chunk(p, split_chunk);
  if (chunk < 0) return KVQ_ERR_INVALID_ARG;
  const uint64_t nc = (uint64_t)((p->max_seq_len + chunk - 1) / chunk);
  const uint64_t chunked = nc <= 1 ? 0 : (uint64_t)p->batch * p->num_q_heads * nc * (kHeadDim + 2) * 4ull;
  *out_bytes = mfma_format(p) ? mfma_partial_bytes(p, split_chunk) : chunked;
  return KVQ_OK;
}

int32_t kvq_decode_attention(const kvq_params* pin, const kvq_cache* cache, const void* q_bf16,
                             const int32_t* seq_lens, const int32_t* block_table,
                             float sm_scale, int32_t split_chunk, float* out, void* workspace,
                             uint64_t ws_bytes, void* stream) {
  return decode_impl(pin, cache, q_bf16, seq_lens, block_table, sm_scale, split_chunk, out,
                     workspace, ws_bytes, false, stream);
}

int32_t kvq_decode_attention_noalloc(const kvq_params* pin, const kvq_cache* cache,
                                     const void* q_bf16, const int32_t* seq_lens,
                                     const int32_t* block_table, float sm_scale,
                                     int32_t split_chunk, float* out, void* stream) {
  return decode_impl(pin, cache, q_bf16, seq_lens, block_table, sm_scale, split_chunk, out,
                     nullptr, 0, true, stream);
}

int32_t kvq_append_decode(const kvq_params* pin, const kvq_cache* cache, const float* k_new,
                          const float* v_new, const void* q_bf16, const int32_t* seq_lens,
                          float sm_scale, int32_t split_chunk, float* out, void* workspace,
                          uint64_t ws_bytes, void* stream) {
  if (!k_new || !v_new) return KVQ_ERR_INVALID_ARG;
  return decode_impl(pin, cache, q_bf16, seq_lens, nullptr, sm_scale, split_chunk, out, workspace,
                     ws_bytes, false, stream, nullptr, k_new, v_new);
}

int32_t kvq_mass_workspace_bytes(const kvq_params* pin, int32_t split_chunk, uint64_t* out_bytes) {
  int32_t st = check_params(pin);
  if (st) return st;
  if (!out_bytes) return KVQ_ERR_INVALID_ARG;
  if (!pin->page_size) return KVQ_ERR_UNSUPPORTED;
  const Params n(pin);
  uint64_t need = 0;
  st = kvq_workspace_bytes(&n.p, split_chunk, &need);
  if (st) return st;
  *out_bytes = mass_ws_bytes(&n.p, need);
  return KVQ_OK;
}

int32_t kvq_decode_attention_mass(const kvq_params* pin, const kvq_cache* cache, const void* q_bf16,
                                  const int32_t* seq_lens, const int32_t* block_table,
                                  float sm_scale, int32_t split_chunk, float* out,
                                  float* page_mass, void* workspace, uint64_t ws_bytes,
                                  void* stream) {
  if (!page_mass) return KVQ_ERR_INVALID_ARG;
  return decode_impl(pin, cache, q_bf16, seq_lens, block_table, sm_scale, split_chunk, out,
                     workspace, ws_bytes, false, stream, page_mass);
}

namespace {
uint64_t retier_n_cand(const kvq_params* p, int32_t n_free) {
  return (uint64_t)(n_free < p->num_pages_fp8 ? n_free : p->num_pages_fp8);
}
}  // namespace

int32_t kvq_retier_workspace_bytes(const kvq_params* pin, int32_t n_free, uint64_t* out_bytes) {
  int32_t st = check_params(pin);
  if (st) return st;
  if (!out_bytes || n_free < 0) return KVQ_ERR_INVALID_ARG;
  if (!pin->page_size) return KVQ_ERR_UNSUPPORTED;
  if (pin->max_pages_per_seq > kRetierMaxPages) return KVQ_ERR_UNSUPPORTED;
  const uint64_t cells = (uint64_t)pin->batch * pin->max_pages_per_seq;
  const uint64_t nc = retier_n_cand(pin, n_free);
  *out_bytes = 3 * cells * 4 + nc * 4 + nc * (uint64_t)pin->num_kv_heads * 2 * kBlock * 4 * 4;
  return KVQ_OK;
}

int32_t kvq_retier(const kvq_params* pin, const kvq_cache* cache, int32_t* block_table,
                   const int32_t* seq_lens, const float* page_mass, float keep_frac,
                   const int32_t* free_slots, int32_t n_free, int32_t* freed_slots,
                   int32_t* n_moved, void* workspace, uint64_t ws_bytes, void* stream) {
  uint64_t need = 0;
  int32_t st = kvq_retier_workspace_bytes(pin, n_free, &need);
  if (st) return st;
  const Params n(pin);
  const kvq_params* p = &n.p;
  st = check_cache(p, cache);
  if (st) return st;
  if (!block_table || !seq_lens || !page_mass || !n_moved || !(keep_frac >= 0.0f && keep_frac <= 1.0f))
    return KVQ_ERR_INVALID_ARG;
  const uint64_t nc = retier_n_cand(p, n_free);
  if (nc > 0 && (!free_slots || !freed_slots || !cache->codes8[0] || !cache->scale8[0]))
    return KVQ_ERR_INVALID_ARG;
  if (need && (!workspace || ws_bytes < need)) return KVQ_ERR_WORKSPACE;
  RetierLaunch r;
  r.L = make_layout(p, cache->outl_capacity);
  r.cache = *cache;
  r.block_table = block_table;
  r.seq_lens = seq_lens;
  r.mass = page_mass;
  r.keep_frac = keep_frac;
  r.free_slots = free_slots;
  r.n_free = n_free;
  r.n_cand = (int)nc;
  r.freed = freed_slots;
  r.n_moved = n_moved;
  const uint64_t cells = (uint64_t)p->batch * p->max_pages_per_seq;
  r.cand = (int32_t*)workspace;
  r.moves = r.cand + cells;
  r.rank = r.moves + cells;
  r.moved = r.rank + cells;
  r.bitmaps = (uint32_t*)(r.moved + nc);
  r.outl = p->outlier_dtype;
  r.tau2 = p->outlier_sigma * p->outlier_sigma;
  r.lloyd = p->lloyd_iters;
  hipStream_t s = (hipStream_t)stream;
  if (launch_retier_select(r, s) != hipSuccess) return KVQ_ERR_HIP;
  if (launch_retier_demote(r, s) != hipSuccess) return KVQ_ERR_HIP;
  if (launch_retier_commit(r, s) != hipSuccess) return KVQ_ERR_HIP;
  return KVQ_OK;
}

int32_t kvq_prologue_workspace_bytes(const kvq_params* pin, int32_t d_model, uint64_t* out_bytes) {
  int32_t st = check_params(pin);
  if (st) return st;
  const Params n(pin);
  if (!out_bytes || d_model < 128 || d_model % 128) return KVQ_ERR_INVALID_ARG;
  const PrologueShape sh = prologue_shape(&n.p, d_model);
  *out_bytes = sh.control_bytes + sh.rows_bytes + sh.partial_bytes;
  return KVQ_OK;
}

int32_t kvq_prologue_pack_weights(const kvq_params* pin, int32_t d_model, const void* weight_bf16,
                                  void* packed_bf16, void* stream) {
  uint64_t need = 0;
  int32_t st = kvq_prologue_workspace_bytes(pin, d_model, &need);
  if (st) return st;
  if (!weight_bf16 || !packed_bf16 || weight_bf16 == packed_bf16) return KVQ_ERR_INVALID_ARG;
  if (((uintptr_t)weight_bf16 | (uintptr_t)packed_bf16) & 15) return KVQ_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)(pin->num_q_heads + 2 * pin->num_kv_heads) * kHeadDim;
  if (launch_pack_weights(weight_bf16, packed_bf16, d_model, rows, (hipStream_t)stream) != hipSuccess)
    return KVQ_ERR_HIP;
  return KVQ_OK;
}

int32_t kvq_attention_prologue(const kvq_params* pin, const kvq_cache* cache, const void* hidden_bf16,
                               const void* gain_bf16, const void* weight_bf16, int32_t d_model,
                               float eps, const int32_t* positions, const int32_t* block_table,
                               void* q_bf16_out, float* proj_out, void* workspace, uint64_t ws_bytes,
                               void* stream) {
  uint64_t need = 0;
  int32_t st = kvq_prologue_workspace_bytes(pin, d_model, &need);
  if (st) return st;
  const Params n(pin);
  const kvq_params* p = &n.p;
  st = check_cache(p, cache);
  if (st) return st;
  if (!hidden_bf16 || !gain_bf16 || !weight_bf16 || !positions || !q_bf16_out) return KVQ_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || !isfinite(eps)) return KVQ_ERR_INVALID_ARG;
  if (((uintptr_t)hidden_bf16 | (uintptr_t)gain_bf16 | (uintptr_t)weight_bf16) & 15) return KVQ_ERR_INVALID_ARG;
  if (p->page_size && !block_table) return KVQ_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < need) return KVQ_ERR_WORKSPACE;
  const PrologueShape sh = prologue_shape(p, d_model);
  PrologueLaunch a;
  a.L = make_layout(p, cache->outl_capacity);
  a.cache = *cache;
  a.hidden = (const uint16_t*)hidden_bf16;
  a.gain = (const uint16_t*)gain_bf16;
  a.weight = (const uint16_t*)weight_bf16;
  a.positions = positions;
  a.block_table = p->page_size ? block_table : nullptr;
  a.q_out = (uint16_t*)q_bf16_out;
  a.proj_out = proj_out;
  int32_t* ctl = (int32_t*)workspace;
  a.arrive = ctl;
  a.ready = a.arrive + (size_t)sh.row_blocks * (2 * p->num_kv_heads + p->num_q_heads);
  a.claim = a.ready + (size_t)sh.row_blocks * 2 * p->num_kv_heads;
  a.ticket = a.claim + sh.row_blocks;
  a.done = a.ticket + 1;
  a.kvrows = (float*)((uint8_t*)workspace + sh.control_bytes);
  a.partials = (float*)((uint8_t*)workspace + sh.control_bytes + sh.rows_bytes);
  a.row_blocks = sh.row_blocks;
  a.Hq = p->num_q_heads;
  a.d = d_model;
  a.splits_kv = sh.splits_kv;
  a.splits_q = sh.splits_q;
  a.eps = eps;
  a.fmt = p->format;
  a.group = p->group_size;
  a.outl = p->outlier_dtype;
  a.fit = n.fit;
  a.lloyd = p->lloyd_iters;
  a.tau2 = p->outlier_sigma * p->outlier_sigma;
  if (launch_prologue(a, (hipStream_t)stream) != hipSuccess) return KVQ_ERR_HIP;
  return KVQ_OK;
}

int32_t kvq_probe_read(const void* src, uint64_t bytes, void* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16) return KVQ_ERR_INVALID_ARG;
  return launch_probe_read(src, bytes, sink, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int32_t kvq_probe_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16) return KVQ_ERR_INVALID_ARG;
  return launch_probe_copy(src, dst, bytes, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

const char* kvq_status_string(int32_t s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported format / shape";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_HIP: return "HIP launch error";
    case KVQ_ERR_CAPACITY: return "outlier list capacity exceeded";
    default: return "unknown status";
  }
}

}  // extern "C"
