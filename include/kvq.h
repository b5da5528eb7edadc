/*
 * kvq — quantized-KV decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libkvq.so.  Every pointer argument named "device" is a HIP device pointer; every
 * other pointer is host memory.  The caller owns and frees every buffer; the library keeps no
 * global state and allocates no device memory (kvq_decode_attention_noalloc keeps one static
 * scratch array per GPU, see there).  Work is enqueued on the caller's stream
 * (``stream`` is a hipStream_t, passed as void*; NULL is the default stream) and the call
 * returns before the work completes.  Functions return KVQ_OK (0) or a negative kvq_status.
 *
 * What is computed (pages cited by title and section):
 *  - "Hierarchical Token Routing and Sub-2-Bit Non-Linear KV Compression ...", section
 *    "Paradigm 2: Sub-2-Bit Non-Linear KV-Cache Quantization": outliers beyond tau standard
 *    deviations are isolated and kept in FP8 (E4M3); the remaining values are coded against a
 *    4-centroid (2-bit) codebook fitted by k-means per group; section "Hardware-Kernel Fusion:
 *    Eliminating DRAM Round-Trips": dequantization is fused into the attention kernel.
 *  - "The Sub-10ms Barrier: Fusing Sparse MoE Routing with FP4 KV-Cache Quantization",
 *    section "2. FP4/INT4 KV-Cache Quantization": block-wise asymmetric INT4 with
 *    S = (max - min)/(2^b - 1) per group of 32 or 64 along the head dimension, or FP4 E2M1,
 *    computed at token insertion and dequantized inside flash-decoding.
 *  - "Hierarchical Token Gating and Tiered KV-Cache Paging ...", section "2. Entropy-Guided
 *    Tiered KV-Cache Quantization": 16-token pages held either in an FP8 tier or in the 2-bit
 *    tier, read through a paged-attention block table.
 *  - "Sub-5ms MoE Inference ...", section "Sub-Byte KV-Cache Quantization": fp16 outlier
 *    tensor beside packed 2-bit codes.
 *
 * Logical row encoding (one row = D values of one token, one KV head, K or V; a group = g
 * consecutive channels):
 *  - statistics per group in float32 with a fixed pairwise reduction tree; value x is an
 *    outlier iff (x - mean)^2 * (g - 1) > tau^2 * sum((x - mean)^2)  (i.e. |x - mean| > tau *
 *    unbiased std), one pass, strict;
 *  - the quantizer is fitted on the non-outliers; an outlier slot holds the code of 0.0;
 *  - INT4_ASYM: codes 0..15, per group fp16 scale S and fp16 zero z (= fp16(min)),
 *    value = code * S + z.  Metadata per group: [S, z] (4 bytes).
 *  - FP4_E2M1: codes sign<<3 | magnitude index into {0,.5,1,1.5,2,3,4,6}, per group an E4M3
 *    scale = E4M3(absmax / 6) (1 byte).  value = e2m1(code) * scale.
 *  - CENTROID2: codes 0..3, per group 4 fp16 centroids (8 bytes) from quartile-bin seeds and
 *    ``lloyd_iters`` Lloyd iterations.  value = centroid[code].
 *  - FP8_E4M3_ROW: codes E4M3(x / s), one fp32 scale s = absmax / 448 per row (4 bytes), no
 *    outliers.  value = e4m3(code) * s.
 *  - Format variants (contiguous caches only), laid out exactly like their base format and
 *    decoded by the same kernels; only the quantizer's fit differs:
 *    UNIFORM2 (as CENTROID2, g = 64): the uniform codebook of the compress_kv_head listing of
 *    the "Hierarchical Token Routing ..." page: with the outlier slots set to 0, centroids
 *    min, min + step, max - step, max of the group (step = fl32((max - min) / 3), torch's
 *    linspace), fp16, nearest centroid with the first index on ties;
 *    INT4_SYM (as INT4_ASYM, g = 32 or 64): the symmetric INT4 of the quantize_kv_cache_fp4
 *    listing of "The Sub-10ms Barrier ..." page, section "2. FP4/INT4 KV-Cache Quantization":
 *    S = fp16(max(absmax / 7, 1e-5)) over the non-outliers, code = clamp(rint(x / S), -8, 7) + 8,
 *    z = fp16(-8 S).
 *  - INT3_ASYM (contiguous caches, g = 32 or 64): the asymmetric 3-bit codes of the "Sub-5ms
 *    MoE Inference ..." page, section "Sub-Byte KV-Cache Quantization", fitted as INT4_ASYM
 *    with 2^b - 1 = 7: codes 0..7, S = fp16((max - min) / 7), z = fp16(min), value = code * S
 *    + z; metadata per group [S, z] (4 bytes); 48 code bytes per 128-channel row.  A quotient
 *    (x - z) / S with no value (S and z both beyond the fp16 range) gives code 0.
 *  Code packing along the channel axis:
 *    2-bit: each block of 16 channels fills 4 bytes; byte j of a block holds channels j, 4+j,
 *           8+j, 12+j in bit pairs 0, 1, 2, 3 (channel 16k + 4s + j in bits 2s..2s+1 of byte
 *           4k + j), so the 32-bit little-endian word of a block yields channels 4s..4s+3 from
 *           bit pair s of its four bytes;
 *    4-bit: channel 2k in bits 0-3 and channel 2k+1 in bits 4-7 of byte k;
 *    3-bit: one little-endian bit stream per row, channel c in stream bits 3c..3c+2.
 *
 * Outlier side lists: one per (sequence b, KV head h, K=0 / V=1), records in ascending
 * (token, channel) order: uint32 index = token * D + channel and the ORIGINAL value rounded to
 * the outlier dtype (fp16 bits or an E4M3 byte).  outl_count[b][h][kv] holds the record
 * count; outl_block_start[b][h][kv][blk] holds the number of records with token < 16 * blk
 * (written when token 16 * blk is appended).  Dequantization overwrites the code value at an
 * outlier position with the record's value.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1,  /* shape, pointer or range check failed on the host or device */
  KVQ_ERR_UNSUPPORTED = -2,  /* format / group / head-dim combination not implemented */
  KVQ_ERR_WORKSPACE = -3,    /* workspace pointer NULL, not 16-byte aligned, or smaller than
                                kvq_workspace_bytes */
  KVQ_ERR_HIP = -4,          /* a HIP launch returned an error */
  KVQ_ERR_CAPACITY = -5      /* device status only: an outlier list overflowed its capacity */
} kvq_status;

typedef enum {
  KVQ_FMT_FP16 = 0,          /* unquantized, for kvq_kv_bytes only */
  KVQ_FMT_FP8_E4M3_ROW = 1,  /* FP8 tier of a paged cache */
  KVQ_FMT_INT4_ASYM = 2,
  KVQ_FMT_FP4_E2M1 = 3,
  KVQ_FMT_CENTROID2 = 4,
  KVQ_FMT_BF16 = 5,          /* unquantized, for kvq_kv_bytes only */
  KVQ_FMT_UNIFORM2 = 6,      /* variant: stored and decoded as CENTROID2 */
  KVQ_FMT_INT4_SYM = 7,      /* variant: stored and decoded as INT4_ASYM */
  KVQ_FMT_INT3_ASYM = 8      /* contiguous caches only */
} kvq_format;

typedef enum { KVQ_OUTL_NONE = 0, KVQ_OUTL_FP16 = 1, KVQ_OUTL_FP8_E4M3 = 2 } kvq_outlier_dtype;

/* Problem description (the pages' GQA heads H, head dim D, context S, batch B, group size,
 * bit width via the format, and outlier threshold tau).  Constraints checked on the host:
 * head_dim == 128; num_q_heads % num_kv_heads == 0 with 1 <= num_q_heads/num_kv_heads <= 16;
 * group_size in {32, 64} dividing head_dim (INT4 / FP4 / INT4_SYM / INT3: 32 or 64; CENTROID2 /
 * UNIFORM2: 64);
 * max_seq_len >= 1; outlier_sigma > 0; lloyd_iters in [0, 64]; page_size 0 (contiguous) or 16
 * (paged, tiered: tier 2 = ``format``, tier 1 = FP8_E4M3_ROW; only CENTROID2 tier 2).
 * Every entry point accepts the format variants and treats their buffers as the base format's. */
typedef struct {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_seq_len;       /* token capacity per sequence */
  int32_t format;            /* kvq_format of the (tier-2) codes */
  int32_t group_size;
  int32_t outlier_dtype;     /* kvq_outlier_dtype */
  float outlier_sigma;       /* tau */
  int32_t lloyd_iters;       /* CENTROID2 only */
  int32_t page_size;         /* 0 = contiguous, 16 = paged */
  int32_t num_pages;         /* paged: slots in the tier-2 page pool */
  int32_t num_pages_fp8;     /* paged: slots in the FP8 tier-1 page pool */
  int32_t max_pages_per_seq; /* paged: row length of the block table */
} kvq_params;

/* Device buffers of one cache layer; index [0] = keys, [1] = values.
 * Contiguous:  codes[kv]  [B][H][max_seq_len][code_bytes]      code_bytes = D*bits/8
 *              meta[kv]   [B][H][max_seq_len][meta_bytes]      per-row group metadata
 * Paged:       codes[kv]  [num_pages][H][16][code_bytes]       tier-2 pool (128-byte aligned)
 *              meta[kv]   [num_pages][H][16][meta_bytes]
 *              codes8[kv] [num_pages_fp8][H][16][D]            FP8 tier-1 pool
 *              scale8[kv] [num_pages_fp8][H][16] float         per-row FP8 scales
 * Outliers:    outl_idx[kv] [B][H][outl_capacity] uint32 (outl_capacity <= 2^28), outl_val[kv] [B][H][outl_capacity]
 *              (uint16 fp16 bits or uint8 E4M3), outl_count [B][H][2] int32,
 *              outl_block_start [B][H][2][ceil(max_seq_len/16)] int32.
 *              outl_val buffers are 4-byte aligned and as large as kvq_cache_sizes reports
 *              (rounded up to whole 32-bit words: the decoder reads the aligned word around
 *              each value).
 * status: one int32 the kernels set (first error wins) to KVQ_ERR_CAPACITY or
 *         KVQ_ERR_INVALID_ARG when a device-side check fails; the library never clears it.
 * Buffers may be uninitialised except outl_count / status (zero before first use).
 * chan_mask: NULL for the tau test, or a static channel mask ("The Sub-10ms Barrier ...", section
 *         "Key Production Engineering Takeaways", item 2: the top channels by absolute magnitude
 *         kept at high precision): bit c % 32 of word [kv][h][c / 32] set = channel c of that
 *         list's rows is kept as an outlier record (at outlier_dtype, which must not be NONE) in
 *         every appended row, in place of the tau test; the fit runs on the other channels.
 *         Read by kvq_quantize_append only; decoding needs nothing more (the records are
 *         ordinary records). */
typedef struct {
  void* codes[2];
  void* meta[2];
  void* codes8[2];
  float* scale8[2];
  uint32_t* outl_idx[2];
  void* outl_val[2];
  int32_t* outl_count;
  int32_t* outl_block_start;
  int64_t outl_capacity;
  int32_t* status;
  const uint32_t* chan_mask; /* device [2][H][4] or NULL: see below */
} kvq_cache;

/* Byte sizes of every buffer of kvq_cache for these params (host only). */
typedef struct {
  uint64_t codes;        /* per kv */
  uint64_t meta;         /* per kv */
  uint64_t codes8;       /* per kv, paged */
  uint64_t scale8;       /* per kv, paged */
  uint64_t outl_idx;     /* per kv, for outl_capacity records per list */
  uint64_t outl_val;     /* per kv */
  uint64_t outl_count;
  uint64_t outl_block_start;
  uint32_t code_bytes_per_row;
  uint32_t meta_bytes_per_row;
} kvq_cache_sizes_t;

/* KV bytes for num_tokens tokens over num_layers layers: for FP16/BF16 exactly
 * 2 * L * H * D * 2 * tokens ("Hierarchical Token Routing ...", section "The Bottleneck",
 * KV size per token = 2 x L x H x D x precision); for quantized formats
 * 2 * L * H * tokens * (code_bytes + meta_bytes per row) + num_outliers * (value bytes + 4).
 * Uses num_kv_heads, head_dim, format, group_size, outlier_dtype of *p.  Host only. */
int32_t kvq_kv_bytes(const kvq_params* p, int32_t num_layers, int64_t num_tokens,
                     int64_t num_outliers, uint64_t* out_bytes);

int32_t kvq_cache_sizes(const kvq_params* p, int64_t outl_capacity, kvq_cache_sizes_t* out);

/* Quantize-on-append ("computed dynamically ... during token insertion", "The Sub-10ms
 * Barrier", section "2. FP4/INT4 KV-Cache Quantization", item 2).
 * k_new, v_new: device float32 [B][H][max_new][D].  positions, counts: device int32 [B];
 * sequence b receives rows i < counts[b] at tokens positions[b] + i.  Appending at position p
 * first truncates every outlier list of b to the records of tokens < p (so re-appending a
 * token replaces it); tokens < p must already be in the cache.  block_table: device int32
 * [B][max_pages_per_seq] (paged) or NULL; entry bit 31 = FP8 tier, bits 0..30 = slot in that
 * tier's pool.  Device-side errors (position + count > max_seq_len, list overflow) set
 * *status; overflowing records are dropped. */
int32_t kvq_quantize_append(const kvq_params* p, const kvq_cache* cache, const float* k_new,
                            const float* v_new, int32_t max_new, const int32_t* positions,
                            const int32_t* counts, const int32_t* block_table, void* stream);

/* Workspace for kvq_decode_attention.
 * 2-bit caches, and contiguous FP4 caches with groups of 32 (the MFMA decoder; paged pools
 * whose rows need byte offsets of 2^32 or more take the generic decoder): N workgroups share the
 * 32-token steps of all (sequence, KV head) lists, each a contiguous range in (sequence, head,
 * token) order, the ranges even in a weight of one per step plus a fixed cost per list (so that
 * ranges over many short lists take fewer steps).  A list cut between workgroups is merged by
 * log-sum-exp by the last workgroup to finish a part of it, from two (max, sum, output) slots per
 * workgroup, N * 2 * (Hq / H) * (D + 2) floats, followed by 32 bytes per workgroup whose first 8
 * count the finished parts of the cut list ending in its range, tagged with the call (so the
 * workspace needs no clearing; calls that share a workspace must not overlap):
 * N * (8 * (Hq / H) * (D + 2) + 32) bytes.  split_chunk 0: N = min(256, ceil(B * H *
 * ceil(max_seq_len / 32) / 12)) (one workgroup per CU of an MI355X, at least 12 steps each);
 * split_chunk > 0: N = min(B * H * ceil(max_seq_len / 32), 16384, ceil(B * H * max_seq_len /
 * split_chunk)).
 * Other formats (the generic decoder): split-K chunks of each list, whose (max, sum, output)
 * partials a second kernel merges by log-sum-exp: B * Hq * ceil(max_seq_len / chunk) * (D + 2)
 * floats (0 when one chunk covers max_seq_len); chunk = split_chunk, or by default 4096 for
 * paged caches and, for contiguous caches, enough chunks for 1024 (sequence, KV head, chunk)
 * units, chunks of at least 64 tokens, rounded up to a multiple of 64.  split_chunk must be a
 * multiple of 64.  The workspace must be 16-byte aligned. */
int32_t kvq_workspace_bytes(const kvq_params* p, int32_t split_chunk, uint64_t* out_bytes);

/* Fused dequantize + flash-decoding attention ("Fused Dequantization & FlashAttention
 * Kernel" of the figure in "The Bottleneck"; "Attention Phase / Flash-Decoding Engine" of
 * the figure in "The Twin Bottlenecks").  For each b and query head hq (KV head
 * hq * H / Hq): out[b][hq] = softmax_t(sm_scale * q . k_t) . v_t over tokens t < seq_lens[b],
 * with k_t, v_t dequantized on the fly; the parts of a list that different workgroups take
 * (see kvq_workspace_bytes) are merged by log-sum-exp.  sm_scale: any finite value, or NaN for the default 1/sqrt(head_dim);
 * an infinite scale is rejected.  q_bf16: device bfloat16 [B][Hq][D] (values must be finite
 * and within fp16 range); seq_lens: device int32 [B], 1 <= seq_lens[b] <= max_seq_len and no
 * more than the tokens appended; a sequence whose length is out of that range sets *status to
 * KVQ_ERR_INVALID_ARG and its out[b] is left unwritten (the other sequences are computed as
 * usual); block_table as above (paged) or NULL; out: device float32 [B][Hq][D]; workspace:
 * device, ws_bytes >= kvq_workspace_bytes.  A block-table entry of a live page that names a
 * slot outside its tier's pool sets *status to KVQ_ERR_INVALID_ARG; that page's rows then read
 * as zeros (nothing outside the pools is read). */
int32_t kvq_decode_attention(const kvq_params* p, const kvq_cache* cache, const void* q_bf16,
                             const int32_t* seq_lens, const int32_t* block_table,
                             float sm_scale, int32_t split_chunk, float* out, void* workspace,
                             uint64_t ws_bytes, void* stream);

/* One decode step with the quantize-on-append fused into the decode ("Sub-5ms MoE Inference
 * ...", section "Engineering Real-Time Autonomous Workflows", item 1: the KV-cache write fused
 * with the attention step): the same result as kvq_quantize_append of one token per sequence at
 * position seq_lens[b] - 1 (positions = seq_lens - 1, counts = 1, max_new = 1) followed by
 * kvq_decode_attention over seq_lens, in one launch.  The cache bytes it writes (codes,
 * metadata, outlier records, block starts, counts) are those of that append; the attention
 * output is that decode's within its floating-point rounding (the new token's contribution is
 * computed from the row it stores).  k_new, v_new: device float32 [B][H][D], the new token of
 * every (sequence, KV head); q_bf16, seq_lens, sm_scale, split_chunk, out, workspace, ws_bytes
 * as for kvq_decode_attention (same workspace size).  A sequence whose length is out of range
 * sets *status to KVQ_ERR_INVALID_ARG; nothing is appended to it and its out[b] is left
 * unwritten.  Contiguous caches of the MFMA decoder's formats (2-bit, FP4 with groups of 32)
 * only: any other cache returns KVQ_ERR_UNSUPPORTED and launches nothing (use the two calls). */
int32_t kvq_append_decode(const kvq_params* p, const kvq_cache* cache, const float* k_new,
                          const float* v_new, const void* q_bf16, const int32_t* seq_lens,
                          float sm_scale, int32_t split_chunk, float* out, void* workspace,
                          uint64_t ws_bytes, void* stream);

/* kvq_decode_attention for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation and the
 * same kernels, with the split-K partials in a scratch array the library holds in each GPU's
 * memory (a static device array of KVQ_NOALLOC_SCRATCH_BYTES, kept until the process ends);
 * nothing is allocated by the call.  The caller still passes the inputs and the output; the
 * current device must be the device of `stream`.  Returns KVQ_ERR_WORKSPACE when the partials
 * of this call (kvq_workspace_bytes for the same params and split_chunk) exceed
 * KVQ_NOALLOC_SCRATCH_BYTES; choose a longer split_chunk then.  All calls on one GPU share its
 * scratch array: calls that may overlap on one GPU (different streams without ordering) race
 * and must not be issued.  Otherwise as kvq_decode_attention. */
#define KVQ_NOALLOC_SCRATCH_BYTES (32ull << 20)
int32_t kvq_decode_attention_noalloc(const kvq_params* p, const kvq_cache* cache,
                                     const void* q_bf16, const int32_t* seq_lens,
                                     const int32_t* block_table, float sm_scale,
                                     int32_t split_chunk, float* out, void* stream);

/* Entropy-guided tiering of paged caches ("Hierarchical Token Gating and Tiered KV-Cache Paging
 * ...", section "2. Entropy-Guided Tiered KV-Cache Quantization": the pages holding most of the
 * attention weight stay FP8, the rest is 2-bit; "Operational Blueprint for AI Systems Engineers",
 * item 2: the ranking is refreshed every N decode steps).  A decode with page masses feeds the
 * re-tiering call; the caller runs the pair every N steps and appends new tokens into FP8 pages.
 *
 * kvq_decode_attention_mass: kvq_decode_attention of a paged cache (2-bit tier, pools below
 * 4 GiB; otherwise KVQ_ERR_UNSUPPORTED, nothing launched) that also writes page_mass (device
 * float32 [B][max_pages_per_seq]): the attention mass of page p of sequence b, the mean over the
 * Hq query heads of the sum of the softmax weights of its tokens (each sequence's masses sum to
 * 1; entries of pages past seq_lens[b], and of sequences whose length is rejected, are 0).  The
 * workspace (ws_bytes >= kvq_mass_workspace_bytes) holds the split-K partials and per-page and
 * per-head log-sum-exps. */
int32_t kvq_mass_workspace_bytes(const kvq_params* p, int32_t split_chunk, uint64_t* out_bytes);
int32_t kvq_decode_attention_mass(const kvq_params* p, const kvq_cache* cache, const void* q_bf16,
                                  const int32_t* seq_lens, const int32_t* block_table,
                                  float sm_scale, int32_t split_chunk, float* out,
                                  float* page_mass, void* workspace, uint64_t ws_bytes,
                                  void* stream);

/* kvq_retier: moves the cold FP8 pages of a paged cache to the 2-bit tier.  Per sequence b
 * (tokens < seq_lens[b], all appended), the hot pages are its ceil(keep_frac * n) pages of
 * largest page_mass (device float32 [B][max_pages_per_seq], e.g. from
 * kvq_decode_attention_mass), ties to the lower page; every FP8 page that is not hot is a
 * candidate.  Candidates in (sequence, page) order take the slots free_slots[0], [1], ... (device
 * int32 slots of the 2-bit pool, n_free of them); those past n_free or past num_pages_fp8 stay
 * FP8.  A moved page's rows (every KV head, K and V) are dequantized from FP8 in float32,
 * x = fl32(e4m3(code) * row scale), and quantized again exactly as kvq_quantize_append quantizes
 * a 2-bit row (outlier predicate or channel mask, Lloyd fit, records of the original x at the
 * outlier dtype); its records enter each sorted outlier list at its tokens' place (later records
 * move up; block starts and counts are rewritten; records past a list's capacity are dropped
 * and set *status to KVQ_ERR_CAPACITY).  Then block_table (device, in/out) names the new slots.
 * 2-bit pages never move up.  On return of the device work: *n_moved (device int32) = k, the
 * number of slots handed out; freed_slots[0 .. k-1] (device int32, capacity min(n_free,
 * num_pages_fp8)) = the FP8 slots released, in the same order as the free slots taken (-1 where
 * a free slot named a slot outside the 2-bit pool: that page stayed, *status is set to
 * KVQ_ERR_INVALID_ARG).  workspace: ws_bytes >= kvq_retier_workspace_bytes(p, n_free).  Paged
 * caches with max_pages_per_seq <= 8192 only (else KVQ_ERR_UNSUPPORTED). */
int32_t kvq_retier_workspace_bytes(const kvq_params* p, int32_t n_free, uint64_t* out_bytes);
int32_t kvq_retier(const kvq_params* p, const kvq_cache* cache, int32_t* block_table,
                   const int32_t* seq_lens, const float* page_mass, float keep_frac,
                   const int32_t* free_slots, int32_t n_free, int32_t* freed_slots,
                   int32_t* n_moved, void* workspace, uint64_t ws_bytes, void* stream);

/* Attention prologue of one decode step in a single kernel ("Sub-5ms MoE Inference ...",
 * section "Engineering Real-Time Autonomous Workflows", item 1: RMSNorm, the self-attention
 * projection and the KV-cache write fused into one kernel).  For every sequence b:
 *   x = h_b / sqrt(mean_i h_b[i]^2 + eps) * gain            (RMSNorm, d = d_model channels)
 *   y = W x,  W [(Hq + 2H) * D][d]: rows of Q heads 0..Hq-1, then K heads 0..H-1, then V heads
 *   q[b][hq] = y[hq D .. hq D + D - 1] rounded to bfloat16 (nearest even) -> q_bf16_out
 *   the K and V rows of KV head h (y[(Hq + h) D ..], y[(Hq + H + h) D ..]) are appended to the
 *   cache at token positions[b], exactly as kvq_quantize_append of those float32 rows with
 *   count 1 (positions[b] < 0: no write for that sequence; >= max_seq_len: *status is set to
 *   KVQ_ERR_INVALID_ARG and nothing is written).  No bias and no rotary embedding.
 * Arithmetic: bf16(h * gain) x W on bf16 MFMA with fp32 accumulation, scaled per row by
 * 1 / sqrt(sum(h^2) / d + eps) after the product; deterministic (independent of scheduling).
 * hidden_bf16 [B][d], gain_bf16 [d]: device bfloat16, 16-byte aligned; weight_bf16: W packed
 * by kvq_prologue_pack_weights (device, 16-byte aligned);
 * d_model a multiple of 128; eps >= 0 and finite; positions: device int32 [B]; block_table as
 * for appends (paged) or NULL; q_bf16_out: device bfloat16 [B][Hq][D]; proj_out: NULL or device
 * float32 [B][(Hq + 2H) D] receiving y (the rows the cache write quantizes); workspace: device,
 * ws_bytes >= kvq_prologue_workspace_bytes, zero-filled before its first use with this
 * library (every call leaves its arrival counters at zero again; calls sharing a workspace must
 * not overlap). */
int32_t kvq_prologue_workspace_bytes(const kvq_params* p, int32_t d_model, uint64_t* out_bytes);
/* Repacks W ([(Hq + 2H) D][d_model] bfloat16, row-major, as above) once into the block order
 * kvq_attention_prologue reads: for each group of 16 output rows cg and each step of 32 inputs
 * ks, one 1 KB block at byte (cg * d_model / 32 + ks) * 1024 whose 16-byte unit u = 16 q + j
 * (q < 4, j < 16) holds W[16 cg + j][32 ks + 8 q .. 32 ks + 8 q + 7], so that each wave streams
 * its rows through d_model contiguously.  weight_bf16 and packed_bf16: distinct device buffers
 * of (Hq + 2H) D d_model bfloat16, 16-byte aligned; enqueued on `stream`. */
int32_t kvq_prologue_pack_weights(const kvq_params* p, int32_t d_model, const void* weight_bf16,
                                  void* packed_bf16, void* stream);
int32_t kvq_attention_prologue(const kvq_params* p, const kvq_cache* cache, const void* hidden_bf16,
                               const void* gain_bf16, const void* weight_bf16, int32_t d_model,
                               float eps, const int32_t* positions, const int32_t* block_table,
                               void* q_bf16_out, float* proj_out, void* workspace,
                               uint64_t ws_bytes, void* stream);

/* Streaming read of `bytes` (multiple of 16) from device buffer src, XOR-reduced into sink
 * (device, >= 4 * 1024 * 256 bytes): measures the practical HBM read ceiling. */
int32_t kvq_probe_read(const void* src, uint64_t bytes, void* sink, void* stream);
/* Device-to-device copy of `bytes` (multiple of 16), used to calibrate byte counters. */
int32_t kvq_probe_copy(const void* src, void* dst, uint64_t bytes, void* stream);

const char* kvq_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
