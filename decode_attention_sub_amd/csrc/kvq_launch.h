// Host-side launch descriptors shared by the C ABI (kvq_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "kvq_device.h"

namespace kvq {

struct QuantizeLaunch {
  Layout L;
  kvq_cache cache;
  const float* k_new;
  const float* v_new;
  const int32_t* positions;
  const int32_t* counts;
  const int32_t* block_table;
  int max_new;
  int outl;
  float tau2;
  int lloyd;
  int fmt;            // storage format
  int group;
  int fit;            // kFitDefault or the variant fit of a format stored as fmt
};

struct DecodeLaunch {
  Layout L;
  kvq_cache cache;
  const uint16_t* q;          // bf16 [B][Hq][D]
  const int32_t* seq_lens;
  const int32_t* block_table;
  float* out;                 // [B][Hq][D]
  float* partials;            // generic decoder: [B][Hq][n_chunks][D + 2] or null when n_chunks
                              // == 1; MFMA decoder: [nwg][2 slots][Hq / H][D + 2]
  float* page_lse;            // paged, or null: [B][Hq][max_pages] log2-sum-exp of each page
  float* total_lse;           // with page_lse: [B][Hq] log2-sum-exp of every token
  int Hq;
  int fmt;
  int group;
  int outl;
  int chunk;                  // tokens per split-K chunk (multiple of 64)
  int n_chunks;               // ceil(S_cap / chunk)
  float scale_log2;           // sm_scale * log2(e)
  int nwg;                    // MFMA decoder: workgroups sharing the steps of all lists
  uint32_t nonce;             // MFMA decoder: nonzero, different for every call (tags the arrival
                              // counts of cut lists in the workspace)
  // fused append (contiguous MFMA caches; k_new null otherwise): the row of token seq_lens[b] - 1
  // of every list, float32 [B][H][D] each, is quantized into the cache by the decode
  const float* k_new;
  const float* v_new;
  float tau2;                 // fl32(tau * tau)
  int fit;                    // kFitDefault or the variant fit of the storage format
  int lloyd;
};

// The MFMA decoder takes 2-bit caches and FP4 caches with groups of 32 (contiguous), and paged
// 2-bit caches whose pools it addresses with 32-bit byte offsets (the largest must stay below
// the offset that marks a skipped row); everything else takes the generic decoder.
inline bool mfma_decodes(int fmt, int group, bool paged, int64_t num_pages, int64_t num_pages_fp8,
                         int H) {
  if (fmt != FMT_C2 && !(fmt == FMT_FP4 && group == 32)) return false;
  if (!paged) return true;
  const uint64_t rows2 = (uint64_t)num_pages * (uint64_t)H * kBlock;
  const uint64_t rows8 = (uint64_t)num_pages_fp8 * (uint64_t)H * kBlock;
  return fmt == FMT_C2 && rows2 * 32 <= 0xFFFFF000ull && rows8 * kHeadDim <= 0xFFFFF000ull;
}

// Page attention masses of a paged decode (tiering.hip)
struct MassLaunch {
  const float* page_lse;      // [B][Hq][max_pages]
  const float* total_lse;     // [B][Hq]
  const int32_t* seq_lens;
  float* mass;                // [B][max_pages]
  int B, Hq, max_pages, S_cap;
};

// Demotion of cold FP8 pages to the 2-bit tier (tiering.hip, quantize.hip)
constexpr int kRetierMaxPages = 8192;   // pages per sequence the selection sorts in LDS
struct RetierLaunch {
  Layout L;
  kvq_cache cache;
  int32_t* block_table;       // [B][max_pages], entries of moved pages rewritten at the end
  const int32_t* seq_lens;
  const float* mass;          // [B][max_pages]
  float keep_frac;
  const int32_t* free_slots;  // free 2-bit pool slots, taken in order
  int n_free;
  int n_cand;                 // min(n_free, FP8 pool size): the most pages one call moves
  int32_t* freed;             // [n_cand] FP8 slots released, in rank order
  int32_t* n_moved;           // device: ranks handed out
  int32_t* cand;              // workspace [B][max_pages]: 1 = cold FP8 page
  int32_t* moves;             // workspace [B][max_pages]: new 2-bit slot or -1
  int32_t* rank;              // workspace [B][max_pages]: rank of a moved page or -1
  int32_t* moved;             // workspace [n_cand]: b * max_pages + p of each rank, or -1
  uint32_t* bitmaps;          // workspace [n_cand][H][2][16 rows][4]: outlier flags of moved rows
  int outl;
  float tau2;
  int lloyd;
};

// Attention prologue of a decode step (prologue.hip): RMSNorm, joint Q/K/V projection and the
// KV-cache write of the new token
constexpr int kPrologueRows = 64;     // batch rows per row block of the projection
struct PrologueLaunch {
  Layout L;
  kvq_cache cache;
  const uint16_t* hidden;     // bf16 [B][d]
  const uint16_t* gain;       // bf16 [d]
  const uint16_t* weight;     // bf16 [(Hq + 2H) * 128][d] (rows: Q heads, K heads, V heads) in
                              // the packed block order of launch_pack_weights
  const int32_t* positions;   // [B]: token of the new K / V rows, < 0: no write
  const int32_t* block_table;
  uint16_t* q_out;            // bf16 [B][Hq][128]
  float* proj_out;            // optional fp32 [B][(Hq + 2H) * 128]
  float* partials;            // [row blocks][workgroups][64 * 128 + 64]
  float* kvrows;              // [row blocks][2H][64][128] finished K / V rows
  // control words, zero between calls: arrival counters [row blocks][2H + Hq], K / V tile ready
  // flags [row blocks][2H], row-batch claims [row blocks], the role ticket, finished workgroups
  int32_t* arrive;
  int32_t* ready;
  int32_t* claim;
  int32_t* ticket;
  int32_t* done;
  int Hq, d;
  int splits_kv, splits_q;    // workgroups per K / V tile and per Q tile
  int row_blocks;
  float eps;
  int fmt, group, outl, fit, lloyd;
  float tau2;
};

hipError_t launch_prologue(const PrologueLaunch& a, hipStream_t st);
hipError_t launch_pack_weights(const void* w, void* out, int d, int64_t rows, hipStream_t st);
hipError_t launch_mass_normalize(const MassLaunch& m, hipStream_t st);
hipError_t launch_retier_select(const RetierLaunch& r, hipStream_t st);
hipError_t launch_retier_demote(const RetierLaunch& r, hipStream_t st);
hipError_t launch_retier_commit(const RetierLaunch& r, hipStream_t st);
hipError_t launch_quantize_append(const QuantizeLaunch& q, hipStream_t st);
hipError_t launch_decode_generic(const DecodeLaunch& d, hipStream_t st);
hipError_t launch_decode_mfma(const DecodeLaunch& d, hipStream_t st, bool* handled);
hipError_t launch_lse_merge(const DecodeLaunch& d, hipStream_t st);
hipError_t launch_probe_read(const void* src, uint64_t bytes, void* sink, hipStream_t st);
hipError_t launch_probe_copy(const void* src, void* dst, uint64_t bytes, hipStream_t st);

}  // namespace kvq
