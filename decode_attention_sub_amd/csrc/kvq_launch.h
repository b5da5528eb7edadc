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
  float* partials;            // [B][Hq][n_chunks][D + 2] or null when n_chunks == 1
  float* page_lse;            // paged, or null: [B][Hq][max_pages] log2-sum-exp of each page
  float* total_lse;           // with page_lse: [B][Hq] log2-sum-exp of every token
  int Hq;
  int fmt;
  int group;
  int outl;
  int chunk;                  // tokens per split-K chunk (multiple of 64)
  int n_chunks;               // ceil(S_cap / chunk)
  float scale_log2;           // sm_scale * log2(e)
  int cpw;                    // MFMA decoder: chunks per workgroup (set by its launcher)
};

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
