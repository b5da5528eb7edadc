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
  int Hq;
  int fmt;
  int group;
  int outl;
  int chunk;                  // tokens per split-K chunk (multiple of 64)
  int n_chunks;               // ceil(S_cap / chunk)
  float scale_log2;           // sm_scale * log2(e)
  int cpw;                    // MFMA decoder: chunks per workgroup (set by its launcher)
};

hipError_t launch_quantize_append(const QuantizeLaunch& q, hipStream_t st);
hipError_t launch_decode_generic(const DecodeLaunch& d, hipStream_t st);
hipError_t launch_decode_mfma(const DecodeLaunch& d, hipStream_t st, bool* handled);
hipError_t launch_lse_merge(const DecodeLaunch& d, hipStream_t st);
hipError_t launch_probe_read(const void* src, uint64_t bytes, void* sink, hipStream_t st);
hipError_t launch_probe_copy(const void* src, void* dst, uint64_t bytes, hipStream_t st);

}  // namespace kvq
