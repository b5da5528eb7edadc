// Device helpers shared by the kvq kernels: number-format codecs, wave shuffles and the
// addressing of the contiguous and paged cache layouts.  Written for gfx950 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kBlock = 16;      // tokens per outlier block and per page

enum Fmt : int { FMT_FP8ROW = KVQ_FMT_FP8_E4M3_ROW, FMT_INT4 = KVQ_FMT_INT4_ASYM,
                 FMT_FP4 = KVQ_FMT_FP4_E2M1, FMT_C2 = KVQ_FMT_CENTROID2,
                 FMT_INT3 = KVQ_FMT_INT3_ASYM };
// Quantizer fits: a format variant is stored (and decoded) as its base format and differs only
// in how the quantizer fits the group (uniform 2-bit codebook as FMT_C2, symmetric INT4 as
// FMT_INT4).
enum Fit : int { kFitDefault = 0, kFitUniform = 1, kFitSym = 2 };
__host__ __device__ constexpr int storage_fmt(int fmt) {
  return fmt == KVQ_FMT_UNIFORM2 ? FMT_C2 : (fmt == KVQ_FMT_INT4_SYM ? FMT_INT4 : fmt);
}
__host__ __device__ constexpr int fit_of(int fmt) {
  return fmt == KVQ_FMT_UNIFORM2 ? kFitUniform : (fmt == KVQ_FMT_INT4_SYM ? kFitSym : kFitDefault);
}

__host__ __device__ constexpr int code_bits(int fmt) {
  return fmt == FMT_C2 ? 2 : (fmt == FMT_FP8ROW ? 8 : (fmt == FMT_INT3 ? 3 : 4));
}
__host__ __device__ constexpr int meta_bytes_per_group(int fmt) {
  return fmt == FMT_INT4 || fmt == FMT_INT3 ? 4 : (fmt == FMT_FP4 ? 1 : (fmt == FMT_C2 ? 8 : 0));
}

// ------------------------------------------------------------------ scalar bit casts
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// round to nearest even binary16 (v_cvt_f16_f32), returned as bits
__device__ __forceinline__ uint32_t f32_to_half_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// ------------------------------------------------------------------ E4M3FN (OCP FP8)
// bias 7, 3 mantissa bits, subnormals m * 2^-9, max finite 448 (0x7E); 0x7F is NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e == 0 ? (float)m * 0.001953125f  // m * 2^-9
                   : as_f32(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
  return (c & 0x80u) ? -v : v;
}

// nearest even E4M3 code of a finite float, saturating to +-448
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t sign = (as_u32(x) >> 24) & 0x80u;
  const float a = __builtin_fabsf(x);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {                 // below 2^-6: multiples of 2^-9, code = multiple
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  const uint32_t ua = as_u32(a);
  int e = (int)((ua >> 23) & 0xFFu) - 127;            // a = m * 2^e, m in [1, 2)
  const float m = as_f32((ua & 0x007FFFFFu) | 0x3F800000u);
  uint32_t mq = (uint32_t)__builtin_rintf((m - 1.0f) * 8.0f);
  if (mq == 8u) { mq = 0u; e += 1; }
  return sign | ((uint32_t)(e + 7) << 3) | mq;
}

// ------------------------------------------------------------------ E2M1 (OCP MX FP4)
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t mag = c & 7u;
  // 0, .5, 1, 1.5, 2, 3, 4, 6
  const float v = mag < 2u ? 0.5f * (float)mag
                           : (mag < 4u ? 1.0f + 0.5f * (float)(mag - 2u)
                                       : (mag < 6u ? 2.0f + (float)(mag - 4u)
                                                   : 4.0f + 2.0f * (float)(mag - 6u)));
  return (c & 8u) ? -v : v;
}

// nearest magnitude in {0,.5,1,1.5,2,3,4,6}, ties to the even code, saturating at 6;
// sign bit = sign bit of y
__device__ __forceinline__ uint32_t f32_to_e2m1(float y) {
  const float a = __builtin_fabsf(y);
  uint32_t m = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
             : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return m | ((as_u32(y) >> 28) & 8u);
}

// ------------------------------------------------------------------ wave helpers
// lane i reads lane i ^ w.  w < 16 stays inside a 16-lane DPP row and takes DPP moves (a few
// cycles): quad permutes for 1 and 2, row shifts for 4 (two moves, one per pair of banks) and
// a row rotation for 8; w = 16 goes through ds_swizzle (within the 32-lane half).
template <int W>
__device__ __forceinline__ int xor_i32(int v) {
  if constexpr (W == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);        // quad_perm [1,0,3,2]
  } else if constexpr (W == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);        // quad_perm [2,3,0,1]
  } else if constexpr (W == 4) {
    const int t = __builtin_amdgcn_update_dpp(v, v, 0x104, 0xF, 0x5, false);   // banks 0, 2: lane + 4
    return __builtin_amdgcn_update_dpp(t, v, 0x114, 0xF, 0xA, false);         // banks 1, 3: lane - 4
  } else if constexpr (W == 8) {
    return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);       // row_ror 8
  } else {
    return __builtin_amdgcn_ds_swizzle(v, (W << 10) | 0x1F);
  }
}
template <int W>
__device__ __forceinline__ float xor_f32(float v) {
  return as_f32((uint32_t)xor_i32<W>((int)as_u32(v)));
}
// lane S of the lane's 16-lane DPP row
template <int S>
__device__ __forceinline__ int row_bcast_i32(int v) {
  return __builtin_amdgcn_mov_dpp(v, 0x150 + S, 0xF, 0xF, false);    // row_newbcast S
}

// ------------------------------------------------------------------ cache addressing
struct Layout {
  int B, H, S_cap;
  int paged;               // 0 contiguous, 1 paged (16-token pages)
  int max_pages;           // block-table row length
  int code_bytes, meta_bytes;
  int nblk;                // outlier blocks per list = ceil(S_cap / 16)
  int64_t outl_cap;
  int num_pages;           // paged: tier-2 pool slots
  int num_pages_fp8;       // paged: tier-1 pool slots
};

struct RowRef {
  const uint8_t* codes;
  const uint8_t* meta;     // per-group metadata, or the fp32 scale of an FP8-tier row
  int tier1;               // 1: FP8 tier row
  int ok;                  // 0: the block-table entry names a slot outside its pool
};

// block-table entry -> (tier, slot); false when the slot is outside the tier's pool
__device__ __forceinline__ bool page_slot(const Layout& L, const int32_t* block_table, int b,
                                          int t, int* tier1, size_t* slot) {
  const uint32_t e = (uint32_t)block_table[(size_t)b * L.max_pages + (t >> 4)];
  *tier1 = (int)(e >> 31);
  *slot = e & 0x7FFFFFFFu;
  return *slot < (size_t)(*tier1 ? L.num_pages_fp8 : L.num_pages);
}

__device__ __forceinline__ RowRef row_ref(const Layout& L, const kvq_cache& c, int kv, int b,
                                          int h, int t, const int32_t* block_table) {
  RowRef r;
  r.ok = 1;
  if (!L.paged) {
    const size_t row = ((size_t)b * L.H + h) * (size_t)L.S_cap + (size_t)t;
    r.codes = (const uint8_t*)c.codes[kv] + row * L.code_bytes;
    r.meta = (const uint8_t*)c.meta[kv] + row * L.meta_bytes;
    r.tier1 = 0;
  } else {
    size_t slot;
    r.ok = page_slot(L, block_table, b, t, &r.tier1, &slot) ? 1 : 0;
    if (!r.ok) slot = 0;
    const size_t row = (slot * L.H + h) * kBlock + (size_t)(t & 15);
    if (r.tier1) {
      r.codes = (const uint8_t*)c.codes8[kv] + row * kHeadDim;
      r.meta = (const uint8_t*)(c.scale8[kv] + row);
    } else {
      r.codes = (const uint8_t*)c.codes[kv] + row * L.code_bytes;
      r.meta = (const uint8_t*)c.meta[kv] + row * L.meta_bytes;
    }
  }
  return r;
}

__device__ __forceinline__ size_t list_id(const Layout& L, int b, int h, int kv) {
  return ((size_t)b * L.H + h) * 2 + kv;
}

__device__ __forceinline__ void report(int32_t* status, int32_t code) {
  if (status) atomicCAS(status, 0, code);
}

}  // namespace kvq
