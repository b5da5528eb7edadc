// Fused dequantize + flash-decoding attention on the MFMA matrix cores (gfx950) for caches whose
// dequantized values are exact in fp16: 2-bit centroid codes (fp16 centroids, E4M3 or fp16
// outliers) and FP4 E2M1 codes with E4M3 block scales (E2M1 x E4M3 has at most 6 significant
// bits and stays inside the fp16 range).
//
// "Hierarchical Token Routing and Sub-2-Bit Non-Linear KV Compression ...", section
// "Hardware-Kernel Fusion: Eliminating DRAM Round-Trips" (stream packed codes, expand on chip);
// "Sub-5ms MoE Inference ...", section "Engineering Real-Time Autonomous Workflows", item 3
// (bit-unpacked matrix products in matrix-core operand registers); "The Sub-10ms Barrier ...",
// section "2. FP4/INT4 KV-Cache Quantization", item 3 (dequantize into fp16 operand space inside
// the flash-attention reduction).
//
// Work split: the (sequence, KV head) lists are cut into 32-token steps and laid end to end; each
// workgroup of 12 waves (three per SIMD) takes an equal contiguous range of steps (one
// workgroup per CU by default), so sequences of any mix of lengths keep every CU equally busy.
// A workgroup's range is a run of pieces, each the part of one list inside the range; the waves
// take the 32-token steps of a piece in turn.  Per step a lane owns (token, 64-channel half row): it loads the
// packed codes and group metadata with 128-bit loads (prefetched one step ahead; 2-bit rows with
// non-temporal loads, as they are read once), expands them to fp16 in registers and writes the
// rows into the wave's LDS tile; outlier records of the step are written over their positions.  Scores are computed transposed,
// S^T = K^ Q^T, with v_mfma_f32_16x16x32_f16 (16 tokens x 16 padded query rows), which leaves
// every lane holding the probabilities of one query row for 4+4 tokens - exactly the B operand of
// O^T = V^T P^T.  V^T operands come out of the LDS tile with ds_read_b64_tr_b16.  P is split into
// fp16 hi + lo parts so that large outlier values in V see fp32-grade probabilities; with at most
// 8 query rows both parts ride in one B operand (hi parts in columns 0-7, lo parts in the padding
// columns 8-15), otherwise they take two MFMAs.  The waves' states are merged in LDS; a piece
// that is a whole list writes the final output, a part of a list (only the first and the last
// piece of a range can be one) a (max, sum, output) partial that streamk_merge_kernel combines.
// The waves of a SIMD keep pace with each other through their issue priority.
//
// 2-bit expansion: per 64-bit centroid word, two byte tables (low bytes and high bytes of the 4
// fp16 centroids) are built once; the four codes of one bit pair of a 32-bit code word (one per
// byte) form a selector that gives the low and high bytes of their centroids with one v_perm
// each, and two more v_perm interleave them into two fp16 pairs.  The packing puts channel 4s + j
// of a 16-channel word in byte j, bit pair s, so bit pair s yields channels 4s .. 4s+3 in order.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_launch.h"
#include "quant_row.h"   // (the row quantizers of the fused append; they turn contraction off)
#pragma clang fp contract(fast)

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef _Float16 __attribute__((address_space(3))) lds_half;

// 4 x 16-bit transposed LDS read (see the lane mapping in the file comment)
__device__ __forceinline__ half4v read_tr16(const lds_half* p) {
  const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)p);
  return __builtin_bit_cast(half4v, v);
}

constexpr int kStep = 32;                  // tokens per wave step
constexpr int kRow = 136;                  // LDS row stride in halfs (272 bytes)
constexpr int kTile = kStep * kRow;        // halfs per tile

// Workgroup shape: 12 waves (three per SIMD), one LDS tile per wave that holds the K rows and
// then the V rows of a step, one step of codes and records in flight, score MFMAs issued before
// the V rows are expanded (their operands then die early): the registers fit three waves per
// SIMD.
constexpr int kWaves = 12;
constexpr int kPF = 1;                     // steps of codes / records in flight per wave
// Paged caches: a workgroup lists the pages of its piece by tier, this many pages at a time.
constexpr int kSegPages = 1024;
// Work split: each list counts as kPieceSteps steps more than it holds, the fixed cost of a piece
// (its setup, page listing and epilogue) in units of one step of a workgroup, half before its
// steps and half after them (a list cut in two costs a piece in each workgroup), so that
// workgroups whose ranges cover many short lists take fewer steps.
template <bool PAGED> constexpr int kPieceSteps = PAGED ? 48 : 16;
constexpr uint32_t kDead = 0xFFFFFFFFu;    // no page: its rows read as zeros
// Fused append: the cost of appending a list's new token in units of one step, counted with the
// list's fixed cost after its steps, so that the workgroup holding the list's last step takes
// that many fewer steps.  The appending wave's fits (eight Lloyd iterations for 2-bit rows, one
// pass for FP4 rows) and their dependent loads hold the workgroup back by far more than their
// VALU work: the weights are measured (2-bit: 64 against 11, 32, 96 and 128, on 128 lists of
// 8192 tokens; FP4: 48 against 3 and 96, on 32 lists of 131072 tokens).
template <int FMT> constexpr int kAppSteps = FMT == FMT_C2 ? 64 : 48;

template <int FMT> struct Buf;
template <> struct Buf<FMT_C2> { uint4 kc, vc; uint2 km, vm; };
template <> struct Buf<FMT_FP4> { uint4 kc0, kc1, vc0, vc1; uint32_t km, vm; };

// A step of a paged cache: two pages of one tier (uniform): their pool rows of this KV head
// (kDead: no page) and logical page numbers.
struct PStep { uint32_t rowA, rowB; int pA, pB; };

// FP8-tier rows of a step (paged caches): a lane's K and V half rows, and the row scales of the
// tokens of its scores (K) and probabilities (V)
struct Buf8 { uint4 k[4], v[4]; floatx4 ks0, ks1, vs0, vs1; };

// FP8 row codes -> fp16 in channel order (E4M3 values are exact in fp16)
__device__ __forceinline__ void expand_fp8(const uint4 (&c)[4], _Float16* dst) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w[4] = {c[k].x, c[k].y, c[k].z, c[k].w};
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[j], 1.0f, false));
      o[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[j], 1.0f, true));
    }
    uint4* dd = (uint4*)(dst + 16 * k);
    dd[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dd[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

// The outlier records of one step of one list: records a0 .. a0 + na - 1, then (paged caches:
// those of the step's second page) b0 .. b0 + nb - 1.  baseA / baseB: the record index (token *
// 128 + channel) of tile row 0 for the records of each range.
struct RecList { int a0, na, b0, nb; uint32_t baseA, baseB; };
// Lane slot i of a list holds record i of the step.  Values are kept as the aligned 32-bit words
// that hold them; kb, vb (paged caches): the lane's record's base (a multiple of 2048) plus its
// value's bit offset inside the word (0, 8, 16 or 24).
struct Recs {
  uint32_t ik, vk;         // K: index word, value word
  uint32_t iv, vv;         // V: index word, value word
  uint32_t kb, vb;
  RecList k, v;
};

// raw buffer resource (gfx9 family): loads at byte offsets >= num_records return zero
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// CP: cache policy (kNT: non-temporal, for data read once)
constexpr int kNT = 2;
template <int CP = 0>
__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CP));
}
template <int CP = 0>
__device__ __forceinline__ uint2 ld64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, CP));
}
__device__ __forceinline__ uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
// with a uniform part of the offset in the scalar offset (the range check covers the sum)
template <int CP = 0>
__device__ __forceinline__ uint4 ld128s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, CP));
}
template <int CP = 0>
__device__ __forceinline__ uint2 ld64s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, CP));
}
__device__ __forceinline__ uint32_t ld32s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t ld16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// 64 channels of one 2-bit row -> 64 fp16 in channel order at dst
__device__ __forceinline__ void expand_c2(uint4 c, uint2 m, _Float16* dst) {
  const uint32_t tl = __builtin_amdgcn_perm(m.y, m.x, 0x06040200u);  // low bytes of C0..C3
  const uint32_t th = __builtin_amdgcn_perm(m.y, m.x, 0x07050301u);  // high bytes
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t o[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t x = (w[k] >> (2 * s)) & 0x03030303u;
      const uint32_t lo = __builtin_amdgcn_perm(th, tl, x);
      const uint32_t hi = __builtin_amdgcn_perm(tl, th, x);
      o[2 * s] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
      o[2 * s + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
    }
    uint4* d = (uint4*)(dst + 16 * k);
    d[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

// 64 channels of one FP4 row (two groups of 32) -> fp16 in natural order
__device__ __forceinline__ void expand_fp4(uint4 c0, uint4 c1, uint32_t m, _Float16* dst) {
  const _Float16 s0 = (_Float16)e4m3_to_f32(m & 0xFFu);
  const _Float16 s1 = (_Float16)e4m3_to_f32((m >> 8) & 0xFFu);
  const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const half2v sc = k < 4 ? half2v{s0, s0} : half2v{s1, s1};
    const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 0) * sc;
    const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 1) * sc;
    const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 2) * sc;
    const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 3) * sc;
    uint4 v;
    v.x = __builtin_bit_cast(uint32_t, a);
    v.y = __builtin_bit_cast(uint32_t, b);
    v.z = __builtin_bit_cast(uint32_t, c);
    v.w = __builtin_bit_cast(uint32_t, d);
    *(uint4*)(dst + 8 * k) = v;
  }
}

// stored outlier value -> fp16 (E4M3 values are exact in fp16)
// E4M3 bits placed as fp16 bits (exponent and mantissa shifted left by 7, sign on bit 15) encode
// value * 2^-8 for every code, subnormals included (both formats' subnormal steps line up); one
// exact fp16 multiply by 256 restores the value.  v + (v & 0x80) moves the sign bit up by one.
template <int OUTL>
__device__ __forceinline__ _Float16 outl_half(uint32_t v) {
  if constexpr (OUTL == KVQ_OUTL_FP16) {
    return __builtin_bit_cast(_Float16, (uint16_t)v);
  } else {
    const uint32_t h = (v + (v & 0x80u)) << 7;
    return __builtin_bit_cast(_Float16, (uint16_t)h) * (_Float16)256.0f;
  }
}

// outlier value stored at bit offset `bit` (mod 32) of word w -> fp16
template <int OUTL>
__device__ __forceinline__ _Float16 outl_from_word(uint32_t w, uint32_t bit) {
  if constexpr (OUTL == KVQ_OUTL_FP16) {
    return __builtin_bit_cast(_Float16, (uint16_t)__builtin_amdgcn_ubfe(w, bit, 16));
  } else {
    const uint32_t code = __builtin_amdgcn_ubfe(w, bit, 8);
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)code, 1.0f, false)[0];
  }
}

// LDS tile position of record offset dd = 128 * t + c (token t of the step, channel c < 128);
// the caller guarantees t < 32.
__device__ __forceinline__ uint32_t tile_pos(uint32_t dd) {
  static_assert(kRow == kHeadDim + 8, "row pad of 8 halfs assumed");
  return dd + ((dd >> 7) << 3);   // t * kRow + c = dd + 8 t
}

// V tiles keep token t in row 2 (t % 16) + t / 16: the four rows that one transposing read
// touches (tokens 4i .. 4i+3) are then 8 banks apart, and the rows written by lanes 0..7 of a
// 128-bit store are still 4 banks apart.  Lane row r therefore loads V of token vtok(r).
__device__ __forceinline__ int vrow_of(int t) { return 2 * (t & 15) + (t >> 4); }
__device__ __forceinline__ int vtok(int row) { return 16 * (row & 1) + (row >> 1); }
__device__ __forceinline__ uint32_t tile_pos_v(uint32_t dd) {
  const uint32_t t = dd >> 7;
  return (uint32_t)vrow_of((int)t) * (uint32_t)kRow + (dd & 127u);
}

// Overwrite one outlier position of a tile straight from the record (crowded steps); base is the
// record index of tile row 0.  A record outside the step's valid tokens goes to a pad slot (row
// 0, column 128) that no operand read touches.
template <int FMT, int OUTL, bool VT>
__device__ __forceinline__ void patch_at(_Float16* tile, uint32_t idx, uint32_t val, uint32_t base, int nval) {
  const uint32_t dd = idx - base;
  const uint32_t at = dd < (uint32_t)nval * 128u ? (VT ? tile_pos_v(dd) : tile_pos(dd)) : (uint32_t)kHeadDim;
  tile[at] = outl_half<OUTL>(val);
}

// p - (float)h for the low / high fp16 half h of pair, one mixed-precision FMA each (the exact
// remainder of the fp16 split: both values are fp32 and h is p rounded toward zero)
__device__ __forceinline__ float rem_lo(uint32_t pair, float p) {
  float r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(p));
  return r;
}
__device__ __forceinline__ float rem_hi(uint32_t pair, float p) {
  float r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(p));
  return r;
}

// DPP helpers (row = 16 lanes)
template <int CTRL, int BANKS>
__device__ __forceinline__ float dpp_f32(float old, float src) {
  return as_f32((uint32_t)__builtin_amdgcn_update_dpp((int)as_u32(old), (int)as_u32(src), CTRL, 0xF,
                                                      BANKS, false));
}
template <int CTRL, int BANKS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t src) {   // banks not written keep old
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, 0xF, BANKS, false);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t src) {   // lanes without a source: undefined
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)src, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float src) {
  return as_f32(dpp_u32<CTRL>(as_u32(src)));
}
constexpr int kRowShl8 = 0x108;   // lane i <- lane i + 8 of its row
constexpr int kRowShr8 = 0x118;   // lane i <- lane i - 8 of its row
constexpr int kRowRor8 = 0x128;   // lane i <- lane (i + 8) mod 16 of its row

// CMP: at most 8 query heads per KV head.  Score tiles then hold real query rows only in lanes
// r < 8; the softmax runs on 4 scores per lane after moving tile 1's rows into lanes r >= 8.
// PAGED: 2-bit pages behind a block table, some of them (tier 1) FP8 rows with a per-row scale.
// The workgroup lists the pages of its piece by tier (kSegPages at a time, in logical order) and
// takes the 2-bit pages two at a time as 32-token steps shaped like a contiguous cache's, then
// the FP8 pages two at a time (attention does not depend on the order of the tokens).  Only the
// last step of each tier's list can hold fewer than 32 tokens (a single page, or the sequence's
// partial last page).
// MASS (paged caches): every step also writes, per query head and page, log2 of the sum of the
// page's exp2-domain probabilities (the page's log-sum-exp), and the epilogue writes each query
// head's total; a later pass turns them into page attention masses.
// a / b for the merge descriptor's 64-bit counts, in 32 bits when both fit (64-bit division is
// a long instruction sequence)
__device__ __forceinline__ uint64_t udivq(uint64_t a, uint64_t b) {
  return ((a | b) >> 32) == 0 ? (uint64_t)((uint32_t)a / (uint32_t)b) : a / b;
}

// After the partials, 32 bytes per workgroup; the first 8 of workgroup i count the parts of the
// cut list whose last step i holds: (call nonce << 32) | parts finished (a word tagged with
// another call's nonce counts as zero, so the workspace needs no clearing).
__device__ __forceinline__ uint64_t* arrivals_of(const DecodeLaunch& d, int wg) {
  const size_t nf = (size_t)d.nwg * 2 * (size_t)(d.Hq / d.L.H) * (kHeadDim + 2);
  return (uint64_t*)((int4*)(d.partials + nf) + 2 * (size_t)wg);
}

// Partials of cut lists cross workgroups on different XCDs, whose L2 caches are not coherent
// with each other: they are stored and loaded with the cache policy bit sc1 of gfx940-family
// memory instructions, which reaches the device's coherence point.
constexpr int kSc1 = 16;
constexpr int kMergeBatch = 16;   // parts of a cut list whose loads are in flight at once
__device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(as_u32(v), r, (int)off, 0, kSc1);
}
__device__ __forceinline__ float load_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return as_f32(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kSc1));
}

// A cut list: the last workgroup to finish a part of it merges the parts of workgroups i0 .. i1
// (the owners of its first and last steps): out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i,
// M = max_i m_i (with page masses also the total log2-sum-exp).  Workgroup i0 holds the list's
// start in its first piece (slot 0) unless its range holds steps of an earlier list (slot 1);
// every later one holds a part in its first piece; workgroups with empty ranges hold nothing.
// Nobody waits: the last to arrive does the work.  Called by every thread of the workgroup after
// its parts are stored, for the list of sequence b, head h (nb steps, first unit pl); s_loc64[1]
// = U.
template <bool MASS>
__device__ __forceinline__ void merge_cut_list(const DecodeLaunch& d, int b, int h, int nb, uint64_t pl,
                                               int K0a, int K0b, const uint64_t* s_loc64, int* s_mg) {
  const int tid = threadIdx.x;
  const int G = d.Hq / d.L.H;
  const uint64_t nwg = gridDim.x;
  const __amdgpu_buffer_rsrc_t rpart = make_rsrc(d.partials, (uint32_t)(nwg * 2u * (uint64_t)G * (kHeadDim + 2) * 4u));
  if (tid == 0) {
    const uint64_t UU = s_loc64[1];
    const uint64_t u0 = pl + (uint64_t)K0a, ul = u0 + (uint64_t)(nb - 1);   // units of its first and last steps
    const uint64_t i0 = udivq((u0 + 1) * nwg - 1, UU), i1 = udivq((ul + 1) * nwg - 1, UU);
    uint32_t np = (uint32_t)(i1 - i0 + 1);
    if (UU < nwg) {
      np = 0;
      for (uint64_t i = i0; i <= i1; ++i) np += udivq(i * UU, nwg) < udivq((i + 1) * UU, nwg) ? 1u : 0u;
    }
    uint64_t* const w = arrivals_of(d, (int)i1);
    uint64_t old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), nw;
    do {
      nw = (uint32_t)(old >> 32) == d.nonce ? old + 1u : ((uint64_t)d.nonce << 32) | 1u;
    } while (!__hip_atomic_compare_exchange_strong(w, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT));
    s_mg[0] = (uint32_t)nw == np;
    s_mg[1] = (int)i0;
    s_mg[2] = (int)i1;
    s_mg[3] = udivq(i0 * UU, nwg) + (uint64_t)K0b >= pl ? 0 : 1;
  }
  __syncthreads();
  if (!s_mg[0]) return;
  const int i0 = s_mg[1], i1 = s_mg[2], slot0 = s_mg[3];
  const uint64_t UU = s_loc64[1];
  const bool may_be_empty = UU < nwg;
  for (int p = tid; p < G * kHeadDim; p += blockDim.x) {
    const int row = p / kHeadDim, ch = p % kHeadDim;
    float M = -INFINITY, den = 0.0f, num = 0.0f;
    for (int ib = i0; ib <= i1; ib += kMergeBatch) {
      float mm[kMergeBatch], ll[kMergeBatch], oo[kMergeBatch];
      bool use[kMergeBatch];
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {   // a batch of parts' loads in flight, at valid slots
        const int i = ib + k;
        use[k] = i <= i1 && !(may_be_empty && i > i0 &&
                              udivq((uint64_t)i * UU, nwg) == udivq((uint64_t)(i + 1) * UU, nwg));
        const uint32_t slot = use[k] ? (uint32_t)i * 2u + (i == i0 ? (uint32_t)slot0 : 0u) : (uint32_t)i0 * 2u + (uint32_t)slot0;
        const uint32_t o = ((slot * (uint32_t)G + (uint32_t)row) * (kHeadDim + 2)) * 4u;
        mm[k] = load_sc1(rpart, o);
        ll[k] = load_sc1(rpart, o + 4u);
        oo[k] = load_sc1(rpart, o + (2u + (uint32_t)ch) * 4u);
      }
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        if (!use[k]) continue;
        const float Mn = fmaxf(M, mm[k]);                      // a part holding tokens: m finite
        const float al = exp2f(M - Mn), wk = exp2f(mm[k] - Mn);   // al = 0 while M is -inf
        den = fmaf(wk, ll[k], den * al);
        num = fmaf(wk, oo[k], num * al);
        M = Mn;
      }
    }
    const size_t hq = (size_t)h * G + row;
    d.out[((size_t)b * d.Hq + hq) * kHeadDim + ch] = num / den;
    if (MASS && ch == 0) d.total_lse[(size_t)b * d.Hq + hq] = M + __builtin_log2f(den);
  }
}

// APP (contiguous caches): fused append.  In the workgroup that holds a list's last step, one
// wave first quantizes the row of token seq_lens[b] - 1 (k_new, v_new) into the cache, as an
// append at that position does, then decodes the list's last step from the cache (after its
// stores have completed and this CU's L1 is invalidated), then its share of the other steps.
// No other wave reads the last step's rows or records (the records of later tokens that a step's
// loads may see are skipped), so nobody waits for the append.
template <int FMT, int OUTL, bool CMP, bool PAGED, bool MASS, bool APP>
__global__ void __launch_bounds__(kWaves * 64) decode_mfma_kernel(DecodeLaunch d) {
  __shared__ __attribute__((aligned(16))) _Float16 s_lds[kWaves * kTile];
  __shared__ float s_ml[kWaves][16][2];
  __shared__ int s_simd[kWaves], s_prog[kWaves];   // SIMD of each wave, groups done
  // paged: the listed pages of each tier: {pool row of this KV head or kDead, logical page}
  __shared__ __attribute__((aligned(16))) uint32_t s_pl[PAGED ? 2 : 1][PAGED ? kSegPages : 1][2];
  __shared__ int s_wn[PAGED ? kSegPages / 64 : 1][2];   // pages per tier of each listing wave
  __shared__ uint64_t s_sc[kWaves];   // per-wave sums of the work split
  __shared__ int s_loc[3];            // the list and unit where the workgroup's range starts
  __shared__ uint64_t s_loc64[2];     // the current list's first unit; U
  __shared__ int s_mg[4];             // a cut list's merge: last part?, i0, i1, slot of i0
  __shared__ int s_cut[2][3];         // the lists of the parts in slots 0 and 1: b (-1: none), h, steps
  __shared__ uint64_t s_cut64[2];     // and their first units

  const Layout& L = d.L;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  constexpr int wpc = kWaves;                        // every wave works on every piece
  const int wi = wave;                               // the wave's place among them
  const int G = d.Hq / L.H;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, kg = lane >> 4;           // MFMA lane coordinates
  const int trow = lane & 31, half = lane >> 5;      // dequant lane coordinates
  constexpr int CB = FMT == FMT_C2 ? 32 : 64;
  constexpr int MB = FMT == FMT_C2 ? 16 : 4;
  constexpr int VB = OUTL == KVQ_OUTL_FP16 ? 2 : 1;
  constexpr bool HAS_OUTL = OUTL != KVQ_OUTL_NONE;

  // One tile per wave: K rows are expanded and read back as operands before V rows overwrite
  // them (a wave's LDS operations complete in issue order).
  _Float16* const ktile = s_lds + wave * kTile;
  _Float16* const vtile = ktile;

  // Two or three waves share each SIMD and the scheduler favours the oldest; every group of
  // steps, a wave that is ahead of the slower of its SIMD peers lowers its priority, so all
  // finish together.
  const int mysimd = (int)((__builtin_amdgcn_s_getreg((31 << 11) | 4) >> 4) & 3);   // HW_ID.simd
  if (lane == 0) { s_simd[wave] = mysimd; s_prog[wave] = 0; }
  __syncthreads();
  // the (up to two) other waves of this SIMD; a wave ahead of the slower of them yields
  int peer1 = wave, peer2 = wave;
  for (int w2 = 0; w2 < kWaves; ++w2) {
    if (w2 != wave && __builtin_amdgcn_readfirstlane(s_simd[w2]) == mysimd) {
      if (peer1 == wave) peer1 = w2;
      else peer2 = w2;
    }
  }
  if (peer2 == wave) peer2 = peer1;
  int* const prog_mine = &s_prog[wave];
  const int* const prog_p1 = &s_prog[peer1];
  const int* const prog_p2 = &s_prog[peer2];


  // ---- this workgroup's share of the work.  Every list (sequence b, KV head h) of a valid
  // sequence is cut into n_b = ceil(S_b / 32) steps and weighs m_b = K0 + n_b units: K0a units
  // of fixed cost, one per step, K0b units of fixed cost (K0a + K0b = K0 = kPieceSteps).  The
  // lists are laid end to end
  // in (sequence, head) order, U units in all, and workgroup i of N takes units [floor(i U /
  // N), floor((i + 1) U / N)): the steps of those units.  A piece is the part of one list
  // inside that range: only the first and the last piece of a workgroup can be parts of a list,
  // every other piece is a whole list.  Units per head of every sequence, summed, then scanned
  // to find the sequence that holds the range's first unit: all threads of the workgroup, 768
  // sequences at a time.
  // (fused append: the list's post units also count the append, so that the workgroup holding
  // its last step takes fewer steps)
  constexpr int K0 = kPieceSteps<PAGED> + (APP ? kAppSteps<FMT> : 0);
  constexpr int K0a = kPieceSteps<PAGED> / 2, K0b = K0 - K0a;
  constexpr int kT = kWaves * 64;
  const int tid = threadIdx.x;
  auto seq_steps = [&](int bb) -> uint64_t {
    if (bb >= L.B) return 0u;
    const int Sb = d.seq_lens[bb];
    return Sb >= 1 && Sb <= L.S_cap ? (uint64_t)((Sb + kStep - 1) / kStep + K0) : 0u;
  };
  auto wave_sum = [&](uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
  };
  auto wave_scan = [&](uint64_t v) {   // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint64_t y = __shfl_up(v, o, 64);
      if (lane >= o) v += y;
    }
    return v;
  };
  const uint64_t nwg = gridDim.x;
  if (tid == 0) { s_cut[0][0] = -1; s_cut[1][0] = -1; }
  uint64_t U = 0, ub = 0, ue = 0;
  int b = 0, h = 0, off = 0;   // the list of the first piece and the range's unit offset in it
  if (L.B <= kT) {
    // one sequence per thread: one scan gives the total and every sequence's first step
    uint64_t n = 0;
    if (tid < L.B) {
      const int Sb = d.seq_lens[tid];
      const bool ok = Sb >= 1 && Sb <= L.S_cap;
      if (!ok && blockIdx.x == 0) report(d.cache.status, KVQ_ERR_INVALID_ARG);
      n = ok ? (uint64_t)((Sb + kStep - 1) / kStep + K0) : 0u;
    }
    const uint64_t incl = wave_scan(n);
    if (lane == 63) s_sc[wave] = incl;
    __syncthreads();
    uint64_t woff = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      woff += w < wave ? s_sc[w] : 0u;
      U += s_sc[w];
    }
    U *= (uint64_t)L.H;
    ub = (uint64_t)blockIdx.x * U / nwg;
    ue = ((uint64_t)blockIdx.x + 1) * U / nwg;
    if (ub >= ue) return;
    const uint64_t lo = (woff + incl - n) * (uint64_t)L.H;   // the sequence's first step
    if (n > 0 && lo <= ub && ub < lo + n * (uint64_t)L.H) {
      s_loc[0] = tid;
      s_loc[1] = (int)((ub - lo) / n);
      s_loc[2] = (int)((ub - lo) % n);
      s_loc64[0] = lo + (ub - lo) / n * n;
      s_loc64[1] = U;
    }
    __syncthreads();
  } else {
    // blocks of 768 sequences: the total first, then the scan until the range's start
    uint64_t mine = 0;
    for (int bb = tid; bb < L.B; bb += kT) {
      const int Sb = d.seq_lens[bb];
      const bool ok = Sb >= 1 && Sb <= L.S_cap;
      if (!ok && blockIdx.x == 0) report(d.cache.status, KVQ_ERR_INVALID_ARG);
      mine += ok ? (uint64_t)((Sb + kStep - 1) / kStep + K0) : 0u;
    }
    mine = wave_sum(mine);
    if (lane == 0) s_sc[wave] = mine;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) U += s_sc[w];
    U *= (uint64_t)L.H;
    __syncthreads();
    ub = (uint64_t)blockIdx.x * U / nwg;
    ue = ((uint64_t)blockIdx.x + 1) * U / nwg;
    if (ub >= ue) return;
    uint64_t carry = 0;   // steps per head of the sequences before this block of sequences
    for (int c0 = 0;; c0 += kT) {
      const int bb = c0 + tid;
      const uint64_t n = seq_steps(bb);
      const uint64_t incl = wave_scan(n);
      if (lane == 63) s_sc[wave] = incl;
      __syncthreads();
      uint64_t woff = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        woff += w < wave ? s_sc[w] : 0u;
        tot += s_sc[w];
      }
      const uint64_t lo = (carry + woff + incl - n) * (uint64_t)L.H;
      if (n > 0 && lo <= ub && ub < lo + n * (uint64_t)L.H) {
        s_loc[0] = bb;
        s_loc[1] = (int)((ub - lo) / n);
        s_loc[2] = (int)((ub - lo) % n);
        s_loc64[0] = lo + (ub - lo) / n * n;
        s_loc64[1] = U;
      }
      __syncthreads();
      if ((carry + tot) * (uint64_t)L.H > ub) break;   // found in this block
      carry += tot;
    }
  }
  b = s_loc[0];
  h = s_loc[1];
  off = s_loc[2];

  uint64_t left = ue - ub;   // units of the range not yet taken
  for (bool first = true;;) {
  const int S = d.seq_lens[b];
  const int nb = (S + kStep - 1) / kStep;
  const int take = (int)min(left, (uint64_t)(nb + K0 - off));   // units of this list in the range
  const int s0 = min(max(off - K0a, 0), nb), s1 = min(max(off + take - K0a, 0), nb);   // its steps [s0, s1)
  const int t0 = kStep * s0, t1 = min(kStep * s1, S);   // the piece's tokens
  const bool whole = s0 == 0 && s1 == nb;
  // fused append: the piece that holds the list's last step appends its new token (token S - 1)
  const bool app = APP && s1 == nb && s1 > s0;
  if (s1 > s0 || app) {   // (only the first and the last list of a range can have no steps in it)

  // query operand (B of S^T = K^ Q^T): lane (row r, k-group kg), positions 32*ks + 8*kg + e
  half8 qop[4];
  {
    // every lane reads a valid row (padding rows read row 0 and are zeroed after the load)
    const uint16_t* qrow = d.q + ((size_t)b * d.Hq + (size_t)h * G + (r < G ? r : 0)) * kHeadDim;
    uint16_t raw[4][8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) raw[ks][e] = qrow[(32 * ks + 8 * kg + e)];
    // a negative softmax scale is folded into the queries (exact), so the scale below is >= 0
    const float keep = r < G ? (d.scale_log2 < 0.0f ? -1.0f : 1.0f) : 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[ks][e] = (_Float16)(as_f32((uint32_t)raw[ks][e] << 16) * keep);
  }

  // buffer resources.  Contiguous: rows [0, t1) of this (sequence, KV head); rows past t1 read as
  // zero.  Paged: the whole page pools (rows of absent pages get out-of-range offsets).
  const size_t rowbase = PAGED ? 0 : ((size_t)b * L.H + h) * (size_t)L.S_cap;
  const uint32_t nrows = PAGED ? (uint32_t)L.num_pages * (uint32_t)L.H * kBlock : (uint32_t)t1;
  const __amdgpu_buffer_rsrc_t rcK = make_rsrc((const uint8_t*)d.cache.codes[0] + rowbase * CB, nrows * CB);
  const __amdgpu_buffer_rsrc_t rcV = make_rsrc((const uint8_t*)d.cache.codes[1] + rowbase * CB, nrows * CB);
  const __amdgpu_buffer_rsrc_t rmK = make_rsrc((const uint8_t*)d.cache.meta[0] + rowbase * MB, nrows * MB);
  const __amdgpu_buffer_rsrc_t rmV = make_rsrc((const uint8_t*)d.cache.meta[1] + rowbase * MB, nrows * MB);
  const uint32_t coff = (uint32_t)(trow * CB + half * (CB / 2));
  const uint32_t coffv = (uint32_t)(vtok(trow) * CB + half * (CB / 2));
  const uint32_t lane4 = (uint32_t)lane * 4u, laneVB = (uint32_t)lane * VB, laneVB8 = laneVB * 8u;
  const uint32_t moff = (uint32_t)(trow * MB + half * (MB / 2));
  const uint32_t moffv = (uint32_t)(vtok(trow) * MB + half * (MB / 2));

  const size_t lidK = list_id(L, b, h, 0);
  const int cap = (int)min(L.outl_cap, (int64_t)INT32_MAX);
  __amdgpu_buffer_rsrc_t riK, riV, rvK, rvV, rbs;
  int cntK = 0, cntV = 0;
  uint32_t lv3 = 0;   // byte offset of the list's first value inside its aligned 32-bit word
  if constexpr (HAS_OUTL) {
    const size_t lbase = ((size_t)b * L.H + h) * (size_t)L.outl_cap;
    // value words: ranges start at the aligned word holding the list's first value and end at
    // the word holding its last (value buffers are padded to whole words)
    const size_t lvb = lbase * VB, w0 = lvb & ~(size_t)3;
    lv3 = (uint32_t)(lvb & 3);
    const uint32_t vbytes = (uint32_t)(((lvb + (size_t)cap * VB + 3) & ~(size_t)3) - w0);
    rvK = make_rsrc((const uint8_t*)d.cache.outl_val[0] + w0, vbytes);
    rvV = make_rsrc((const uint8_t*)d.cache.outl_val[1] + w0, vbytes);
    riK = make_rsrc(d.cache.outl_idx[0] + lbase, (uint32_t)cap * 4);
    riV = make_rsrc(d.cache.outl_idx[1] + lbase, (uint32_t)cap * 4);
    rbs = make_rsrc(d.cache.outl_block_start + lidK * (size_t)L.nblk, (uint32_t)L.nblk * 8);
    cntK = max(0, min(d.cache.outl_count[lidK], cap));
    cntV = max(0, min(d.cache.outl_count[lidK + 1], cap));
  }

  constexpr uint32_t kOOB = 0xFFFFFFF0u;   // an offset past every buffer range

  floatx4 oacc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) oacc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;   // -inf until the first step sets it
  // raw-score threshold of the lazy rescale: scores above it exceed m_run + 8 once scaled
  // (+inf when the scale is 0 and m_run is set: scaled scores are then all 0)
  float m_thr = -INFINITY;
  const float sl2 = fabsf(d.scale_log2);

  // One 32-token step.  FULL: every token of the step is valid; otherwise tokens < nval are.
  // IS8: FP8-tier rows (b8) with per-row scales, no outliers; otherwise codes (bf) and outlier
  // records (rc; records of tile row 0 at rc's bases).  Records past the first 64 of a step (per
  // list) are written by rarely taken loops.  Otherwise the body is one branch-free block: K rows
  // are expanded and written, the K^ operand reads are issued, the score MFMAs run, V rows are
  // expanded while those finish, the V^T operand reads are issued before the softmax needs them.
  auto consume = [&](const Buf<FMT>& bf, const Buf8& b8, const Recs& rc, uint32_t kb0, uint32_t vb0,
                     int nval, int pA, int pB, auto full_tag, auto is8_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr bool IS8 = decltype(is8_tag)::value;
    _Float16* krow = ktile + trow * kRow + 64 * half;
    _Float16* vrow = vtile + trow * kRow + 64 * half;
    // tile positions of this lane's record slots; an unused slot writes the lane's own pad slot
    // (row trow, column 128 + 4 half: no operand read touches it, and the unused slots of a
    // wave spread over the banks instead of all hitting one address)
    const uint32_t pad = (uint32_t)(trow * kRow + kHeadDim + 4 * half);
    uint32_t posK = pad, posV = pad;
    _Float16 ovK, ovV;
    const int nk = rc.k.na + rc.k.nb, nv = rc.v.na + rc.v.nb;
    if constexpr (HAS_OUTL && !IS8) {
      // bit offsets of the values inside their words (bit-field extraction takes them modulo 32)
      const uint32_t bitK = PAGED ? rc.kb : laneVB8 + ((uint32_t)rc.k.a0 * VB + lv3) * 8u;
      const uint32_t bitV = PAGED ? rc.vb : laneVB8 + ((uint32_t)rc.v.a0 * VB + lv3) * 8u;
      const uint32_t lim = (uint32_t)nval * 128u;
      const uint32_t ddk = rc.ik - (PAGED ? rc.kb & ~31u : kb0);
      posK = lane < nk && ddk < lim ? tile_pos(ddk) : pad;
      ovK = outl_from_word<OUTL>(rc.vk, bitK);
      const uint32_t ddv = rc.iv - (PAGED ? rc.vb & ~31u : vb0);
      posV = lane < nv && ddv < lim ? tile_pos_v(ddv) : pad;
      ovV = outl_from_word<OUTL>(rc.vv, bitV);
    }
    if constexpr (IS8) expand_fp8(b8.k, krow);
    else if constexpr (FMT == FMT_C2) expand_c2(bf.kc, bf.km, krow);
    else expand_fp4(bf.kc0, bf.kc1, bf.km, krow);
    if constexpr (HAS_OUTL && !IS8) {
      ktile[posK] = ovK;
      if (nk > 64) {
        for (int a = 64 + lane; a < nk; a += 64) {  // the rest of a crowded step
          const bool inA = a < rc.k.na;
          const uint32_t at = (uint32_t)(inA ? rc.k.a0 + a : rc.k.b0 + (a - rc.k.na));
          const uint32_t byte = at * VB + lv3;
          const uint32_t v = __builtin_amdgcn_ubfe(ld32(rvK, byte & ~3u), (byte & 3u) * 8u, VB * 8);
          patch_at<FMT, OUTL, false>(ktile, ld32(riK, at * 4u), v, inA ? rc.k.baseA : rc.k.baseB, nval);
        }
      }
    }
    half8 ak[8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      ak[ks] = *(const half8*)(ktile + r * kRow + 32 * ks + 8 * kg);
      ak[4 + ks] = *(const half8*)(ktile + (16 + r) * kRow + 32 * ks + 8 * kg);
    }
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak[ks], qop[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak[4 + ks], qop[ks], s1, 0, 0, 0);
    }
    if constexpr (IS8) expand_fp8(b8.v, vrow);
    else if constexpr (FMT == FMT_C2) expand_c2(bf.vc, bf.vm, vrow);
    else expand_fp4(bf.vc0, bf.vc1, bf.vm, vrow);
    if constexpr (HAS_OUTL && !IS8) {
      vtile[posV] = ovV;
      if (nv > 64) {
        for (int a = 64 + lane; a < nv; a += 64) {
          const bool inA = a < rc.v.na;
          const uint32_t at = (uint32_t)(inA ? rc.v.a0 + a : rc.v.b0 + (a - rc.v.na));
          const uint32_t byte = at * VB + lv3;
          const uint32_t v = __builtin_amdgcn_ubfe(ld32(rvV, byte & ~3u), (byte & 3u) * 8u, VB * 8);
          patch_at<FMT, OUTL, true>(vtile, ld32(riV, at * 4u), v, inA ? rc.v.baseA : rc.v.baseB, nval);
        }
      }
    }
    // V^T operands (16 channels x 32 tokens per M-tile) through transposing LDS reads
    half8 av[8];
    {
      const lds_half* vbase = (const lds_half*)vtile;
      const int col0 = 4 * (r & 3);
      const int rowo = vrow_of(4 * kg + (r >> 2));   // token 4 kg + r / 4; its tile-1 partner is the next row
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const half4v t0v = read_tr16(vbase + rowo * kRow + 16 * mt + col0);
        const half4v t1v = read_tr16(vbase + (rowo + 1) * kRow + 16 * mt + col0);
        av[mt] = half8{t0v[0], t0v[1], t0v[2], t0v[3], t1v[0], t1v[1], t1v[2], t1v[3]};
      }
    }
    // Online softmax in the exp2 domain.  Without CMP a lane holds query row r, tokens 4kg+v
    // (tile 0) and 16+4kg+v (tile 1); with CMP lanes r < 8 hold tile 0 and lanes r >= 8 hold
    // tile 1 of query r - 8.  The running maximum moves only when a scaled score exceeds it by
    // more than 2^8 (lazy rescaling): probabilities stay below 256, exact in fp32 and in the
    // fp16 hi + lo split.
    constexpr int NS = CMP ? 4 : 8;
    float sc[NS];
    if constexpr (CMP) {
#pragma unroll
      for (int v = 0; v < 4; ++v) sc[v] = dpp_f32<kRowShr8, 0xC>(s0[v], s1[v]);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) { sc[v] = s0[v]; sc[4 + v] = s1[v]; }
    }
    if constexpr (IS8) {   // FP8 rows: the K row scales multiply the scores
#pragma unroll
      for (int v = 0; v < NS; ++v) sc[v] *= (v < 4 ? b8.ks0 : b8.ks1)[v % 4];
    }
    bool valid[NS];
#pragma unroll
    for (int v = 0; v < NS; ++v) {
      const int tok = CMP ? (r >= 8 ? 16 : 0) + 4 * kg + v : (v < 4 ? 4 * kg + v : 12 + 4 * kg + v);
      valid[v] = FULL || tok < nval;
      if constexpr (!FULL) sc[v] = valid[v] ? sc[v] : -INFINITY;
    }
    // Lane-local maximum first: the row maximum (across the lanes that hold the row) is formed
    // only when some scaled score exceeds the running maximum by more than 2^8.
    float mx = sc[0];
#pragma unroll
    for (int v = 1; v < NS; ++v) mx = fmaxf(mx, sc[v]);
    if (__builtin_amdgcn_ballot_w64(mx > m_thr)) {
      if constexpr (CMP) mx = fmaxf(mx, dpp_f32<kRowRor8>(mx));
      const auto x16 = __builtin_amdgcn_permlane16_swap(as_u32(mx), as_u32(mx), false, false);
      mx = fmaxf(as_f32(x16[0]), as_f32(x16[1]));
      const auto x32 = __builtin_amdgcn_permlane32_swap(as_u32(mx), as_u32(mx), false, false);
      mx = fmaxf(as_f32(x32[0]), as_f32(x32[1]));
      const float m_new = fmaxf(m_run, mx * sl2);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) oacc[mt] *= alpha;
      m_run = m_new;
      m_thr = sl2 > 0.0f ? (m_run + 8.0f) / sl2 : (m_run == -INFINITY ? -INFINITY : INFINITY);
    }
    uint32_t hw[NS / 2], lw[NS / 2];
    float psum, psumA = 0.0f, psumB = 0.0f;   // without CMP: the tile-0 and tile-1 parts
#pragma unroll
    for (int v = 0; v < NS; v += 2) {
      float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[v], sl2, -m_run));
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[v + 1], sl2, -m_run));
      if constexpr (!FULL) { p0 = valid[v] ? p0 : 0.0f; p1 = valid[v + 1] ? p1 : 0.0f; }
      psum = v == 0 ? p0 + p1 : psum + (p0 + p1);
      if (v < 4) psumA += p0 + p1;
      else psumB += p0 + p1;
      if constexpr (IS8) {   // FP8 rows: the V row scales multiply the probabilities
        const floatx4 vs = v < 4 ? b8.vs0 : b8.vs1;
        p0 = FULL || valid[v] ? p0 * vs[v % 4] : 0.0f;
        p1 = FULL || valid[v + 1] ? p1 * vs[v % 4 + 1] : 0.0f;
      }
      const half2v hi = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(p0, p1));
      hw[v / 2] = __builtin_bit_cast(uint32_t, hi);
      lw[v / 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(rem_lo(hw[v / 2], p0), rem_hi(hw[v / 2], p1)));
    }
    l_run += psum;
    if constexpr (MASS) {
      // page sums: over the 4 lanes (k-groups) holding a query row's tokens of a tile; tile 0 is
      // page pA, tile 1 page pB
      auto kg_sum = [](float x) {
        const auto x16 = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
        x = as_f32(x16[0]) + as_f32(x16[1]);
        const auto x32 = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
        return as_f32(x32[0]) + as_f32(x32[1]);
      };
      const float sA = kg_sum(CMP ? psum : psumA);
      const float sB = CMP ? 0.0f : kg_sum(psumB);
      const int row = CMP ? (r & 7) : r;
      if (kg == 0 && row < G) {
        float* dst = d.page_lse + ((size_t)b * d.Hq + (size_t)h * G + row) * L.max_pages;
        auto lse = [&](float x) { return x > 0.0f ? m_run + __builtin_log2f(x) : -INFINITY; };
        if constexpr (CMP) {
          const int pg = r < 8 ? pA : pB;
          if (pg >= 0) dst[pg] = lse(sA);
        } else {
          if (pA >= 0) dst[pA] = lse(sA);
          if (pB >= 0) dst[pB] = lse(sB);
        }
      }
    }
    if constexpr (CMP) {
      // One B operand carries both parts: column r < 8 the hi parts of query r (tile-0 tokens of
      // its own lane, tile-1 tokens from lane r + 8), column r + 8 the lo parts of query r
      // (tile-0 tokens from lane r, tile-1 tokens of its own lane).  The two columns of a query
      // are summed once, after the last step.
      const uint4 pq = make_uint4(dpp_u32<kRowShr8, 0xC>(hw[0], lw[0]), dpp_u32<kRowShr8, 0xC>(hw[1], lw[1]),
                                  dpp_u32<kRowShl8, 0x3>(lw[0], hw[0]), dpp_u32<kRowShl8, 0x3>(lw[1], hw[1]));
      const half8 pb = __builtin_bit_cast(half8, pq);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[mt], pb, oacc[mt], 0, 0, 0);
    } else {
      const half8 phi = __builtin_bit_cast(half8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      const half8 plo = __builtin_bit_cast(half8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[mt], phi, oacc[mt], 0, 0, 0);
        oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[mt], plo, oacc[mt], 0, 0, 0);
      }
    }
  };

  // Fused append, by one wave: the row of the list's token S - 1 is quantized into the cache as
  // an append at that position does it (lanes 0-31 the K row, lanes 32-63 the V row, staged in
  // the wave's tile, which is free until its walk); the list's new record counts (K, V) are
  // returned for the last step's record bounds.
  auto append_token = [&]() -> int2 {
    constexpr int GQ = FMT == FMT_C2 ? 64 : 32;   // quantization group
    constexpr int QL = GQ / 4;
    RowStage<2>& st = *(RowStage<2>*)ktile;
    const int kv = lane >> 5, rl = lane & 31, gi = rl / QL, jg = rl % QL;
    const float* src = (kv ? d.v_new : d.k_new) + ((size_t)b * L.H + h) * kHeadDim;
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = src[gi * GQ + jg + QL * e];
    auto wsync = [] {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    };
    const int64_t run = records_before<kRowLanes>(d, b, h, kv, S - 1, rl);
    const int cnt = (int)append_row<FMT, GQ>(d, true, b, h, kv, S - 1, run, x, rl, kv, st, wsync);
    return int2{__builtin_amdgcn_readlane(cnt, 0), __builtin_amdgcn_readlane(cnt, 32)};
  };

  const Buf8 no8{};
  constexpr int NB = kPF + 1;  // ring slots

  if constexpr (!PAGED) {
    // The piece's full 32-token steps are spread over the waves; the list's ragged last step (if
    // it is in the piece) is left to the first wave after the others, and in a piece that
    // appends, the list's last step to the appending wave.
    const int nsteps = (t1 - t0 + kStep - 1) / kStep;
    const bool ragged = (t1 - t0) % kStep != 0;
    const int nfull = nsteps - (ragged || app ? 1 : 0);
    // Workgroups walk their full steps in rotated order, starting at evenly spread points: lists
    // start at power-of-two-aligned offsets, and walking them in lockstep would send every
    // workgroup to the same HBM channels at the same time.
    const int rot = nfull > 0 ? (int)(((uint64_t)blockIdx.x * (uint64_t)nfull) / nwg) : 0;
    // fused append: wave aw appends the list's new token, then takes the list's last step (which
    // is left out of the other waves' steps)
    const int aw = APP ? (int)(((size_t)b * L.H + h) % kWaves) : 0;
    // RAGGED: the step may hold tokens >= t1 (only the list's last step); the buffer ranges end
    // at row t1, so those rows read as zeros
    auto issue_codes = [&](Buf<FMT>& bf, int tsi) {
      const uint32_t ts = (uint32_t)tsi;
      if constexpr (FMT == FMT_C2) {
        // 2-bit rows are read once: non-temporal loads (measured faster; for FP4 rows, slower)
        bf.kc = ld128s<kNT>(rcK, coff, ts * CB);
        bf.vc = ld128s<kNT>(rcV, coffv, ts * CB);
        bf.km = ld64s<kNT>(rmK, moff, ts * MB);
        bf.vm = ld64s<kNT>(rmV, moffv, ts * MB);
      } else {
        bf.kc0 = ld128s(rcK, coff, ts * CB);
        bf.kc1 = ld128s(rcK, coff + 16, ts * CB);
        bf.vc0 = ld128s(rcV, coffv, ts * CB);
        bf.vc1 = ld128s(rcV, coffv + 16, ts * CB);
        bf.km = ld16s(rmK, moff, ts * MB);
        bf.vm = ld16s(rmV, moffv, ts * MB);
      }
    };
    // lanes 0..3 load {K start, K end, V start, V end} of the step's records (block starts)
    auto issue_bounds = [&](int ts) -> uint32_t {
      if constexpr (HAS_OUTL) {
        const int which = lane & 3;  // 0: K blk, 1: K blk+2, 2: V blk, 3: V blk+2
        const uint32_t off = (uint32_t)(((which >> 1) * L.nblk + (ts >> 4) + 2 * (which & 1)) * 4);
        return ld32(rbs, off);
      }
      return 0u;
    };
    auto issue_recs = [&](Recs& rc, uint32_t bnd, int ts) {
      if constexpr (HAS_OUTL) {
        const bool last = ts + kStep >= S;
        const int k0 = max(0, min(__builtin_amdgcn_readlane((int)bnd, 0), cap));
        const int k1 = last ? cntK : max(0, min(__builtin_amdgcn_readlane((int)bnd, 1), cap));
        const int v0 = max(0, min(__builtin_amdgcn_readlane((int)bnd, 2), cap));
        const int v1 = last ? cntV : max(0, min(__builtin_amdgcn_readlane((int)bnd, 3), cap));
        const uint32_t base = (uint32_t)ts * 128u;   // record index of the step's first row
        rc.k = RecList{k0, max(k1 - k0, 0), 0, 0, base, base};
        rc.v = RecList{v0, max(v1 - v0, 0), 0, 0, base, base};
        // Slots past a list's records read past its range (zeros) or unused records.  Values are
        // read as the aligned 32-bit word that holds them and extracted where they are used: a
        // byte or short load would leave the compiler a narrow value that it re-extends at the
        // loop back-edge, waiting for the load there.
        rc.ik = ld32s(riK, lane4, (uint32_t)k0 * 4u);
        rc.iv = ld32s(riV, lane4, (uint32_t)v0 * 4u);
        // value word of a lane's record: the list's byte offset k0 * VB + lv3 (uniform) split
        // into its word-aligned part (scalar offset) and its remainder, which joins the lane's bytes
        const uint32_t bk = (uint32_t)k0 * VB + lv3, bv = (uint32_t)v0 * VB + lv3;
        rc.vk = ld32s(rvK, ((bk & 3u) + laneVB) & ~3u, bk & ~3u);
        rc.vv = ld32s(rvV, ((bv & 3u) + laneVB) & ~3u, bv & ~3u);
      } else {
        rc.k = RecList{0, 0, 0, 0, 0u, 0u};
        rc.v = rc.k;
      }
    };
    // ---- software pipeline: codes and records of the next kPF steps in flight, the record
    // bounds of the step after them too.  Wave wi takes its full steps wi, wi + wpc, ... of the
    // rotated order; whole groups of NB steps run without conditions, so every ring slot keeps
    // its registers and the wait counters stay exact.  Ring slot u holds the step that is
    // consumed at its turn; its token start is then replaced by the one of the step NB later
    // (position an of the wave's next step in the rotated order, advanced modulo nfull).  Steps
    // past the wave's share start past the piece: every load reads zeros without touching memory.
    Buf<FMT> buf[NB];
    Recs rec[NB];
    uint32_t bnd[NB];
    int tsr[NB];
    // the list's last step, alone (tokens < t1 of it)
    auto last_step = [&]() {
      const int ts = t0 + kStep * (nsteps - 1);
      const uint32_t b0 = issue_bounds(ts);
      issue_recs(rec[0], b0, ts);
      issue_codes(buf[0], ts);
      consume(buf[0], no8, rec[0], (uint32_t)ts * 128u, (uint32_t)ts * 128u, t1 - ts, 0, 0,
              std::false_type{}, std::false_type{});
    };
    if (app && wi == aw) {
      const int2 nc = append_token();
      cntK = nc.x;   // the last step's record bounds
      cntV = nc.y;
      // the stores are complete, and this CU's L1 holds no line that other waves read before
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      last_step();
    }
    const int nmine = wi < nfull ? (nfull - wi + wpc - 1) / wpc : 0;
    const int tpast = t1 + 2 * kStep;
    int jn = 0;                                  // the wave's next step to start
    int an = wi + rot;                           // its position in the piece's full steps
    if (an >= nfull) an -= nfull;
    auto next_ts = [&]() {   // (selects, no branches; an is used only while jn < nmine, and
      // wpc >= nfull only when the wave has a single step)
      const int ts = jn < nmine ? t0 + kStep * an : tpast;
      an += wpc;
      an = an >= nfull ? an - nfull : an;
      ++jn;
      return ts;
    };
    int partner_seen = 0;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      tsr[k] = next_ts();
      bnd[k] = issue_bounds(tsr[k]);
    }
#pragma unroll
    for (int k = 0; k < kPF; ++k) {
      issue_recs(rec[k], bnd[k], tsr[k]);
      issue_codes(buf[k], tsr[k]);
    }
    auto walk_step = [&](int u) {
      const uint32_t base = (uint32_t)tsr[u] * 128u;
      tsr[u] = next_ts();
      bnd[u] = issue_bounds(tsr[u]);
      const int up = (u + kPF) % NB;
      issue_recs(rec[up], bnd[up], tsr[up]);
      issue_codes(buf[up], tsr[up]);
      consume(buf[u], no8, rec[u], base, base, kStep, 0, 0, std::true_type{}, std::false_type{});
    };
    const int ngroups = nmine / NB;
    for (int g = 0; g < ngroups; ++g) {
      if (g > partner_seen) __builtin_amdgcn_s_setprio(0);
      else __builtin_amdgcn_s_setprio(1);
      if (lane == 0) *prog_mine = g;
#pragma unroll
      for (int u = 0; u < NB; ++u) walk_step(u);
      partner_seen = min(__builtin_amdgcn_readfirstlane(*prog_p1), __builtin_amdgcn_readfirstlane(*prog_p2));
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int u = 0; u < NB - 1; ++u)   // the wave's last nmine % NB steps
      if (ngroups * NB + u < nmine) walk_step(u);
    if (ragged && !app && wi == 0) last_step();
  } else {
    // ---------------------------------------------------------------- paged caches
    const int pend = (t1 + kBlock - 1) / kBlock;   // pages [t0 / 16, pend) of the piece
    const int32_t* btrow = d.block_table + (size_t)b * L.max_pages;
    const uint32_t rows8 = (uint32_t)L.num_pages_fp8 * (uint32_t)L.H * kBlock;
    const __amdgpu_buffer_rsrc_t r8K = make_rsrc(d.cache.codes8[0], rows8 * kHeadDim);
    const __amdgpu_buffer_rsrc_t r8V = make_rsrc(d.cache.codes8[1], rows8 * kHeadDim);
    const __amdgpu_buffer_rsrc_t rsK = make_rsrc(d.cache.scale8[0], rows8 * 4u);
    const __amdgpu_buffer_rsrc_t rsV = make_rsrc(d.cache.scale8[1], rows8 * 4u);
    // tokens of page p present in the sequence
    auto page_tokens = [&](int p) { return min(kBlock, S - kBlock * p); };
    // the pool row of the lane's K token (row trow of the tile) and V token (vtok(trow)) in a step
    // (fields are copied before any select: a select between two fields of one struct keeps the
    // struct in memory)
    auto krow_of = [&](const PStep& st) {
      const uint32_t ra = st.rowA, rb = st.rowB;
      const uint32_t base = trow < 16 ? ra : rb;
      return base == kDead ? kDead : base + (uint32_t)(trow & 15);
    };
    auto vrow_of_step = [&](const PStep& st) {
      const uint32_t ra = st.rowA, rb = st.rowB;
      const uint32_t base = (trow & 1) ? rb : ra;
      return base == kDead ? kDead : base + (uint32_t)(trow >> 1);
    };
    // step j of a tier's list of n pages (entries 2j, 2j + 1); an absent page has page number
    // -1 and no rows
    auto pstep = [&](int tier, int j, int n) -> PStep {
      if (2 * j >= n) return PStep{kDead, kDead, -1, -1};
      const uint4 e = *(const uint4*)&s_pl[tier][2 * j][0];   // a pair of entries
      const bool hasB = 2 * j + 1 < n;
      return PStep{(uint32_t)__builtin_amdgcn_readfirstlane((int)e.x),
                   hasB ? (uint32_t)__builtin_amdgcn_readfirstlane((int)e.z) : kDead,
                   __builtin_amdgcn_readfirstlane((int)e.y),
                   hasB ? __builtin_amdgcn_readfirstlane((int)e.w) : -1};
    };
    // tokens of a step (a prefix of its 32: only the last entry of a list can be partial)
    auto step_tokens = [&](const PStep& st) {
      return (st.pA < 0 ? 0 : page_tokens(st.pA)) + (st.pB < 0 ? 0 : page_tokens(st.pB));
    };
    // RAGGED: rows of tokens >= nval get out-of-range offsets (they read as zeros)
    auto issue_codes = [&](Buf<FMT>& bf, const PStep& st, int nval, auto ragged_tag) {
      constexpr bool RAGGED = decltype(ragged_tag)::value;
      const uint32_t rk = krow_of(st), rv = vrow_of_step(st);
      const bool okk = rk != kDead && (!RAGGED || trow < nval);
      const bool okv = rv != kDead && (!RAGGED || vtok(trow) < nval);
      bf.kc = ld128<kNT>(rcK, okk ? rk * CB + half * (CB / 2) : kOOB);
      bf.vc = ld128<kNT>(rcV, okv ? rv * CB + half * (CB / 2) : kOOB);
      bf.km = ld64<kNT>(rmK, okk ? rk * MB + half * (MB / 2) : kOOB);
      bf.vm = ld64<kNT>(rmV, okv ? rv * MB + half * (MB / 2) : kOOB);
    };
    // lanes 0..7 load the block starts {K: pA, pA + 1, pB, pB + 1; V: the same}
    auto issue_bounds = [&](const PStep& st) -> uint32_t {
      if constexpr (HAS_OUTL) {
        const int which = lane & 7;
        const int pa = st.pA, pb = st.pB;
        const int p = max((which & 2) ? pb : pa, 0) + (which & 1);
        return ld32(rbs, (uint32_t)(((which >> 2) * L.nblk + p) * 4));
      }
      return 0u;
    };
    auto issue_recs = [&](Recs& rc, uint32_t bnd, const PStep& st) {
      if constexpr (HAS_OUTL) {
        auto range = [&](int l0, int l1, int pg, uint32_t row, int cnt) {
          const int a = max(0, min(__builtin_amdgcn_readlane((int)bnd, l0), cap));
          const int e = kBlock * (pg + 1) >= S ? cnt : max(0, min(__builtin_amdgcn_readlane((int)bnd, l1), cap));
          return int2{a, pg < 0 || row == kDead ? 0 : max(e - a, 0)};   // none for absent pages
        };
        const int2 kA = range(0, 1, st.pA, st.rowA, cntK), kB = range(2, 3, st.pB, st.rowB, cntK);
        const int2 vA = range(4, 5, st.pA, st.rowA, cntV), vB = range(6, 7, st.pB, st.rowB, cntV);
        const uint32_t baseA = (uint32_t)st.pA * (kBlock * 128u);
        const uint32_t baseB = (uint32_t)st.pB * (kBlock * 128u) - kBlock * 128u;
        rc.k = RecList{kA.x, kA.y, kB.x, kB.y, baseA, baseB};
        rc.v = RecList{vA.x, vA.y, vB.x, vB.y, baseA, baseB};
        const bool ka = lane < kA.y, va = lane < vA.y;
        const uint32_t rk = (uint32_t)(ka ? kA.x + lane : kB.x + lane - kA.y);
        const uint32_t rv = (uint32_t)(va ? vA.x + lane : vB.x + lane - vA.y);

        rc.ik = ld32(riK, rk * 4u);
        rc.iv = ld32(riV, rv * 4u);
        const uint32_t bk = rk * VB + lv3, bv = rv * VB + lv3;
        rc.vk = ld32(rvK, bk & ~3u);
        rc.vv = ld32(rvV, bv & ~3u);
        rc.kb = (ka ? baseA : baseB) | (bk & 3u) * 8u;
        rc.vb = (va ? baseA : baseB) | (bv & 3u) * 8u;
      } else {
        rc.k = RecList{0, 0, 0, 0, 0u, 0u};
        rc.v = rc.k;
      }
    };
    auto load8 = [&](Buf8& f, const PStep& st, int nval) {
      const uint32_t rk = krow_of(st), rv = vrow_of_step(st);
      const uint32_t ok = rk != kDead && trow < nval ? rk * kHeadDim + 64u * half : kOOB;
      const uint32_t ov = rv != kDead && vtok(trow) < nval ? rv * kHeadDim + 64u * half : kOOB;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f.k[k] = ld128(r8K, ok == kOOB ? kOOB : ok + 16u * k);
        f.v[k] = ld128(r8V, ov == kOOB ? kOOB : ov + 16u * k);
      }
      // scales of the lane's score tokens: CMP 4 kg + v of tile (r >= 8), else of both tiles
#pragma unroll
      for (int i = 0; i < (CMP ? 1 : 2); ++i) {
        const int tb = (CMP ? (r >= 8 ? 16 : 0) : 16 * i) + 4 * kg;
        const uint32_t ra = st.rowA, rb = st.rowB;
        const uint32_t base = tb < 16 ? ra : rb;
        const uint32_t off = base != kDead && tb < nval ? (base + (uint32_t)(tb & 15)) * 4u : kOOB;
        const floatx4 ks = __builtin_bit_cast(floatx4, ld128(rsK, off));
        const floatx4 vs = __builtin_bit_cast(floatx4, ld128(rsV, off));
        if (i == 0) { f.ks0 = ks; f.vs0 = vs; } else { f.ks1 = ks; f.vs1 = vs; }
      }
    };
    const Buf<FMT> no2{};
    Recs norec;
    norec.k = RecList{0, 0, 0, 0, 0u, 0u};
    norec.v = norec.k;

    for (int sp0 = t0 / kBlock; sp0 < pend; sp0 += kSegPages) {
      const int np = min(kSegPages, pend - sp0);
      // ---- list the segment's pages by tier, in logical order: page k of the segment is taken by
      // thread k mod 768 (pass k / 768); its 64-page group k / 64 is one wave's ballot
      constexpr int kListers = kWaves * 64;
      constexpr int kPasses = (kSegPages + kListers - 1) / kListers;
      int tier[kPasses];
      uint32_t prow[kPasses];
      uint64_t m0[kPasses], m1[kPasses];
#pragma unroll
      for (int k = 0; k < kPasses; ++k) {
        const int pi = tid + kListers * k;
        tier[k] = -1;
        prow[k] = kDead;
        if (pi < np) {
          const uint32_t e = (uint32_t)btrow[sp0 + pi];
          const uint32_t slot = e & 0x7FFFFFFFu;
          const bool is8 = (e >> 31) != 0;
          const bool in_pool = slot < (uint32_t)(is8 ? L.num_pages_fp8 : L.num_pages);
          if (!in_pool) report(d.cache.status, KVQ_ERR_INVALID_ARG);
          tier[k] = in_pool && is8 ? 1 : 0;   // a slot outside its pool: listed as a page of no rows
          prow[k] = in_pool ? (slot * (uint32_t)L.H + (uint32_t)h) * kBlock : kDead;
        }
        m0[k] = __builtin_amdgcn_ballot_w64(tier[k] == 0);
        m1[k] = __builtin_amdgcn_ballot_w64(tier[k] == 1);
        if (pi < kSegPages && lane == 0) {
          s_wn[pi >> 6][0] = __builtin_popcountll(m0[k]);
          s_wn[pi >> 6][1] = __builtin_popcountll(m1[k]);
        }
      }
      if (lane == 0) *prog_mine = 0;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kPasses; ++k) {
        if (tier[k] >= 0) {
          const int pi = tid + kListers * k;
          int pos = 0;
          for (int w2 = 0; w2 < (pi >> 6); ++w2) pos += s_wn[w2][tier[k]];
          const uint64_t m = tier[k] ? m1[k] : m0[k];
          pos += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          s_pl[tier[k]][pos][0] = prow[k];
          s_pl[tier[k]][pos][1] = (uint32_t)(sp0 + pi);
        }
      }
      int n2 = 0, n8 = 0;
#pragma unroll
      for (int w2 = 0; w2 < kSegPages / 64; ++w2) { n2 += s_wn[w2][0]; n8 += s_wn[w2][1]; }
      n2 = __builtin_amdgcn_readfirstlane(n2);
      n8 = __builtin_amdgcn_readfirstlane(n8);
      __syncthreads();

      // ---- 2-bit pages, two per step: full steps pipelined as for contiguous caches
      const int ns2 = (n2 + 1) / 2;
      const bool rag2 = n2 > 0 && ((n2 & 1) || page_tokens((int)s_pl[0][n2 - 1][1]) < kBlock);
      const int nfull = ns2 - (rag2 ? 1 : 0);
      {
        Buf<FMT> buf[NB];
        Recs rec[NB];
        uint32_t bnd[NB];
        PStep st[NB];
        const int nmine = wi < nfull ? (nfull - wi + wpc - 1) / wpc : 0;
        auto wst = [&](int j) { return pstep(0, j < nmine ? wi + wpc * j : nfull, 2 * nfull); };
        int partner_seen = 0;
#pragma unroll
        for (int k = 0; k < NB; ++k) { st[k] = wst(k); bnd[k] = issue_bounds(st[k]); }
#pragma unroll
        for (int k = 0; k < kPF; ++k) {
          issue_recs(rec[k], bnd[k], st[k]);
          issue_codes(buf[k], st[k], kStep, std::false_type{});
        }
        const int ngroups = nmine / NB;
        for (int g = 0; g < ngroups; ++g) {
          if (g > partner_seen) __builtin_amdgcn_s_setprio(0);
          else __builtin_amdgcn_s_setprio(1);
          if (lane == 0) *prog_mine = g;
#pragma unroll
          for (int u = 0; u < NB; ++u) {
            const int jj = g * NB + u;
            const int cA = st[u].pA, cB = st[u].pB;
            st[u] = wst(jj + NB);
            bnd[u] = issue_bounds(st[u]);
            issue_recs(rec[(u + kPF) % NB], bnd[(u + kPF) % NB], st[(u + kPF) % NB]);
            issue_codes(buf[(u + kPF) % NB], st[(u + kPF) % NB], kStep, std::false_type{});
            consume(buf[u], no8, rec[u], 0u, 0u, kStep, cA, cB, std::true_type{}, std::false_type{});
          }
          partner_seen = min(__builtin_amdgcn_readfirstlane(*prog_p1), __builtin_amdgcn_readfirstlane(*prog_p2));
        }
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int jj = ngroups * NB + u;
          if (jj < nmine) {
            const int cA = st[u].pA, cB = st[u].pB;
            st[u] = wst(jj + NB);
            bnd[u] = issue_bounds(st[u]);
            issue_recs(rec[(u + kPF) % NB], bnd[(u + kPF) % NB], st[(u + kPF) % NB]);
            issue_codes(buf[(u + kPF) % NB], st[(u + kPF) % NB], kStep, std::false_type{});
            consume(buf[u], no8, rec[u], 0u, 0u, kStep, cA, cB, std::true_type{}, std::false_type{});
          }
        }
        if (rag2 && wi == nfull % wpc) {   // the list's last, partly filled step
          const PStep sr = pstep(0, ns2 - 1, n2);
          const int nval = step_tokens(sr);
          const uint32_t b0 = issue_bounds(sr);
          issue_recs(rec[0], b0, sr);
          issue_codes(buf[0], sr, nval, std::true_type{});
          consume(buf[0], no8, rec[0], 0u, 0u, nval, sr.pA, sr.pB, std::false_type{}, std::false_type{});
        }
      }
      // ---- FP8 pages, two per step, continuing the round-robin over the waves
      {
        const int ns8 = (n8 + 1) / 2;
        for (int j = (wi - ns2 % wpc + wpc) % wpc; j < ns8; j += wpc) {
          const PStep s8 = pstep(1, j, n8);
          const int nval = step_tokens(s8);
          Buf8 f;
          load8(f, s8, nval);
          consume(no2, f, norec, 0u, 0u, nval, s8.pA, s8.pB, std::false_type{}, std::true_type{});
        }
      }
      __syncthreads();   // the lists are rebuilt for the next segment
    }
  }

  // ---- merge the waves of the workgroup for the piece
  if constexpr (CMP) {   // column r of query r < 8 += its lo column r + 8
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) oacc[mt][v] += dpp_f32<kRowShl8>(oacc[mt][v]);
  }
  float l_row = l_run;
  if constexpr (CMP) l_row += dpp_f32<kRowRor8>(l_row);
  l_row += __shfl_xor(l_row, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);
  float* s_o = (float*)(s_lds + wave * kTile);   // [16 rows][128 channels] of this wave
  const __amdgpu_buffer_rsrc_t rpart = make_rsrc(d.partials, (uint32_t)(nwg * 2u * (uint64_t)G * (kHeadDim + 2) * 4u));
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) s_o[r * kHeadDim + (16 * mt + 4 * kg + v)] = oacc[mt][v];
  if (kg == 0) { s_ml[wave][r][0] = m_run; s_ml[wave][r][1] = l_row; }
  __syncthreads();
  for (int i = threadIdx.x; i < G * kHeadDim; i += kWaves * 64) {
    const int row = i / kHeadDim, ch = i % kHeadDim;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][row][0]);
    float num = 0.0f, den = 0.0f;
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_ml[w][row][0];
      const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      den += f * s_ml[w][row][1];
      num += f * ((const float*)(s_lds + w * kTile))[row * kHeadDim + ch];
    }
    const size_t hq = (size_t)h * G + row;
    if (whole) {
      d.out[((size_t)b * d.Hq + hq) * kHeadDim + ch] = num / den;
      if (MASS && ch == 0) d.total_lse[(size_t)b * d.Hq + hq] = M + __builtin_log2f(den);
    } else {
      // a part of a list leaves a (max, sum, output) partial per query head in slot 0 (the
      // workgroup's first piece) or 1 (its last)
      const uint32_t o = (uint32_t)(((blockIdx.x * 2u + (first ? 0u : 1u)) * (uint32_t)G + (uint32_t)row) *
                                    (kHeadDim + 2)) * 4u;
      if (ch == 0) { store_sc1(rpart, o, M); store_sc1(rpart, o + 4u, den); }
      store_sc1(rpart, o + (2u + (uint32_t)ch) * 4u, num);
    }
  }
  if (!whole && tid == 0) {   // the list of a part, merged once the workgroup's work is done
    const int sl = first ? 0 : 1;
    s_cut[sl][0] = b;
    s_cut[sl][1] = h;
    s_cut[sl][2] = nb;
    s_cut64[sl] = s_loc64[0];
  }
  if (lane == 0) *prog_mine = 0;
  }
  left -= (uint64_t)take;
  if (left == 0) break;
  if (s1 > s0 || app) {
    first = false;
    __syncthreads();   // the tiles, the wave states and the list's first unit are reused next
  }
  if (tid == 0) s_loc64[0] += (uint64_t)(nb + K0);
  off = 0;
  if (++h == L.H) {   // the next list with steps (a sequence of invalid length has none)
    h = 0;
    do { ++b; } while (!(d.seq_lens[b] >= 1 && d.seq_lens[b] <= L.S_cap));
  }
  }
  // ---- the parts of cut lists: stored (coherently) by the pieces above; the last workgroup to
  // finish a part of a list merges it
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);   // this workgroup's partial stores have completed
  __syncthreads();
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    if (s_cut[sl][0] >= 0)
      merge_cut_list<MASS>(d, s_cut[sl][0], s_cut[sl][1], s_cut[sl][2], s_cut64[sl], K0a, K0b, s_loc64, s_mg);
    __syncthreads();   // s_mg is written again
  }
}

template <int FMT, bool CMP, bool PAGED, bool MASS, bool APP>
void launch_cmp(const DecodeLaunch& d, dim3 grid, hipStream_t st) {
  switch (d.outl) {
    case KVQ_OUTL_NONE: decode_mfma_kernel<FMT, KVQ_OUTL_NONE, CMP, PAGED, MASS, APP><<<grid, kWaves * 64, 0, st>>>(d); break;
    case KVQ_OUTL_FP16: decode_mfma_kernel<FMT, KVQ_OUTL_FP16, CMP, PAGED, MASS, APP><<<grid, kWaves * 64, 0, st>>>(d); break;
    default: decode_mfma_kernel<FMT, KVQ_OUTL_FP8_E4M3, CMP, PAGED, MASS, APP><<<grid, kWaves * 64, 0, st>>>(d); break;
  }
}

template <int FMT, bool PAGED, bool MASS = false, bool APP = false>
void launch_fmt(const DecodeLaunch& d, dim3 grid, hipStream_t st) {
  if (d.Hq / d.L.H <= 8) launch_cmp<FMT, true, PAGED, MASS, APP>(d, grid, st);
  else launch_cmp<FMT, false, PAGED, MASS, APP>(d, grid, st);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeLaunch& d, hipStream_t st, bool* handled) {
  *handled = false;
  if (!mfma_decodes(d.fmt, d.group, d.L.paged, d.L.num_pages, d.L.num_pages_fp8, d.L.H)) return hipSuccess;
  if (d.nwg < 1 || !d.partials) return hipSuccess;
  const dim3 grid(d.nwg);
  if (d.k_new && (d.L.paged || d.page_lse)) return hipErrorInvalidValue;   // (checked by the caller)
  if (d.L.paged && d.page_lse) launch_fmt<FMT_C2, true, true>(d, grid, st);
  else if (d.L.paged) launch_fmt<FMT_C2, true>(d, grid, st);
  else if (d.k_new && d.fmt == FMT_C2) launch_fmt<FMT_C2, false, false, true>(d, grid, st);
  else if (d.k_new) launch_fmt<FMT_FP4, false, false, true>(d, grid, st);
  else if (d.fmt == FMT_C2) launch_fmt<FMT_C2, false>(d, grid, st);
  else launch_fmt<FMT_FP4, false>(d, grid, st);
  *handled = true;
  return hipGetLastError();
}

}  // namespace kvq
